// Internal helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define TRG_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#include <utility>

namespace trg {

constexpr int kWave = 64;

// Compile-time loop: f(std::integral_constant<int, 0>) ... f(<N-1>).  Keeps
// register-array indices constant where #pragma unroll may give up.
template <class F, int... I>
TRG_DEV void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
TRG_DEV void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- bfloat16 <-> float (storage is raw uint16_t) ---------------------------
// A 16-byte store with the non-temporal hint, for output rows that the
// writing kernel does not read again and that go out as whole lines.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
TRG_DEV void store_nt16(void* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4_t*)p);
}

TRG_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
TRG_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
TRG_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round to nearest even; NaN stays NaN.
// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays
// a quiet NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
TRG_DEV uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
TRG_DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element access for the two storage types.
template <class T> struct Elt;
template <> struct Elt<float> {
  static TRG_DEV float ld(const float* p) { return *p; }
  static TRG_DEV void st(float* p, float v) { *p = v; }
  static constexpr int kVec = 4;  // elements per 16-byte vector
};
template <> struct Elt<uint16_t> {
  static TRG_DEV float ld(const uint16_t* p) { return bf2f(*p); }
  static TRG_DEV void st(uint16_t* p, float v) { *p = f2bf(v); }
  static constexpr int kVec = 8;
};

// Unpack a 16-byte vector into floats, and pack floats back.
template <class T> TRG_DEV void unpack16(const uint4& v, float* f);
template <> TRG_DEV void unpack16<float>(const uint4& v, float* f) {
  f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
  f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
}
template <> TRG_DEV void unpack16<uint16_t>(const uint4& v, float* f) {
  f[0] = bf_lo(v.x); f[1] = bf_hi(v.x); f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
  f[4] = bf_lo(v.z); f[5] = bf_hi(v.z); f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
template <class T> TRG_DEV uint4 pack16(const float* f);
template <> TRG_DEV uint4 pack16<float>(const float* f) {
  return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                    __float_as_uint(f[3]));
}
template <> TRG_DEV uint4 pack16<uint16_t>(const float* f) {
  return make_uint4(pack_bf2(f[0], f[1]), pack_bf2(f[2], f[3]), pack_bf2(f[4], f[5]),
                    pack_bf2(f[6], f[7]));
}

// ---- wave reductions ---------------------------------------------------------
TRG_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
TRG_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Exclusive scan of one value per thread over a block of 1024 threads: a
// shuffle scan inside each wave, then the 16 wave totals scanned by wave 0
// (three barriers; integer sums, so the result does not depend on the order).
TRG_DEV int block_excl_scan_1024(int v, int* tmp /* >= 32 */, int* total) {
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  int x = v;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int w = lane < 16 ? tmp[lane] : 0;  // inclusive scan of the wave totals
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(w, o, kWave);
      if (lane >= o) w += y;
    }
    if (lane < 16) tmp[16 + lane] = w;
  }
  __syncthreads();
  const int before = wv > 0 ? tmp[16 + wv - 1] : 0;
  *total = tmp[31];
  __syncthreads();  // tmp is reused by the next call
  return before + x - v;
}

// The epilogues' activation functions with the hardware reciprocal (1 ulp;
// the results are stored in bf16): an IEEE division costs about ten
// instructions more per element.  Limits: g -> -inf gives -0 and 0, g -> +inf
// gives g and 1.
TRG_DEV float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }
TRG_DEV float silu_f(float g) { return g * sigmoid_f(g); }

}  // namespace trg
