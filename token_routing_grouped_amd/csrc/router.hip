// Router GEMMs and the softmax backward.
//   logits = x Wr^T;  dlogits = p * (g - <p, g>);  dWr = dlogits^T x;
//   dx += dlogits Wr.
// For few experts (E < 64) these are skinny and HBM-bound on x, so they run on
// the vector ALUs: one wave per token row for the logits, column-parallel
// partial sums over token chunks (reduced in a fixed order) for dWr, and one
// workgroup per token row for dx.  For E >= 64 (bf16, E % 8 == 0) the three
// products are real GEMMs and go to the matrix-core kernels.
#include "common.h"
#include "kernels.h"

namespace trg {

template <class T, int EB>
__global__ __launch_bounds__(256) void router_logits_valu_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                                 int Tn, int d, int E, float* __restrict__ logits) {
  constexpr int V = Elt<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= Tn) return;
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  const uint4* xr = (const uint4*)(x + (long)t * d);
  const int nv = d / V;
  for (int v = lane; v < nv; v += 64) {
    float f[V];
    unpack16<T>(xr[v], f);
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      if (e < E) {
        float w[V];
        unpack16<T>(((const uint4*)(wr + (long)e * d))[v], w);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[e] = fmaf(f[i], w[i], acc[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if (e < E) {
      const float s = wave_sum(acc[e]);
      if (lane == 0) logits[(long)t * E + e] = s;
    }
  }
}

// Softmax backward through the gates.  One wave per token.
template <int EPL>
__global__ __launch_bounds__(256) void router_dl_kernel(const float* __restrict__ probs, const int* __restrict__ idx,
                                                        const float* __restrict__ dgate,
                                                        const float* __restrict__ aux_g, int Tn, int E, int k,
                                                        float* __restrict__ dL, uint16_t* __restrict__ dLb) {
  const int lane = threadIdx.x & 63;
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= Tn) return;
  float p[EPL], gh[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? probs[(long)t * E + e] : 0.f;
    gh[i] = 0.f;
  }
  // the balance loss's probability gradient (the same for every token), added
  // before the gates' own (disjoint slots are written below)
  float ga[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) ga[i] = (aux_g != nullptr && lane + 64 * i < E) ? aux_g[lane + 64 * i] : 0.f;
  for (int j = 0; j < k; ++j) {
    const int ej = idx[(long)t * k + j];
    const float gj = dgate[(long)t * k + j];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == ej) gh[i] = gj;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) gh[i] += ga[i];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s = fmaf(p[i], gh[i], s);
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float v = p[i] * (gh[i] - s);
      dL[(long)t * E + e] = v;
      if (dLb) dLb[(long)t * E + e] = f2bf(v);
    }
  }
}

constexpr int kDwrChunk = 256;  // tokens per dWr partial sum

// dWr partial sums over one chunk of kDwrChunk tokens.  Thread layout: 32
// column groups of CV = 64/EB consecutive columns x 8 token lanes (the token
// lanes of a group are neighbouring lanes of one wave, reduced with shuffles),
// so each wave load covers whole 128-byte row pieces of x and every thread has
// several independent loads in flight.
template <class T, int EB>
__global__ __launch_bounds__(256) void router_dwr_partial_kernel(const float* __restrict__ dL, const T* __restrict__ x,
                                                                 int Tn, int d, int E, float* __restrict__ part) {
  constexpr int CV = 64 / EB;  // columns per thread; EB * CV = 64 accumulators
  struct alignas(CV * sizeof(T)) Vec { T v[CV]; };
  __shared__ float sdl[64][EB];
  const int tl = threadIdx.x & 7, cg = threadIdx.x >> 3;
  const int c0 = blockIdx.x * (32 * CV) + cg * CV;
  const int chunk = blockIdx.y;
  const int t0 = chunk * kDwrChunk, t1 = min(Tn, t0 + kDwrChunk);
  float acc[EB][CV];
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int v = 0; v < CV; ++v) acc[e][v] = 0.f;
  const bool full = c0 + CV <= d;
  for (int tb = t0; tb < t1; tb += 64) {
    const int nt = min(64, t1 - tb);
    for (int q = threadIdx.x; q < 64 * EB; q += 256) {
      const int tt = q / EB, e = q % EB;
      sdl[tt][e] = (tt < nt && e < E) ? dL[(long)(tb + tt) * E + e] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = tl; tt < 64; tt += 8) {
      float xv[CV];
      if (tt < nt && full) {
        const Vec w = *(const Vec*)(x + (long)(tb + tt) * d + c0);
#pragma unroll
        for (int v = 0; v < CV; ++v) xv[v] = Elt<T>::ld(&w.v[v]);
      } else {
#pragma unroll
        for (int v = 0; v < CV; ++v)
          xv[v] = (tt < nt && c0 + v < d) ? Elt<T>::ld(x + (long)(tb + tt) * d + c0 + v) : 0.f;
      }
#pragma unroll
      for (int e = 0; e < EB; ++e)
#pragma unroll
        for (int v = 0; v < CV; ++v) acc[e][v] = fmaf(sdl[tt][e], xv[v], acc[e][v]);
    }
    __syncthreads();
  }
  // sum the 8 token lanes (fixed order)
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int v = 0; v < CV; ++v) {
      float a = acc[e][v];
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      acc[e][v] = a;
    }
  if (tl == 0) {
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int v = 0; v < CV; ++v)
        if (c0 + v < d) part[((long)chunk * E + e) * d + c0 + v] = acc[e][v];
  }
}

template <class T>
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float* __restrict__ part, int nch, long n,
                                                        T* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = part[i];
  for (int c = 1; c < nch; ++c) s += part[(long)c * n + i];
  Elt<T>::st(out + i, s);
}

template <class T, int EB>
__global__ __launch_bounds__(256) void router_dx_valu_kernel(const float* __restrict__ dL, const T* __restrict__ wr,
                                                             int d, int E, T* __restrict__ dx) {
  constexpr int V = Elt<T>::kVec;
  __shared__ float sdl[EB];
  const int t = blockIdx.x;
  if (threadIdx.x < EB) sdl[threadIdx.x] = threadIdx.x < E ? dL[(long)t * E + threadIdx.x] : 0.f;
  __syncthreads();
  const int nv = d / V;
  uint4* row = (uint4*)(dx + (long)t * d);
  for (int v = threadIdx.x; v < nv; v += 256) {
    float acc[V];
    unpack16<T>(row[v], acc);
    for (int e = 0; e < E; ++e) {
      float w[V];
      unpack16<T>(((const uint4*)(wr + (long)e * d))[v], w);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(sdl[e], w[i], acc[i]);
    }
    row[v] = pack16<T>(acc);
  }
}

template <class T>
__global__ __launch_bounds__(256) void zero_fill_kernel(T* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = T(0);
}

static inline bool router_uses_mfma(bool bf16, int E) { return bf16 && E >= 64 && E % 8 == 0; }
static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t router_bwd_ws_bytes(int T, int d, int E) {
  const size_t dl = align256((size_t)T * E * sizeof(float));
  const size_t dlb = align256((size_t)T * E * sizeof(uint16_t));
  const size_t valu = align256((size_t)((T + kDwrChunk - 1) / kDwrChunk) * E * d * sizeof(float));
  const size_t mf = align256(router_dwr_mfma_part_bytes(T, d, E));
  return dl + dlb + (valu > mf ? valu : mf);
}

template <class T, int EB>
static void logits_valu(const void* x, const void* wr, int Tn, int d, int E, float* out, hipStream_t s) {
  router_logits_valu_kernel<T, EB><<<(Tn + 3) / 4, 256, 0, s>>>((const T*)x, (const T*)wr, Tn, d, E, out);
}

template <class T>
static void logits_valu_any(const void* x, const void* wr, int Tn, int d, int E, float* out, hipStream_t s) {
  if (E <= 8) logits_valu<T, 8>(x, wr, Tn, d, E, out, s);
  else if (E <= 16) logits_valu<T, 16>(x, wr, Tn, d, E, out, s);
  else if (E <= 32) logits_valu<T, 32>(x, wr, Tn, d, E, out, s);
  else logits_valu<T, 64>(x, wr, Tn, d, E, out, s);
}

hipError_t launch_router_logits(const void* x, bool bf16, const void* wr, int T, int d, int E, float* logits,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (router_uses_mfma(bf16, E))
    return launch_dense_nt_f32out((const uint16_t*)x, (const uint16_t*)wr, logits, T, E, d, s);
  if (E > 64) return hipErrorInvalidValue;
  if (bf16) logits_valu_any<uint16_t>(x, wr, T, d, E, logits, s);
  else logits_valu_any<float>(x, wr, T, d, E, logits, s);
  return hipGetLastError();
}

template <class T, int EB>
static void bwd_valu(const float* dL, const void* x, const void* wr, int Tn, int d, int E, void* dx, void* dwr,
                     float* part, hipStream_t s) {
  const int nch = (Tn + kDwrChunk - 1) / kDwrChunk;
  constexpr int cols_per_block = 32 * (64 / EB);
  dim3 grid((d + cols_per_block - 1) / cols_per_block, nch);
  router_dwr_partial_kernel<T, EB><<<grid, 256, 0, s>>>(dL, (const T*)x, Tn, d, E, part);
  const long n = (long)E * d;
  chunk_sum_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, nch, n, (T*)dwr);
  router_dx_valu_kernel<T, EB><<<Tn, 256, 0, s>>>(dL, (const T*)wr, d, E, (T*)dx);
}

template <class T>
static void bwd_valu_any(const float* dL, const void* x, const void* wr, int Tn, int d, int E, void* dx, void* dwr,
                         float* part, hipStream_t s) {
  if (E <= 8) bwd_valu<T, 8>(dL, x, wr, Tn, d, E, dx, dwr, part, s);
  else if (E <= 16) bwd_valu<T, 16>(dL, x, wr, Tn, d, E, dx, dwr, part, s);
  else if (E <= 32) bwd_valu<T, 32>(dL, x, wr, Tn, d, E, dx, dwr, part, s);
  else bwd_valu<T, 64>(dL, x, wr, Tn, d, E, dx, dwr, part, s);
}

hipError_t launch_router_bwd(const float* probs, const int* idx, const float* dgate, const float* aux_g,
                             const void* x, const void* wr, int T, int d, int E, int k, bool bf16, void* dx, void* dwr,
                             void* ws, hipStream_t s) {
  const bool mf = router_uses_mfma(bf16, E);
  if (!mf && E > 64) return hipErrorInvalidValue;
  char* p = (char*)ws;
  float* dL = (float*)p;
  p += align256((size_t)T * E * sizeof(float));
  uint16_t* dLb = (uint16_t*)p;
  p += align256((size_t)T * E * sizeof(uint16_t));
  float* part = (float*)p;
  if (T == 0) {  // no tokens: dWr is zero (a fill kernel, not a memset node)
    const long n = (long)E * d;
    if (bf16) zero_fill_kernel<uint16_t><<<(unsigned)((n + 255) / 256), 256, 0, s>>>((uint16_t*)dwr, n);
    else zero_fill_kernel<float><<<(unsigned)((n + 255) / 256), 256, 0, s>>>((float*)dwr, n);
    return hipGetLastError();
  }
  const dim3 gw((T + 3) / 4);
  uint16_t* dlb_out = mf ? dLb : nullptr;
  if (E <= 64) router_dl_kernel<1><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 128) router_dl_kernel<2><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 256) router_dl_kernel<4><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 512) router_dl_kernel<8><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else router_dl_kernel<16><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  if (mf) {
    hipError_t err = launch_router_dwr_mfma(dLb, (const uint16_t*)x, (uint16_t*)dwr, part, T, d, E, s);
    if (err != hipSuccess) return err;
    return launch_router_dx_mfma(dLb, (const uint16_t*)wr, (uint16_t*)dx, T, d, E, s);
  }
  if (bf16) bwd_valu_any<uint16_t>(dL, x, wr, T, d, E, dx, dwr, part, s);
  else bwd_valu_any<float>(dL, x, wr, T, d, E, dx, dwr, part, s);
  return hipGetLastError();
}

}  // namespace trg
