// MXFP8 quantisation: OCP microscaling with E4M3FN elements and one E8M0
// scale per 32 consecutive values along a GEMM's reduction dimension.  The
// pages name MXFP8 as the low-precision format that cuts both compute and the
// data moved between experts (Olmo-core 3 overview, "Precision optimisation
// with MXFP8"); the encoding is OCP MX v1.0:
//   s = clamp(floor(log2(amax)) - 8, -127, 127) from the exponent bits of the
//       block's largest magnitude (s = -127 for an all-zero block); scale byte
//       s + 127;
//   q = E4M3FN(v * 2^-s), round to nearest even, saturating to +-448, sign of
//       zero kept.
//
// One kernel writes both layouts a MoE layer needs from a single read of the
// source:
//   row layout      q_row [rows, cols]                             (blocks
//                   along the columns: the forward and dgrad K);
//   column layout   q_col [cols, ldc]                              (blocks of
//                   32 consecutive rows inside each segment, zero-padded at
//                   the segment's end; segment e starts at column off128[e]:
//                   the weight-gradient K).
// Scale bytes are stored K-chunk major: the scale of block b (of 32 values
// along K) of row r of an n-row MX matrix is byte (b / 4 * n + r) * 4 + b % 4,
// so the four scales of one 128-wide K chunk of a row form one dword and the
// chunk's dwords of consecutive rows are contiguous: a GEMM K step of 128
// reads its tile's scales as one piece instead of a dword per row.
// Rows can be gathered on the fly (row r reads in[src[r] / k]), which fuses
// the rowwise dispatch of the layer input into its quantisation; a gathered
// row can also be scaled by gate[src[r]] and rounded to bf16 first, which is
// the combine backward's dYp row (gate * dy[t]) quantised without being
// stored.
#include "common.h"
#include "kernels.h"

namespace trg {

// floor(log2(a)) for a normal float a > 0, from the exponent bits; -127 for
// zero and float subnormals (both clamp to the smallest scale anyway).
TRG_DEV int ilog2_floor(float a) {
  const int ex = (int)((__float_as_uint(a) >> 23) & 0xFF);
  return ex == 0 ? -127 : ex - 127;
}

// Block scale exponent s for a block whose largest magnitude is amax.
TRG_DEV int mx_scale_exp(float amax) {
  if (amax == 0.0f) return -127;
  const int s = ilog2_floor(amax) - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

// E4M3FN codes of four values already divided by the block scale (|x| <
// 512): clamped to +-448 (the saturating rule; the sign of zero survives the
// clamp), then gfx950's OCP fp8 conversion, which rounds to nearest even and
// keeps subnormals.  Byte z of the result is the code of the z-th value.
TRG_DEV float sat448(float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); }
TRG_DEV uint32_t e4m3_x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

TRG_DEV float to_f32(float v) { return v; }
TRG_DEV float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

constexpr int kMxRows = 128;  // padded rows per workgroup (four 32-row blocks)
constexpr int kMxCols = 128;  // columns per workgroup

// OR of v over the four lanes 4q .. 4q+3 (all of them take part).
TRG_DEV uint32_t or4(uint32_t v) {
  v |= __shfl_xor(v, 1);
  return v | __shfl_xor(v, 2);
}

// Segment of the 32-row block starting at padded row base32: the block's first
// source row, the segment's end row; false past the padded row space.
TRG_DEV bool mx_block_rows(int base32, int rows, const int* seg_off, const int* seg_off128, int nseg, int seg_rows,
                           int& r0, int& seg_hi) {
  if (seg_off != nullptr) {
    if (base32 >= seg_off128[nseg]) return false;
    int lo = 0, hi = nseg;  // last e with seg_off128[e] <= base32
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg_off128[mid] <= base32) lo = mid; else hi = mid;
    }
    r0 = seg_off[lo] + (base32 - seg_off128[lo]);
    seg_hi = seg_off[lo + 1];
  } else {
    // fixed-size segments of seg_rows rows (rows a multiple of seg_rows, or a
    // single segment), each padded to a multiple of 32 rows
    const int seg32 = (seg_rows + 31) / 32 * 32;
    const int nsegf = (rows + seg_rows - 1) / seg_rows;
    if (base32 >= nsegf * seg32) return false;
    const int e = base32 / seg32;
    r0 = e * seg_rows + (base32 - e * seg32);
    seg_hi = min(rows, e * seg_rows + seg_rows);
  }
  return true;
}

// One workgroup: 128 rows of the padded row space (four 32-row blocks, each
// inside one segment) x 128 columns; every thread takes two units per pass.
//   rowwise pass: unit u -> row u/4, 32 columns from (u%4)*32: the four units
//   of a row are neighbouring lanes, so each row's 128 payload bytes go out as
//   one piece and its 4 scale bytes as one dword;
//   columnwise pass: unit u -> column u/4, 32-row block u%4: likewise 128
//   payload bytes and one scale dword per column.
template <class T>
__global__ __launch_bounds__(256) void mx_dual_kernel(const T* __restrict__ in, long ld_in, int rows, int cols,
                                                      const int* __restrict__ src, int gk,
                                                      const float* __restrict__ gate,
                                                      const int* __restrict__ seg_off,
                                                      const int* __restrict__ seg_off128, int nseg, int seg_rows,
                                                      uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                      uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                      long ldc) {
  // The tile keeps the source values in their own type (bf16: 33 KiB).  Row
  // pitch kMxCols + PAD elements plus 64 bytes per 32-row block: the
  // columnwise pass reads four blocks x 16 columns per wave from distinct
  // banks.
  constexpr int PAD = sizeof(T) == 2 ? 2 : 1;
  constexpr int PITCH = kMxCols + PAD;
  constexpr int BLKSKIP = 64 / sizeof(T);
  constexpr int V = 16 / sizeof(T);  // values per 16-byte load
  __shared__ __attribute__((aligned(16))) T tile[kMxRows * PITCH + 4 * BLKSKIP];
  auto at = [&](int r, int c) -> T& { return tile[r * PITCH + (r >> 5) * BLKSKIP + c]; };
  const int tid = threadIdx.x, q4 = tid & 3;
  // workgroups walk the column blocks of a row band first: neighbouring
  // workgroups read neighbouring pieces of the same source rows
  const int ncb = (cols + kMxCols - 1) / kMxCols;
  const int base = (int)(blockIdx.x / ncb) * kMxRows;
  const int col0 = (int)(blockIdx.x % ncb) * kMxCols;
  // whole scale dwords (a row's four blocks of a 128-chunk) where the base is
  // 4-byte aligned and all four blocks are written
  const bool row_dw = ((uintptr_t)s_row & 3) == 0;
  const bool col_dw = ((uintptr_t)s_col & 3) == 0;

  // The band's four 32-row blocks -> (first source row, segment end, valid),
  // looked up once per workgroup.  Segment starts go through LDS first (one
  // coalesced load instead of a chain of dependent loads per thread: the
  // search's latency was a large part of a band's time).
  __shared__ int s_off[1025];
  __shared__ int blk[4][3];
  if (seg_off != nullptr && nseg <= 1024) {
    for (int e = tid; e <= nseg; e += 256) s_off[e] = seg_off128[e];
    __syncthreads();
  }
  if (tid < 4) {
    const int b32 = base + tid * 32;
    int r0 = 0, seg_hi = 0, ok = 0;
    if (seg_off != nullptr && nseg <= 1024) {
      if (b32 < s_off[nseg]) {
        int lo = 0, hi = nseg;  // last e with seg_off128[e] <= b32
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_off[mid] <= b32) lo = mid; else hi = mid;
        }
        r0 = seg_off[lo] + (b32 - s_off[lo]);
        seg_hi = seg_off[lo + 1];
        ok = 1;
      }
    } else {
      ok = mx_block_rows(b32, rows, seg_off, seg_off128, nseg, seg_rows, r0, seg_hi) ? 1 : 0;
    }
    blk[tid][0] = r0;
    blk[tid][1] = seg_hi;
    blk[tid][2] = ok;
  }
  __syncthreads();

  // ---- rowwise: both units' loads first
  uint4 raw[2][32 / V];
  int rr[2];
  bool rok[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = (tid >> 2) + 64 * k;
    const int r0 = blk[i >> 5][0], seg_hi = blk[i >> 5][1];
    const bool blk_ok = blk[i >> 5][2] != 0;
    rr[k] = r0 + (i & 31);
    const int c = col0 + q4 * 32;
    rok[k] = blk_ok && rr[k] < seg_hi && c < cols;
    if (rok[k]) {
      long srow = rr[k];
      float gw = 1.0f;
      if (src != nullptr) {
        const int sr = src[rr[k]];
        srow = sr / gk;
        if (gate != nullptr) gw = gate[sr];
      }
      const uint4* p = (const uint4*)(in + srow * ld_in + c);
#pragma unroll
      for (int q = 0; q < 32 / V; ++q) raw[k][q] = p[q];
      if (gate != nullptr) {  // the gated row, rounded to the source type (bf16 RNE)
#pragma unroll
        for (int q = 0; q < 32 / V; ++q) {
          float f[V];
          unpack16<T>(raw[k][q], f);
#pragma unroll
          for (int z = 0; z < V; ++z) f[z] *= gw;
          raw[k][q] = pack16<T>(f);
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < 32 / V; ++q) raw[k][q] = make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int i = (tid >> 2) + 64 * k;
    const int c = col0 + q4 * 32;
    // the source bits go to the tile as they are
#pragma unroll
    for (int z = 0; z < 32; ++z) at(i, q4 * 32 + z) = ((const T*)raw[k])[z];
    if (q_row != nullptr) {
      float v[32];
#pragma unroll
      for (int q = 0; q < 32 / V; ++q) unpack16<T>(raw[k][q], v + q * V);
      float amax = 0.f;
#pragma unroll
      for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(v[z]));
      const int s = mx_scale_exp(amax);
      const uint32_t all = or4((rok[k] ? 1u : 0u) << q4);
      const uint32_t sw = or4((uint32_t)(s + 127) << (8 * q4));
      if (rok[k]) {
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = e4m3_x4(ldexpf(v[q * 4], -s), ldexpf(v[q * 4 + 1], -s), ldexpf(v[q * 4 + 2], -s),
                         ldexpf(v[q * 4 + 3], -s));
        uint4* dst = (uint4*)(q_row + (long)rr[k] * cols + c);
        store_nt16(dst, make_uint4(w[0], w[1], w[2], w[3]));
        store_nt16(dst + 1, make_uint4(w[4], w[5], w[6], w[7]));
        uint8_t* sp = s_row + ((long)(c >> 7) * rows + rr[k]) * 4 + ((c >> 5) & 3);
        if (row_dw && all == 15u) {
          if (q4 == 0) *(uint32_t*)sp = sw;
        } else {
          *sp = (uint8_t)(s + 127);
        }
      }
    }
  }
  if (q_col == nullptr) return;
  __syncthreads();

  // ---- columnwise (rows outside a segment are zero in the tile)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int cc = (tid >> 2) + 64 * k, sb = q4;
    const int c = col0 + cc;
    const bool ok = blk[sb][2] != 0 && c < cols;
    float x[32];
#pragma unroll
    for (int z = 0; z < 32; ++z) x[z] = to_f32(at(sb * 32 + z, cc));
    float amax = 0.f;
#pragma unroll
    for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(x[z]));
    const int s = mx_scale_exp(amax);
    const uint32_t all = or4((ok ? 1u : 0u) << q4);
    const uint32_t sw = or4((uint32_t)(s + 127) << (8 * q4));
    if (ok) {
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = e4m3_x4(ldexpf(x[q * 4], -s), ldexpf(x[q * 4 + 1], -s), ldexpf(x[q * 4 + 2], -s),
                       ldexpf(x[q * 4 + 3], -s));
      uint4* dst = (uint4*)(q_col + (long)c * ldc + base + sb * 32);
      store_nt16(dst, make_uint4(w[0], w[1], w[2], w[3]));
      store_nt16(dst + 1, make_uint4(w[4], w[5], w[6], w[7]));
      const int b = (base + sb * 32) >> 5;  // block along the padded rows
      uint8_t* sp = s_col + ((long)(b >> 2) * cols + c) * 4 + (b & 3);
      if (col_dw && all == 15u) {
        if (sb == 0) *(uint32_t*)sp = sw;
      } else {
        *sp = (uint8_t)(s + 127);
      }
    }
  }
}

hipError_t launch_mx_quantize(const void* in, bool bf16, long ld_in, int rows, int cols, const int* src, int gk,
                              const int* seg_off, const int* seg_off128, int nseg, int seg_rows, int max_blocks32,
                              uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, long ldc,
                              hipStream_t s, const float* gate) {
  if (rows == 0 || max_blocks32 == 0) return hipSuccess;
  const long nblk = (long)((max_blocks32 + 3) / 4) * ((cols + kMxCols - 1) / kMxCols);
  if (nblk > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)nblk;
  if (bf16)
    mx_dual_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)in, ld_in, rows, cols, src, gk, gate, seg_off,
                                                  seg_off128, nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  else
    mx_dual_kernel<float><<<grid, 256, 0, s>>>((const float*)in, ld_in, rows, cols, src, gk, gate, seg_off, seg_off128,
                                               nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  return hipGetLastError();
}

}  // namespace trg
