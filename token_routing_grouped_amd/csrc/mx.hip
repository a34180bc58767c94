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
//   row layout      q_row [rows, cols], s_row [rows, cols/32]      (blocks
//                   along the columns: the forward and dgrad K);
//   column layout   q_col [cols, ldc], s_col [cols, ldc/32]        (blocks of
//                   32 consecutive rows inside each segment, zero-padded at
//                   the segment's end; segment e starts at column off32[e]:
//                   the weight-gradient K).
// Rows can be gathered on the fly (row r reads in[src[r] / k]), which fuses
// the rowwise dispatch of the layer input into its quantisation.
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

// E4M3FN code of x (already divided by the block scale; |x| < 512),
// nearest-even, saturating to 448, signed zero kept.
TRG_DEV uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal spacing 2^-9; 8 -> smallest normal
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    const int e = ilog2_floor(a);                                   // -6 .. 8
    const float m = __builtin_rintf(ldexpf(a, 3 - e));              // 8 .. 16, exact scaling
    code = (uint32_t)(((e + 7) << 3) + ((int)m - 8));               // m == 16 carries into e
  }
  if (code > 0x7Eu) code = 0x7Eu;  // 0x7F is NaN in E4M3FN: saturate to 448
  return sign | code;
}

constexpr int kMxRows = 128;  // padded rows per workgroup (four 32-row blocks)
constexpr int kMxCols = 64;   // columns per workgroup

// Segment of the 32-row block starting at padded row base32: the block's first
// source row, the segment's end row; false past the padded row space.
TRG_DEV bool mx_block_rows(int base32, int rows, const int* seg_off, const int* seg_off32, int nseg, int seg_rows,
                           int& r0, int& seg_hi) {
  if (seg_off != nullptr) {
    if (base32 >= seg_off32[nseg]) return false;
    int lo = 0, hi = nseg;  // last e with seg_off32[e] <= base32
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg_off32[mid] <= base32) lo = mid; else hi = mid;
    }
    r0 = seg_off[lo] + (base32 - seg_off32[lo]);
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
// inside one segment) x 64 columns.
//   rowwise pass: thread t -> row t/2, 32 columns from (t%2)*32;
//   columnwise pass: thread t -> column t/4, 32-row block t%4; the four
//   blocks of a column are neighbouring lanes, so each column's 128 payload
//   bytes and 4 scale bytes go out as one contiguous piece.
template <class T>
__global__ __launch_bounds__(256) void mx_dual_kernel(const T* __restrict__ in, long ld_in, int rows, int cols,
                                                      const int* __restrict__ src, int gk,
                                                      const int* __restrict__ seg_off,
                                                      const int* __restrict__ seg_off32, int nseg, int seg_rows,
                                                      uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                      uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                      long ldc) {
  // row stride 65 plus 16 words per 32-row block: the columnwise pass reads
  // four blocks x 16 columns per wave from 64 distinct banks
  __shared__ float tile[kMxRows * (kMxCols + 1) + 4 * 16];
  auto at = [&](int r, int c) -> float& { return tile[r * (kMxCols + 1) + (r >> 5) * 16 + c]; };
  const int tid = threadIdx.x;
  const int base = blockIdx.x * kMxRows;
  const int col0 = blockIdx.y * kMxCols;

  // ---- rowwise
  {
    const int i = tid >> 1, cb = (tid & 1) * 32;
    int r0, seg_hi;
    const bool blk_ok = mx_block_rows(base + (i & ~31), rows, seg_off, seg_off32, nseg, seg_rows, r0, seg_hi);
    const int r = r0 + (i & 31);
    const int c = col0 + cb;
    float v[32];
    const bool ok = blk_ok && r < seg_hi && c < cols;
    if (ok) {
      long srow = r;
      if (src != nullptr) srow = src[r] / gk;
      const T* p = in + srow * ld_in + c;
      constexpr int V = 16 / sizeof(T);
#pragma unroll
      for (int q = 0; q < 32 / V; ++q) {
        float f[V];
        unpack16<T>(((const uint4*)p)[q], f);
#pragma unroll
        for (int z = 0; z < V; ++z) v[q * V + z] = f[z];
      }
    } else {
#pragma unroll
      for (int z = 0; z < 32; ++z) v[z] = 0.f;
    }
#pragma unroll
    for (int z = 0; z < 32; ++z) at(i, cb + z) = v[z];
    if (ok && q_row != nullptr) {
      float amax = 0.f;
#pragma unroll
      for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(v[z]));
      const int s = mx_scale_exp(amax);
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        w[q] = 0;
#pragma unroll
        for (int z = 0; z < 4; ++z) w[q] |= e4m3_code(ldexpf(v[q * 4 + z], -s)) << (8 * z);
      }
      uint4* dst = (uint4*)(q_row + (long)r * cols + c);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      s_row[(long)r * (cols / 32) + c / 32] = (uint8_t)(s + 127);
    }
  }
  if (q_col == nullptr) return;
  __syncthreads();

  // ---- columnwise (rows outside a segment are zero in the tile)
  {
    const int cc = tid >> 2, sb = tid & 3;
    const int c = col0 + cc;
    int r0, seg_hi;
    const bool blk_ok = mx_block_rows(base + sb * 32, rows, seg_off, seg_off32, nseg, seg_rows, r0, seg_hi);
    if (blk_ok && c < cols) {
      float amax = 0.f;
#pragma unroll
      for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(at(sb * 32 + z, cc)));
      const int s = mx_scale_exp(amax);
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        w[q] = 0;
#pragma unroll
        for (int z = 0; z < 4; ++z) w[q] |= e4m3_code(ldexpf(at(sb * 32 + q * 4 + z, cc), -s)) << (8 * z);
      }
      uint4* dst = (uint4*)(q_col + (long)c * ldc + base + sb * 32);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      s_col[(long)c * (ldc / 32) + (base + sb * 32) / 32] = (uint8_t)(s + 127);
    }
  }
}

hipError_t launch_mx_quantize(const void* in, bool bf16, long ld_in, int rows, int cols, const int* src, int gk,
                              const int* seg_off, const int* seg_off32, int nseg, int seg_rows, int max_blocks32,
                              uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, long ldc,
                              hipStream_t s) {
  if (rows == 0 || max_blocks32 == 0) return hipSuccess;
  dim3 grid((max_blocks32 + 3) / 4, (cols + kMxCols - 1) / kMxCols);
  if (bf16)
    mx_dual_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)in, ld_in, rows, cols, src, gk, seg_off,
                                                  seg_off32, nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  else
    mx_dual_kernel<float><<<grid, 256, 0, s>>>((const float*)in, ld_in, rows, cols, src, gk, seg_off, seg_off32,
                                               nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  return hipGetLastError();
}

}  // namespace trg
