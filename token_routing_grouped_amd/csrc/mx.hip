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
//   column layout   blocks of 32 consecutive rows inside each segment,
//                   zero-padded at the segment's end (the weight-gradient K),
//                   stored expert-major.  Gathered segments (padded rows
//                   off128[e] .. off128[e+1], len_e of them): segment e is the
//                   block [cols, len_e] at byte off128[e] * cols, so column c
//                   of the segment is one row of len_e bytes.  Fixed segments
//                   (the weights' dgrad copies): [nseg * cols, ldc], row
//                   e * cols + c holding column c of segment e.  One segment:
//                   the plain transpose [cols, ldc].
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

// bf16 blocks are quantised from packed pairs (two bf16 per dword) without
// unpacking them to fp32:
//   amax: an unsigned 16-bit max of the magnitude bits (bf16 magnitudes order
//   like their bit patterns), whose exponent field gives the scale byte
//   max(ex - 8, 0): the same s as mx_scale_exp for every finite block;
//   codes: gfx950's scaled conversion divides each value by the scale operand
//   (2^s, a float subnormal for s = -127) and rounds to nearest even, but
//   returns the NaN code S.1111.111 where the quotient overflows +-448 instead
//   of saturating; nan_to_448 turns those bytes into S.1111.110 (+-448).  On
//   every bf16 bit pattern and scales 2^-127 .. 2^119 a hardware probe gave
//   the same bytes as the clamp + unscaled conversion path used for fp32.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));

TRG_DEV uint32_t nan_to_448(uint32_t w) {
  const uint32_t t = ((w & 0x7f7f7f7fu) + 0x01010101u) & 0x80808080u;  // bit 7 set where a byte is S.1111.111
  return w ^ (t >> 7);
}
// Codes of the four bf16 values in the pairs a, b (bytes in element order).
TRG_DEV uint32_t e4m3_bf16x4(uint32_t a, uint32_t b, float scale) {
  // the first conversion writes the low half over a's own bits (no zeroing
  // move), the second the high half
  i16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(i16x2_t, a), __builtin_bit_cast(bf16x2_t, a),
                                                        scale, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, b), scale, true);
  return nan_to_448(__builtin_bit_cast(uint32_t, r));
}
// Scale byte of a block of 2n bf16 values held as n pairs.
template <int N>
TRG_DEV int scale_byte_bf16(const uint32_t* p) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, p[0] & 0x7fff7fffu);
#pragma unroll
  for (int q = 1; q < N; ++q) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, p[q] & 0x7fff7fffu));
  const int amax = max((int)m.x, (int)m.y);
  return max(((amax >> 7) & 0xff) - 8, 0);
}
// The scale operand 2^(sb - 127) of scale byte sb.
TRG_DEV float scale_of_byte(int sb) { return __uint_as_float(sb ? (uint32_t)sb << 23 : 0x00400000u); }
// The eight code dwords of a 32-value bf16 block held as 16 pairs.
TRG_DEV void quant_block_bf16(const uint32_t* p, int sb, uint32_t* w) {
  const float sc = scale_of_byte(sb);
#pragma unroll
  for (int q = 0; q < 8; ++q) w[q] = e4m3_bf16x4(p[2 * q], p[2 * q + 1], sc);
}

constexpr int kMxRows = 128;  // padded rows per workgroup (four 32-row blocks)
constexpr int kMxCols = 128;  // columns per workgroup

// OR of v over the four lanes 4q .. 4q+3 (all of them take part).
TRG_DEV uint32_t or4(uint32_t v) {
  v |= __shfl_xor(v, 1);
  return v | __shfl_xor(v, 2);
}
// OR of v over the N (2 or 4) neighbouring lanes of an aligned group.
template <int N>
TRG_DEV uint32_t or_n(uint32_t v) {
  v |= __shfl_xor(v, 1);
  if constexpr (N == 4) v |= __shfl_xor(v, 2);
  return v;
}

// Segment of the 32-row block starting at padded row base32: the block's first
// source row, the segment's end row; false past the padded row space.
TRG_DEV bool mx_block_rows(int base32, int rows, const int* seg_off, const int* seg_off128, int nseg, int seg_rows,
                           int& r0, int& seg_hi, int& pstart, int& plen) {
  if (seg_off != nullptr) {
    if (base32 >= seg_off128[nseg]) return false;
    int lo = 0, hi = nseg;  // last e with seg_off128[e] <= base32
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (seg_off128[mid] <= base32) lo = mid; else hi = mid;
    }
    r0 = seg_off[lo] + (base32 - seg_off128[lo]);
    seg_hi = seg_off[lo + 1];
    pstart = seg_off128[lo];
    plen = seg_off128[lo + 1] - seg_off128[lo];
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

// One workgroup: RB rows of the padded row space (NB = RB/32 blocks of 32
// rows, each inside one segment) x 128 columns, 256 threads.
//   rowwise pass: unit u -> row u/4, 32 columns from (u%4)*32: the four units
//   of a row are neighbouring lanes, so each row's 128 payload bytes go out as
//   one piece and its 4 scale bytes as one dword (RB/64 units per thread);
//   columnwise pass: unit u -> column u/NB, 32-row block u%NB: NB*32 payload
//   bytes of a column as one piece, its scale bytes as dwords (four blocks
//   each) or, for NB = 2, a half dword (NB/2 units per thread).
// RB = 128 makes each column's payload piece one whole 128-byte line: with RB
// = 64 (half the LDS, twice the workgroups per CU) the half-line pieces made
// the weights' two-layout pass 30% slower, and RB = 256 (two-line pieces, two
// workgroups per CU) 5% slower.
template <class T, int RB>
__global__ __launch_bounds__(256) void mx_dual_kernel(const T* __restrict__ in, long ld_in, int rows, int cols,
                                                      const int* __restrict__ src, int gk,
                                                      const float* __restrict__ gate,
                                                      const int* __restrict__ seg_off,
                                                      const int* __restrict__ seg_off128, int nseg, int seg_rows,
                                                      uint8_t* __restrict__ q_row, uint8_t* __restrict__ s_row,
                                                      uint8_t* __restrict__ q_col, uint8_t* __restrict__ s_col,
                                                      long ldc) {
  // The tile keeps the source values in their own type.  Row pitch kMxCols +
  // PAD elements plus 64 bytes per 32-row block: the columnwise pass reads
  // its blocks x columns of a wave from distinct banks.
  constexpr int NB = RB / 32, KU = RB / 64, KC = NB / 2;
  constexpr int PAD = sizeof(T) == 2 ? 2 : 1;
  constexpr int PITCH = kMxCols + PAD;
  constexpr int BLKSKIP = 64 / sizeof(T);
  constexpr int V = 16 / sizeof(T);  // values per 16-byte load
  __shared__ __attribute__((aligned(16))) T tile[RB * PITCH + NB * BLKSKIP];
  static_assert(sizeof(tile) >= 1025 * sizeof(int), "the segment starts are staged in the tile");
  auto at = [&](int r, int c) -> T& { return tile[r * PITCH + (r >> 5) * BLKSKIP + c]; };
  const int tid = threadIdx.x, q4 = tid & 3;
  // workgroups walk the column blocks of a row band first: neighbouring
  // workgroups read neighbouring pieces of the same source rows
  const int ncb = (cols + kMxCols - 1) / kMxCols;
  const int base = (int)(blockIdx.x / ncb) * RB;
  const int col0 = (int)(blockIdx.x % ncb) * kMxCols;
  // whole scale dwords (a row's four blocks of a 128-chunk) where the base is
  // 4-byte aligned and all four blocks are written
  const bool row_dw = ((uintptr_t)s_row & 3) == 0;
  // Fixed segments (weights: experts of seg_rows rows) go out expert-major:
  // the columnwise copy is an MX matrix of nsegf * cols rows, row e * cols + c
  // holding column c of segment e (its padded rows, row stride ldc), so a GEMM
  // that reads one expert's copy reads rows ldc bytes apart.  A single
  // segment (seg_rows = rows) is the plain transpose either way.
  const bool emaj = seg_off == nullptr && seg_rows < rows;
  const int seg32 = (seg_rows + 31) / 32 * 32;
  const int nsegf = emaj ? rows / seg_rows : 1;
  const bool col_dw = ((uintptr_t)s_col & 3) == 0 && (!emaj || seg32 % 128 == 0);

  // The band's 32-row blocks -> (first source row, segment end, valid),
  // looked up once per workgroup.  Segment starts go through LDS first (one
  // coalesced load instead of a chain of dependent loads per thread: the
  // search's latency was a large part of a band's time); they sit in the
  // tile's space, which is written only after the lookup.
  int* s_off = (int*)tile;
  __shared__ int blk[NB][5];  // first source row, segment end, valid, padded segment start and length
  if (seg_off != nullptr && nseg <= 1024) {
    for (int e = tid; e <= nseg; e += 256) s_off[e] = seg_off128[e];
    __syncthreads();
  }
  if (tid < NB) {
    const int b32 = base + tid * 32;
    int r0 = 0, seg_hi = 0, ok = 0, pstart = 0, plen = 0;
    if (seg_off != nullptr && nseg <= 1024) {
      if (b32 < s_off[nseg]) {
        int lo = 0, hi = nseg;  // last e with seg_off128[e] <= b32
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_off[mid] <= b32) lo = mid; else hi = mid;
        }
        r0 = seg_off[lo] + (b32 - s_off[lo]);
        seg_hi = seg_off[lo + 1];
        pstart = s_off[lo];
        plen = s_off[lo + 1] - s_off[lo];
        ok = 1;
      }
    } else {
      ok = mx_block_rows(b32, rows, seg_off, seg_off128, nseg, seg_rows, r0, seg_hi, pstart, plen) ? 1 : 0;
    }
    blk[tid][0] = r0;
    blk[tid][1] = seg_hi;
    blk[tid][2] = ok;
    blk[tid][3] = pstart;
    blk[tid][4] = plen;
  }
  __syncthreads();

  // ---- rowwise: all units' loads first
  uint4 raw[KU][32 / V];
  int rr[KU];
  bool rok[KU];
#pragma unroll
  for (int k = 0; k < KU; ++k) {
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
  for (int k = 0; k < KU; ++k) {
    const int i = (tid >> 2) + 64 * k;
    const int c = col0 + q4 * 32;
    // the source bits go to the tile as they are
#pragma unroll
    for (int z = 0; z < 32; ++z) at(i, q4 * 32 + z) = ((const T*)raw[k])[z];
    if (q_row != nullptr) {
      int s;
      uint32_t w[8];
      if constexpr (sizeof(T) == 2) {
        const uint32_t* pr = (const uint32_t*)raw[k];
        const int sb = scale_byte_bf16<16>(pr);
        s = sb - 127;
        quant_block_bf16(pr, sb, w);
      } else {
        float v[32];
#pragma unroll
        for (int q = 0; q < 32 / V; ++q) unpack16<T>(raw[k][q], v + q * V);
        float amax = 0.f;
#pragma unroll
        for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(v[z]));
        s = mx_scale_exp(amax);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = e4m3_x4(ldexpf(v[q * 4], -s), ldexpf(v[q * 4 + 1], -s), ldexpf(v[q * 4 + 2], -s),
                         ldexpf(v[q * 4 + 3], -s));
      }
      const uint32_t all = or4((rok[k] ? 1u : 0u) << q4);
      const uint32_t sw = or4((uint32_t)(s + 127) << (8 * q4));
      if (rok[k]) {
        uint4* dst = (uint4*)(q_row + (long)rr[k] * cols + c);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
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
  for (int k = 0; k < KC; ++k) {
    const int cc = tid / NB + (256 / NB) * k, sb = tid % NB;
    const int c = col0 + cc;
    const bool ok = blk[sb][2] != 0 && c < cols;
    int s;
    uint32_t w[8];
    if constexpr (sizeof(T) == 2) {
      uint32_t pr[16];  // rows 2j, 2j+1 of the column as one pair
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        u16x2_t pj;
        pj.x = at(sb * 32 + 2 * j, cc);
        pj.y = at(sb * 32 + 2 * j + 1, cc);
        pr[j] = __builtin_bit_cast(uint32_t, pj);
      }
      const int sbyte = scale_byte_bf16<16>(pr);
      s = sbyte - 127;
      quant_block_bf16(pr, sbyte, w);
    } else {
      float x[32];
#pragma unroll
      for (int z = 0; z < 32; ++z) x[z] = to_f32(at(sb * 32 + z, cc));
      float amax = 0.f;
#pragma unroll
      for (int z = 0; z < 32; ++z) amax = fmaxf(amax, fabsf(x[z]));
      s = mx_scale_exp(amax);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        w[q] = e4m3_x4(ldexpf(x[q * 4], -s), ldexpf(x[q * 4 + 1], -s), ldexpf(x[q * 4 + 2], -s),
                       ldexpf(x[q * 4 + 3], -s));
    }
    // scale bytes in groups of G neighbouring lanes (blocks): one dword (G =
    // 4) or half dword (G = 2) from the group's first lane
    constexpr int G = NB < 4 ? NB : 4;
    const int sg = sb % G;
    const uint32_t all = or_n<G>((ok ? 1u : 0u) << sg);
    const uint32_t sw = or_n<G>((uint32_t)(s + 127) << (8 * sg));
    if (ok) {
      // (matrix row, padded row inside it, rows of the MX matrix)
      long mrow = c;
      int pr = base + sb * 32;
      long nrow = cols;
      uint8_t* qdst;
      if (emaj) {
        const int e = pr / seg32;
        mrow = (long)e * cols + c;
        pr -= e * seg32;
        nrow = (long)nsegf * cols;
        qdst = q_col + mrow * ldc + pr;
      } else if (seg_off != nullptr) {
        // segment e's copy is one [cols, len_e] block at byte off128[e] * cols
        const int ps = blk[sb][3], pl = blk[sb][4];
        qdst = q_col + (long)ps * cols + (long)c * pl + (pr - ps);
      } else {
        qdst = q_col + (long)c * ldc + pr;
      }
      uint4* dst = (uint4*)qdst;
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      const int b = pr >> 5;  // block along the (segment's) padded rows
      uint8_t* sp = s_col + ((long)(b >> 2) * nrow + mrow) * 4 + (b & 3);
      if (col_dw && all == (1u << G) - 1) {  // the group's G bytes at once (base is a multiple of RB)
        if (sg == 0) {
          if constexpr (G == 4) *(uint32_t*)sp = sw;
          else *(uint16_t*)sp = (uint16_t)sw;
        }
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
  constexpr int NB = kMxRows / 32;
  const long nblk = (long)((max_blocks32 + NB - 1) / NB) * ((cols + kMxCols - 1) / kMxCols);
  if (nblk > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)nblk;
  if (bf16)
    mx_dual_kernel<uint16_t, kMxRows><<<grid, 256, 0, s>>>((const uint16_t*)in, ld_in, rows, cols, src, gk, gate, seg_off,
                                                  seg_off128, nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  else
    mx_dual_kernel<float, kMxRows><<<grid, 256, 0, s>>>((const float*)in, ld_in, rows, cols, src, gk, gate, seg_off, seg_off128,
                                               nseg, seg_rows, q_row, s_row, q_col, s_col, ldc);
  return hipGetLastError();
}

}  // namespace trg
