// Register-staged bf16 GEMMs on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation, used for the router's dense products when the expert count
// makes them real GEMMs (logits, dWr with a fixed-order split-K, dx).  The
// grouped expert GEMMs live in ggemm.hip.
//
// Design (CDNA4-first):
//  * 256 threads = 4 waves in a WM x WN grid; block tile BM x BN, K step 64.
//  * Both operands are staged in LDS as [rows][64] bf16 (128 B rows) with a
//    16-byte-chunk XOR swizzle (chunk ^ (row & 7)), double-buffered through
//    registers: the next K tile's global loads are issued before the current
//    tile's MFMAs.
//  * An operand stored K-contiguous is copied with 16-byte loads.  An operand
//    stored MN-contiguous (the dgrad / wgrad cases) is read as 8x8 blocks of
//    16-byte row pieces and transposed in registers before the LDS write, so
//    every GEMM feeds the matrix cores from the same LDS layout.
//  * The MFMA is issued as (B fragment, A fragment): each lane then owns 4
//    consecutive output columns of one row, stored as one 8- or 16-byte write.
//  * Grouping modes: DENSE (one problem, optional split-K), RAGGED_M (expert
//    segments of the routed rows; the per-expert tile prefix is derived on the
//    device from the offsets), RAGGED_K (weight gradients: the reduction runs
//    over the expert's rows).
//  * Epilogues: bf16 / fp32 store, SwiGLU forward (G, U, H), SwiGLU backward
//    (dG, dU from dH, G, U), and read-add-write bf16.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace trg {

enum Mode { DENSE = 0, RAGGED_M = 1, RAGGED_K = 2 };
enum BSel { BSEL_NONE = 0, BSEL_GLU = 1, BSEL_KSPLIT = 2 };
enum CSel { CSEL_NONE = 0, CSEL_MSPLIT = 1 };
enum Epi { EPI_BF16 = 0, EPI_F32 = 1, EPI_SWIGLU_FWD = 2, EPI_SWIGLU_BWD = 3, EPI_ADD_BF16 = 4 };

struct GemmArgs {
  // A[m][k]: K-contiguous -> A[m*lda + k]; MN-contiguous -> A[k*lda + m]
  const uint16_t* A;
  long lda, a_es;  // a_es: per-expert element stride (0 = shared)
  const uint16_t* B;
  const uint16_t* B2;  // second matrix for BSEL_GLU / BSEL_KSPLIT
  long ldb, b_es;
  void* C;
  void* C2;  // CSEL_MSPLIT second output; SWIGLU_FWD: U
  void* C3;  // SWIGLU_FWD: H
  long ldc, c_es;
  const uint16_t* G;  // SWIGLU_BWD inputs
  const uint16_t* U;
  long ldgu;
  int M, N, K;
  int split;  // h: GLU rows per matrix / K split point / M split point
  const int* offsets;
  const int* tile_off;
  int E;
  int tiles_m, tiles_n;
  int ksplit_len;  // DENSE split-K: K elements per split (multiple of 64); 0 = none
  long c_split_stride;
};

TRG_DEV bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8x8 transpose of 16-bit elements: in[r] holds row r (8 elements), out[c]
// holds column c.
TRG_DEV void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t I[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    I[r][0] = in[r].x; I[r][1] = in[r].y; I[r][2] = in[r].z; I[r][3] = in[r].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t x = I[2 * p][c >> 1], y = I[2 * p + 1][c >> 1];
      d[p] = (c & 1) ? __builtin_amdgcn_perm(y, x, 0x07060302u) : __builtin_amdgcn_perm(y, x, 0x05040100u);
    }
    out[c] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int MODE, int BSEL, int CSEL, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int STAGE = (BM + BN) * 8;  // uint4 per LDS stage
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  static_assert(BSEL != BSEL_GLU || (TN % 2 == 0), "GLU pairs subtiles");
  constexpr int NA = AKC ? BM * 8 / 256 : ((BM + 255) / 256) * 8;
  constexpr int NB = BKC ? BN * 8 / 256 : ((BN + 255) / 256) * 8;
  static_assert(!AKC || (BM * 8) % 256 == 0, "A tile");
  static_assert(!BKC || (BN * 8) % 256 == 0, "B tile");
  __shared__ uint4 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---------------- tile decode ----------------
  int e = 0, m0, m_end, n0, k0, k_end;
  long split_idx = 0;
  if constexpr (MODE == DENSE) {
    int t = blockIdx.x;
    const int per = g.tiles_m * g.tiles_n;
    split_idx = t / per;
    t -= (int)split_idx * per;
    const int mt = t / g.tiles_n, nt = t % g.tiles_n;
    m0 = mt * BM;
    m_end = g.M;
    n0 = nt * BN;
    if (g.ksplit_len > 0) {
      k0 = (int)split_idx * g.ksplit_len;
      k_end = min(g.K, k0 + g.ksplit_len);
    } else {
      k0 = 0;
      k_end = g.K;
    }
  } else if constexpr (MODE == RAGGED_M) {
    const int t = blockIdx.x;
    const int mtg = t / g.tiles_n, nt = t % g.tiles_n;
    if (mtg >= g.tile_off[g.E]) return;  // beyond the real tile count: whole block exits
    int lo = 0, hi = g.E;                // last expert with tile_off[e] <= mtg
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (g.tile_off[mid] <= mtg) lo = mid; else hi = mid;
    }
    e = lo;
    m0 = g.offsets[e] + (mtg - g.tile_off[e]) * BM;
    m_end = g.offsets[e + 1];
    n0 = nt * BN;
    k0 = 0;
    k_end = g.K;
  } else {
    int t = blockIdx.x;
    const int per = g.tiles_m * g.tiles_n;
    e = t / per;
    t -= e * per;
    const int mt = t / g.tiles_n, nt = t % g.tiles_n;
    m0 = mt * BM;
    m_end = g.M;
    n0 = nt * BN;
    k0 = g.offsets[e];
    k_end = g.offsets[e + 1];
  }

  const uint16_t* Ab = g.A + (long)e * g.a_es;
  const uint16_t* Bb = g.B + (long)e * g.b_es;
  const uint16_t* B2b = (BSEL != BSEL_NONE) ? g.B2 + (long)e * g.b_es : nullptr;

  uint4 ra[NA], rb[NB];

  // ---------------- global -> registers ----------------
  auto load_a = [&](int kt) {
    if constexpr (AKC) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int q = tid + 256 * i, row = q >> 3, ch = q & 7;
        const int gm = m0 + row, gk = kt + ch * 8;
        ra[i] = (gm < m_end && gk < k_end) ? *(const uint4*)(Ab + (long)gm * g.lda + gk) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA / 8; ++i) {
        const int q = tid + 256 * i;
        const int kb = q / (BM / 8), mb = q % (BM / 8);
        const int gm = m0 + mb * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gk = kt + kb * 8 + r;
          ra[i * 8 + r] = (q < BM && gk < k_end && gm < m_end) ? *(const uint4*)(Ab + (long)gk * g.lda + gm)
                                                                : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto load_b = [&](int kt) {
    if constexpr (BKC) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = tid + 256 * i, row = q >> 3, ch = q & 7;
        const int gk = kt + ch * 8;
        const uint16_t* src;
        bool ok;
        if constexpr (BSEL == BSEL_GLU) {
          const int part = row / WTN, p = row % WTN;
          const int which = p / (WTN / 2);
          const int hh = n0 / 2 + part * (WTN / 2) + p % (WTN / 2);
          src = (which ? B2b : Bb) + (long)hh * g.ldb + gk;
          ok = hh < g.split && gk < k_end;
        } else {
          const int gn = n0 + row;
          src = Bb + (long)gn * g.ldb + gk;
          ok = gn < g.N && gk < k_end;
        }
        rb[i] = ok ? *(const uint4*)src : make_uint4(0, 0, 0, 0);
      }
    } else {
      const uint16_t* base = Bb;
      int krel = kt;
      if constexpr (BSEL == BSEL_KSPLIT) {
        if (kt >= g.split) {
          base = B2b;
          krel = kt - g.split;
        }
      }
#pragma unroll
      for (int i = 0; i < NB / 8; ++i) {
        const int q = tid + 256 * i;
        const int kb = q / (BN / 8), nb = q % (BN / 8);
        const int gn = n0 + nb * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gk = kt + kb * 8 + r;
          const int kr = krel + kb * 8 + r;
          rb[i * 8 + r] = (q < BN && gk < k_end && gn < g.N) ? *(const uint4*)(base + (long)kr * g.ldb + gn)
                                                               : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  // ---------------- registers -> LDS ----------------
  auto store_tiles = [&](int buf) {
    uint4* sA = smem + buf * STAGE;
    uint4* sB = sA + BM * 8;
    if constexpr (AKC) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int q = tid + 256 * i, row = q >> 3, ch = q & 7;
        sA[row * 8 + (ch ^ (row & 7))] = ra[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA / 8; ++i) {
        const int q = tid + 256 * i;
        if (q < BM) {
          const int kb = q / (BM / 8), mb = q % (BM / 8);
          uint4 in[8], out[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) in[r] = ra[i * 8 + r];
          transpose8x8(in, out);
#pragma unroll
          for (int c = 0; c < 8; ++c) sA[(mb * 8 + c) * 8 + (kb ^ c)] = out[c];
        }
      }
    }
    if constexpr (BKC) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int q = tid + 256 * i, row = q >> 3, ch = q & 7;
        sB[row * 8 + (ch ^ (row & 7))] = rb[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB / 8; ++i) {
        const int q = tid + 256 * i;
        if (q < BN) {
          const int kb = q / (BN / 8), nb = q % (BN / 8);
          uint4 in[8], out[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) in[r] = rb[i * 8 + r];
          transpose8x8(in, out);
#pragma unroll
          for (int c = 0; c < 8; ++c) sB[(nb * 8 + c) * 8 + (kb ^ c)] = out[c];
        }
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = k_end > k0 ? (k_end - k0 + BK - 1) / BK : 0;
  if (nk > 0) {
    load_a(k0);
    load_b(k0);
    store_tiles(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      const int cur = it & 1;
      if (it + 1 < nk) {
        load_a(k0 + (it + 1) * BK);
        load_b(k0 + (it + 1) * BK);
      }
      const uint4* sA = smem + cur * STAGE;
      const uint4* sB = sA + BM * 8;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = kk * 2 + (lane >> 5);
        const int sw = ch ^ (lane & 7);
        uint4 af[TM], bfr[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = sA[(wm * WTM + i * 32 + (lane & 31)) * 8 + sw];
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[j] = sB[(wn * WTN + j * 32 + (lane & 31)) * 8 + sw];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(bfr[j]), as_bf16x8(af[i]), acc[i][j], 0,
                                                                0, 0);
      }
      if (it + 1 < nk) store_tiles(cur ^ 1);
      __syncthreads();
    }
  }

  // ---------------- epilogue ----------------
  // Lane (lrow, lgrp) owns rows m = ... + lrow and 4 consecutive columns per
  // group q: n = ... + q*8 + lgrp + {0..3}.
  const int lrow = lane & 31, lgrp = (lane >> 5) * 4;
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    uint16_t* Gp = (uint16_t*)g.C;
    uint16_t* Up = (uint16_t*)g.C2;
    uint16_t* Hp = (uint16_t*)g.C3;
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int m = m0 + wm * WTM + i * 32 + lrow;
      if (m < m_end) {
        static_for<TN / 2>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            const int hh = n0 / 2 + wn * (WTN / 2) + j * 32 + q * 8 + lgrp;
            if (hh < g.split) {
              float gv[4], uv[4], hv[4];
              static_for<4>([&](auto Rr) {
                constexpr int r = decltype(Rr)::value;
                gv[r] = acc[i][j][q * 4 + r];
                uv[r] = acc[i][j + TN / 2][q * 4 + r];
                hv[r] = silu_f(gv[r]) * uv[r];
              });
              const long o = (long)m * g.ldc + hh;
              *(uint2*)(Gp + o) = make_uint2(pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3]));
              *(uint2*)(Up + o) = make_uint2(pack_bf2(uv[0], uv[1]), pack_bf2(uv[2], uv[3]));
              *(uint2*)(Hp + o) = make_uint2(pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3]));
            }
          });
        });
      }
    });
  } else {
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int m = m0 + wm * WTM + i * 32 + lrow;
      if (m < m_end) {
        void* Cb = g.C;
        int mrow0 = 0;
        if constexpr (CSEL == CSEL_MSPLIT) {
          if (m >= g.split) {
            Cb = g.C2;
            mrow0 = g.split;
          }
        }
        static_for<TN>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            const int n = n0 + wn * WTN + j * 32 + q * 8 + lgrp;
            if (n < g.N) {
              const float v0 = acc[i][j][q * 4 + 0], v1 = acc[i][j][q * 4 + 1];
              const float v2 = acc[i][j][q * 4 + 2], v3 = acc[i][j][q * 4 + 3];
              const long o = (long)e * g.c_es + (long)(m - mrow0) * g.ldc + n;
              if constexpr (EPI == EPI_BF16) {
                *(uint2*)((uint16_t*)Cb + o) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
              } else if constexpr (EPI == EPI_F32) {
                *(float4*)((float*)Cb + split_idx * g.c_split_stride + o) = make_float4(v0, v1, v2, v3);
              } else if constexpr (EPI == EPI_ADD_BF16) {
                const uint2 old = *(uint2*)((uint16_t*)Cb + o);
                *(uint2*)((uint16_t*)Cb + o) = make_uint2(pack_bf2(bf_lo(old.x) + v0, bf_hi(old.x) + v1),
                                                          pack_bf2(bf_lo(old.y) + v2, bf_hi(old.y) + v3));
              } else if constexpr (EPI == EPI_SWIGLU_BWD) {
                // (v0..v3) = dH[m][n..n+3]; n indexes h
                const long gu = (long)m * g.ldgu + n;
                const uint2 gw = *(const uint2*)(g.G + gu);
                const uint2 uw = *(const uint2*)(g.U + gu);
                const float vv[4] = {v0, v1, v2, v3};
                const float gg[4] = {bf_lo(gw.x), bf_hi(gw.x), bf_lo(gw.y), bf_hi(gw.y)};
                const float uu[4] = {bf_lo(uw.x), bf_hi(uw.x), bf_lo(uw.y), bf_hi(uw.y)};
                float dg[4], du[4];
                static_for<4>([&](auto Rr) {
                  constexpr int r = decltype(Rr)::value;
                  const float s = sigmoid_f(gg[r]);
                  du[r] = vv[r] * gg[r] * s;
                  dg[r] = vv[r] * uu[r] * s * (1.0f + gg[r] * (1.0f - s));
                });
                uint16_t* D = (uint16_t*)Cb + (long)m * g.ldc;
                *(uint2*)(D + n) = make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
                *(uint2*)(D + g.split + n) = make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
              }
            }
          });
        });
      }
    });
  }
}

// Fixed-order sum of split-K partials: out[i] = sum_s part[s][i].
__global__ __launch_bounds__(256) void splitk_reduce_bf16_kernel(const float* __restrict__ part, int splits, long n,
                                                                 uint16_t* __restrict__ out) {
  const long i4 = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i4 >= n) return;
  float4 s = *(const float4*)(part + i4);
  for (int k = 1; k < splits; ++k) {
    const float4 v = *(const float4*)(part + (long)k * n + i4);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  *(uint2*)(out + i4) = make_uint2(pack_bf2(s.x, s.y), pack_bf2(s.z, s.w));
}

static inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int MODE, int BSEL, int CSEL, int EPI>
static void run(const char* name, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return;
  ProfScope ps(name, s);
  gemm_bf16_kernel<BM, BN, WM, WN, AKC, BKC, MODE, BSEL, CSEL, EPI><<<grid, 256, 0, s>>>(a);
}

// ---------------- router GEMMs on the matrix cores (E >= 64) ----------------

hipError_t launch_dense_nt_f32out(const uint16_t* A, const uint16_t* B, float* C, int M, int N, int K,
                                  hipStream_t s) {
  GemmArgs a{};
  a.A = A; a.lda = K;
  a.B = B; a.ldb = K;
  a.C = C; a.ldc = N;
  a.M = M; a.N = N; a.K = K;
  a.tiles_m = cdiv(M, 128); a.tiles_n = cdiv(N, 128);
  run<128, 128, 2, 2, true, true, DENSE, BSEL_NONE, CSEL_NONE, EPI_F32>("router_logits_mfma", a, a.tiles_m * a.tiles_n, s);
  return hipGetLastError();
}

static void dwr_split(int T, int d, int E, int* splits, int* klen) {
  const int tiles = cdiv(E, 128) * cdiv(d, 128);
  int sp = cdiv(512, tiles);
  const int kmax = cdiv(T, 64);
  if (sp > kmax) sp = kmax;
  if (sp < 1) sp = 1;
  int kl = cdiv(cdiv(T, sp), 64) * 64;
  *splits = cdiv(T, kl);
  *klen = kl;
}

size_t router_dwr_mfma_part_bytes(int T, int d, int E) {
  int sp, kl;
  dwr_split(T, d, E, &sp, &kl);
  return (size_t)sp * E * d * sizeof(float);
}

hipError_t launch_router_dwr_mfma(const uint16_t* dL, const uint16_t* x, uint16_t* dwr, float* part, int T, int d,
                                  int E, hipStream_t s) {
  int sp, kl;
  dwr_split(T, d, E, &sp, &kl);
  GemmArgs a{};
  a.A = dL; a.lda = E;  // A[m=e][k=t] = dL[t][e]
  a.B = x; a.ldb = d;   // B[n=c][k=t] = x[t][c]
  a.C = part; a.ldc = d; a.c_split_stride = (long)E * d;
  a.M = E; a.N = d; a.K = T;
  a.tiles_m = cdiv(E, 128); a.tiles_n = cdiv(d, 128);
  a.ksplit_len = kl;
  run<128, 128, 2, 2, false, false, DENSE, BSEL_NONE, CSEL_NONE, EPI_F32>("router_dwr_mfma", a, sp * a.tiles_m * a.tiles_n, s);
  const long n = (long)E * d;
  splitk_reduce_bf16_kernel<<<cdiv(n / 4, 256), 256, 0, s>>>(part, sp, n, dwr);
  return hipGetLastError();
}

hipError_t launch_router_dx_mfma(const uint16_t* dL, const uint16_t* wr, uint16_t* dx, int T, int d, int E,
                                 hipStream_t s) {
  GemmArgs a{};
  a.A = dL; a.lda = E;  // A[m=t][k=e] K-contiguous
  a.B = wr; a.ldb = d;  // B[n=c][k=e] = wr[e][c], MN-contiguous
  a.C = dx; a.ldc = d;
  a.M = T; a.N = d; a.K = E;
  a.tiles_m = cdiv(T, 128); a.tiles_n = cdiv(d, 128);
  run<128, 128, 2, 2, true, false, DENSE, BSEL_NONE, CSEL_NONE, EPI_ADD_BF16>("router_dx_mfma", a, a.tiles_m * a.tiles_n, s);
  return hipGetLastError();
}

}  // namespace trg
