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
//    stored MN-contiguous (dWr's both operands, dx's router weights) is read as
//    8x8 blocks of 16-byte row pieces and transposed in registers before the
//    LDS write, so every GEMM feeds the matrix cores from the same LDS layout.
//  * The MFMA is issued as (B fragment, A fragment): each lane then owns 4
//    consecutive output columns of one row, stored as one 16-byte write.
//  * One dense problem per launch, with an optional fixed-order split-K (fp32
//    partials); epilogues: fp32 store, read-add-write into a bf16 output, or
//    (the router's dx with the unpermute-sum folded in) the tile staged in LDS
//    as fp32 and written as whole 16-byte row pieces of
//    bf16(sum_j dxp[pos[m, j]] + product).  The last one reads each gathered
//    row piece once and writes dx once, where read-add-write after a separate
//    unpermute-sum moved dx three times.
#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace trg {

enum Epi { EPI_F32 = 1, EPI_ADD_BF16 = 4, EPI_UNPERMUTE = 8 };

struct GemmArgs {
  // A[m][k]: K-contiguous -> A[m*lda + k]; MN-contiguous -> A[k*lda + m]
  const uint16_t* A;
  long lda;
  const uint16_t* B;
  long ldb;
  void* C;
  long ldc;
  int M, N, K;
  int tiles_m, tiles_n;
  int ksplit_len;  // split-K: K elements per split (multiple of 64); 0 = none
  long c_split_stride;
  // EPI_UNPERMUTE: C[m] = bf16(sum_j dxp[pos[m*k + j]] + product[m]), rows of ldc
  const uint16_t* dxp;
  const int* pos;
  int k;
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

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  constexpr int BK = 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int STAGE = (BM + BN) * 8;  // uint4 per LDS stage
  static_assert(WM * WN == 4, "4 waves");
  static_assert(TM >= 1 && TN >= 1, "wave tile");
  constexpr int NA = AKC ? BM * 8 / 256 : ((BM + 255) / 256) * 8;
  constexpr int NB = BKC ? BN * 8 / 256 : ((BN + 255) / 256) * 8;
  static_assert(!AKC || (BM * 8) % 256 == 0, "A tile");
  static_assert(!BKC || (BN * 8) % 256 == 0, "B tile");
  constexpr int EP = BN + 4;  // fp32 row pitch of the staged tile (EPI_UNPERMUTE)
  constexpr int SMEM = (EPI == EPI_UNPERMUTE && BM * EP / 4 > 2 * STAGE) ? BM * EP / 4 : 2 * STAGE;
  __shared__ uint4 smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---------------- tile: (split, row tile, column tile) ----------------
  int t = blockIdx.x;
  const int per = g.tiles_m * g.tiles_n;
  const long split_idx = t / per;
  t -= (int)split_idx * per;
  const int mt = t / g.tiles_n, nt = t % g.tiles_n;
  const int m0 = mt * BM, m_end = g.M, n0 = nt * BN;
  int k0 = 0, k_end = g.K;
  if (g.ksplit_len > 0) {
    k0 = (int)split_idx * g.ksplit_len;
    k_end = min(g.K, k0 + g.ksplit_len);
  }
  const uint16_t* Ab = g.A;
  const uint16_t* Bb = g.B;

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
        const int gn = n0 + row, gk = kt + ch * 8;
        rb[i] = (gn < g.N && gk < k_end) ? *(const uint4*)(Bb + (long)gn * g.ldb + gk) : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NB / 8; ++i) {
        const int q = tid + 256 * i;
        const int kb = q / (BN / 8), nb = q % (BN / 8);
        const int gn = n0 + nb * 8;
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gk = kt + kb * 8 + r;
          rb[i * 8 + r] = (q < BN && gk < k_end && gn < g.N) ? *(const uint4*)(Bb + (long)gk * g.ldb + gn)
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
  if constexpr (EPI == EPI_UNPERMUTE) {
    // the product tile to LDS (the K loop ended with a barrier: the stages are free)
    float* st = (float*)smem;
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      static_for<TN>([&](auto J) {
        constexpr int j = decltype(J)::value;
        static_for<4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int r = wm * WTM + i * 32 + lrow, c = wn * WTN + j * 32 + q * 8 + lgrp;
          *(float4*)(st + r * EP + c) = make_float4(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1],
                                                    acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
        });
      });
    });
    __syncthreads();
    // 16-byte row pieces: 8 columns of one row; BN / 8 consecutive threads per
    // row, NP pieces per thread.  The position and row piece loads of two
    // slots of all NP pieces are issued together (one pair of round trips per
    // two slots, not per piece and slot); the sums still take the slots in
    // order.
    constexpr int PPR = BN / 8, NP = BM * PPR / 256;
    static_assert(BM * PPR % 256 == 0, "pieces per thread");
    long mrow[NP];
    int ncol[NP];
    bool ok[NP];
    float s[NP][8];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + 256 * i, r = p / PPR, c = (p % PPR) * 8;
      mrow[i] = m0 + r;
      ncol[i] = n0 + c;
      ok[i] = mrow[i] < m_end && ncol[i] < g.N;
#pragma unroll
      for (int z = 0; z < 8; ++z) s[i][z] = 0.f;
    }
    for (int j = 0; j < g.k; j += 2) {  // slots in order, fp32
      const bool two = j + 1 < g.k;
      int pj[2][NP];
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        pj[0][i] = ok[i] ? g.pos[mrow[i] * g.k + j] : 0;
        pj[1][i] = ok[i] && two ? g.pos[mrow[i] * g.k + j + 1] : 0;
      }
      uint4 v[2][NP];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int i = 0; i < NP; ++i)
          v[q][i] = ok[i] && (q == 0 || two) ? *(const uint4*)(g.dxp + (long)pj[q][i] * g.ldc + ncol[i])
                                             : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        if (q == 1 && !two) break;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const uint4 w = v[q][i];
          s[i][0] += bf_lo(w.x); s[i][1] += bf_hi(w.x); s[i][2] += bf_lo(w.y); s[i][3] += bf_hi(w.y);
          s[i][4] += bf_lo(w.z); s[i][5] += bf_hi(w.z); s[i][6] += bf_lo(w.w); s[i][7] += bf_hi(w.w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (ok[i]) {
        const int p = tid + 256 * i, r = p / PPR, c = (p % PPR) * 8;
        const float4 a0 = *(const float4*)(st + r * EP + c), a1 = *(const float4*)(st + r * EP + c + 4);
        *(uint4*)((uint16_t*)g.C + mrow[i] * g.ldc + ncol[i]) =
            make_uint4(pack_bf2(s[i][0] + a0.x, s[i][1] + a0.y), pack_bf2(s[i][2] + a0.z, s[i][3] + a0.w),
                       pack_bf2(s[i][4] + a1.x, s[i][5] + a1.y), pack_bf2(s[i][6] + a1.z, s[i][7] + a1.w));
      }
    }
    return;
  }
  static_for<TM>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const int m = m0 + wm * WTM + i * 32 + lrow;
    if (m < m_end) {
      static_for<TN>([&](auto J) {
        constexpr int j = decltype(J)::value;
        static_for<4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int n = n0 + wn * WTN + j * 32 + q * 8 + lgrp;
          if (n < g.N) {
            const float v0 = acc[i][j][q * 4 + 0], v1 = acc[i][j][q * 4 + 1];
            const float v2 = acc[i][j][q * 4 + 2], v3 = acc[i][j][q * 4 + 3];
            const long o = (long)m * g.ldc + n;
            if constexpr (EPI == EPI_F32) {
              *(float4*)((float*)g.C + split_idx * g.c_split_stride + o) = make_float4(v0, v1, v2, v3);
            } else {  // EPI_ADD_BF16: the bf16 output plus the product, rounded once more
              const uint2 old = *(uint2*)((uint16_t*)g.C + o);
              *(uint2*)((uint16_t*)g.C + o) = make_uint2(pack_bf2(bf_lo(old.x) + v0, bf_hi(old.x) + v1),
                                                         pack_bf2(bf_lo(old.y) + v2, bf_hi(old.y) + v3));
            }
          }
        });
      });
    }
  });
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

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int EPI>
static void run(const char* name, const GemmArgs& a, int grid, hipStream_t s) {
  if (grid <= 0) return;
  ProfScope ps(name, s);
  gemm_bf16_kernel<BM, BN, WM, WN, AKC, BKC, EPI><<<grid, 256, 0, s>>>(a);
}

// ---------------- router GEMMs on the matrix cores (E >= 64) ----------------

hipError_t launch_dense_nt_f32out(const uint16_t* A, const uint16_t* B, float* C, int M, int N, int K,
                                  hipStream_t s) {
  GemmArgs a{};
  a.A = A; a.lda = K;
  a.B = B; a.ldb = K;
  a.C = C; a.ldc = N;
  a.M = M; a.N = N; a.K = K;
  a.tiles_m = cdiv(M, 64); a.tiles_n = cdiv(N, 128);
  run<64, 128, 1, 4, true, true, EPI_F32>("router_logits_mfma", a, a.tiles_m * a.tiles_n, s);
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
  run<128, 128, 2, 2, false, false, EPI_F32>("router_dwr_mfma", a, sp * a.tiles_m * a.tiles_n, s);
  const long n = (long)E * d;
  splitk_reduce_bf16_kernel<<<cdiv(n / 4, 256), 256, 0, s>>>(part, sp, n, dwr);
  return hipGetLastError();
}

hipError_t launch_router_dx_mfma(const uint16_t* dL, const uint16_t* wr, uint16_t* dx, const uint16_t* dxp,
                                 const int* pos, int k, int T, int d, int E, hipStream_t s) {
  GemmArgs a{};
  a.A = dL; a.lda = E;  // A[m=t][k=e] K-contiguous
  a.B = wr; a.ldb = d;  // B[n=c][k=e] = wr[e][c], MN-contiguous
  a.C = dx; a.ldc = d;
  a.M = T; a.N = d; a.K = E;
  a.tiles_m = cdiv(T, 128); a.tiles_n = cdiv(d, 128);
  if (dxp != nullptr) {  // dx = unpermute-sum of dxp + dL wr
    a.dxp = dxp; a.pos = pos; a.k = k;
    run<128, 128, 2, 2, true, false, EPI_UNPERMUTE>("router_dx_mfma", a, a.tiles_m * a.tiles_n, s);
  } else {
    run<128, 128, 2, 2, true, false, EPI_ADD_BF16>("router_dx_mfma", a, a.tiles_m * a.tiles_n, s);
  }
  return hipGetLastError();
}

}  // namespace trg
