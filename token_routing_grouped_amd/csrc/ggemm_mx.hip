// MXFP8 grouped GEMMs on gfx950's scaled matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 operands, one E8M0 scale per 32
// K values on each side, fp32 accumulation).  MXFP8 is the low-precision path
// the pages describe as cutting both compute and the traffic between experts
// (Olmo-core 3 overview, "Precision optimisation with MXFP8").
//
// Every operand arrives quantised along its own GEMM's reduction dimension and
// stored K-contiguous (payload rows of bytes plus a scale row per 32 bytes), so
// one kernel shape serves all six GEMMs of the layer:
//   forward      up (SwiGLU epilogue), down                 ragged M
//   backward     dgrad down (SwiGLU-bwd epilogue), dgrad up  ragged M
//                wgrad down, wgrad up                        ragged K over
//                the experts' column segments (padded to 128
//                rows, so every K step's row pieces start on a 128-byte line)
// The scheduler, the HBM->LDS operand path and the epilogues are the bf16
// kernel's (ggemm_impl.h).  Differences:
//   * K step of 128 bytes = 128 values: LDS rows stay 128 bytes.
//   * A fragment is 32 bytes per lane: for a 64-wide k slice, lane l (row
//     l % 32, half h = l / 32) holds k [16h, 16h+16) and [32+16h, 32+16h+16);
//     its scale register covers the 32-wide block h of its row (probed on the
//     hardware).  Each K step's scale words are staged in LDS with its
//     operands.
//   * K is a multiple of 128 everywhere: the ragged-M side because the call
//     requires d and h to be, the weight gradients because their K segments
//     are the experts' 128-padded column segments (off128), whose padding
//     blocks the quantiser fills with zeros.
//   * Scales are stored K-chunk major (mx.hip): one K step's scale dwords for
//     256 consecutive rows are 1 KiB of contiguous memory, which one wave
//     moves into LDS with a single 16-byte-per-lane load.  (Loaded a dword per
//     row, 64 rows per instruction, they cost every MX GEMM 5-25% of its time.)
#include "ggemm_impl.h"

namespace trg {
namespace gg {

typedef int v8i32_t __attribute__((ext_vector_type(8)));
typedef int v4i32_t __attribute__((ext_vector_type(4)));

// Scale operands in the K-chunk-major layout: the dword of row r and K chunk
// c (128 values) is at base + c * step + 4 r.
struct MxArgs {
  const uint8_t* sA;   // A scales
  long sa_step;        // bytes per K chunk of A (4 x A's rows)
  const uint8_t* sB;   // B scales (GLU: W1; KSPLIT: the first K half)
  const uint8_t* sB2;  // GLU: W3; KSPLIT: the second K half
  long sb_step;        // bytes per K chunk of B
  int sb_row_es;       // B scale rows per expert (weights: N rows each, expert-major)
  long sA_bytes, sB_bytes;  // extents (bounds for the scale loads)
};

// 32-byte fragment of the 64-wide k slice kk for MFMA lane `lane`.
TRG_DEV v8i32_t frag_mx(const char* s, int base, int kk, int lane) {
  const int row = base + (lane & 31);
  const int h = lane >> 5;
  const int sw = (row >> 1) & 7;
  // native vector loads: each stays one 16-byte LDS read through to codegen
  const v4i32_t lo = *(const v4i32_t*)(s + row * 128 + (((kk * 4 + h) ^ sw) << 4));
  const v4i32_t hi = *(const v4i32_t*)(s + row * 128 + (((kk * 4 + 2 + h) ^ sw) << 4));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int BM, int BN, int WM, int WN, int MODE, int BSEL, int CSEL, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void ggemm_mx_kernel(Args g, MxArgs x) {
  constexpr int BK = 128;
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int SA = BM * 128, SB = BN * 128;
  constexpr int STAGE = SA + SB;
  static_assert(BM % 128 == 0 && BN % 128 == 0, "tile");
  static_assert(BSEL != BSEL_GLU || (TN % 2 == 0), "GLU pairs subtiles");
  // Each K step's scale dwords are staged in LDS next to its operands: 256
  // rows of A, 256 rows of B and, for the GLU B, 256 rows of W3 (1 KiB each,
  // one wave each; a 128-row operand reads 128 rows past its own, which it
  // ignores).
  constexpr int NSC = BSEL == BSEL_GLU ? 3 : 2;
  constexpr int SCB = NSC * 1024;
  static_assert(NSC <= WM * WN && BM <= 256 && BN <= 256, "one scale piece per wave");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 2 * SCB];

  const uint8_t* A = (const uint8_t*)g.A;
  const uint8_t* B = (const uint8_t*)g.B;
  const uint8_t* B2 = (const uint8_t*)g.B2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5;

  const int xcd = blockIdx.x & 7, lb = blockIdx.x >> 3, nbx = gridDim.x >> 3;
  // the schedule's per-expert prefixes, from the expert offsets
  __shared__ int pre[2 * 1025];
  __shared__ int ptmp[16];
  if constexpr (MODE == RAGGED_M) rm_prefix<BM, NW * 64>(g.offsets, g.E, g.split_tails, pre, ptmp);
  else wgrad_prefix<NW * 64>(g.offsets, g.E, g.kstep, pre, ptmp);
  // t runs over this XCD's walk: ragged M, positions of its RmSched slices;
  // ragged K, global tile indices of its work-balanced range
  int t_begin, t_end;
  RmSched rms{};
  if constexpr (MODE == RAGGED_M) {
    rms = rm_sched<BM>(pre, g.E, g.tiles_n, xcd);
    t_begin = 0;
    t_end = rms.nf + rms.nl;
  } else {
    wgrad_range(pre, g.E, g.tiles_m * g.tiles_n, g.E * g.tiles_m * g.tiles_n, xcd, t_begin, t_end);
  }

  const __amdgpu_buffer_rsrc_t rsSA = make_rsrc(x.sA, x.sA_bytes);
  const __amdgpu_buffer_rsrc_t rsSB = make_rsrc(x.sB, x.sB_bytes);
  const __amdgpu_buffer_rsrc_t rsSB2 = make_rsrc(BSEL != BSEL_NONE ? x.sB2 : x.sB, x.sB_bytes);
  static_assert(MODE == RAGGED_M || BSEL == BSEL_NONE, "weight gradients have one B");
  const int a_lane[2] = {kc_lane_off(lane, 0, (int)g.lda), kc_lane_off(lane, 1, (int)g.lda)};
  const int b_lane[2] = {kc_lane_off(lane, 0, (int)g.ldb), kc_lane_off(lane, 1, (int)g.ldb)};

  struct Tile {
    int e, m0, m_end, n0, k0, klen;
    int ld;  // weight gradients: the operands' row stride (the segment's padded length)
    __amdgpu_buffer_rsrc_t rsA, rsB, rsB2;
  };
  auto decode = [&](int t) {
    Tile c;
    if constexpr (MODE == RAGGED_M) {
      int nt;
      rm_tile<BM>(pre, g.offsets, g.E, g.tiles_n, rms, t, c.e, c.m0, c.m_end, nt);
      c.n0 = nt * BN;
      c.k0 = 0;
      c.klen = g.K;
      c.rsA = make_rsrc(A + (long)c.m0 * g.lda, (long)(g.R - c.m0) * g.lda);
      if constexpr (BSEL == BSEL_GLU) {
        const long hh0 = c.n0 / 2;
        c.rsB = make_rsrc(B + (long)c.e * g.b_es + hh0 * g.ldb, (g.split - hh0) * g.ldb);
        c.rsB2 = make_rsrc(B2 + (long)c.e * g.b_es + hh0 * g.ldb, (g.split - hh0) * g.ldb);
      } else {
        c.rsB = make_rsrc(B + (long)c.e * g.b_es + (long)c.n0 * g.ldb, (long)(g.N - c.n0) * g.ldb);
        c.rsB2 = (BSEL == BSEL_KSPLIT) ? make_rsrc(B2 + (long)c.e * g.b_es + (long)c.n0 * g.ldb,
                                                   (long)(g.N - c.n0) * g.ldb)
                                       : c.rsB;
      }
    } else {
      // weight gradients: K = the expert's 128-padded column segment; each
      // operand's copy of segment e is one [rows, klen] block at byte
      // off128[e] * rows (expert-major, mx_quantize)
      const int per_e = g.tiles_m * g.tiles_n;
      c.e = t / per_e;
      const int r = t - c.e * per_e;
      const int mt = r / g.tiles_n, nt = r - mt * g.tiles_n;
      c.m0 = mt * BM;
      c.m_end = g.M;
      c.n0 = nt * BN;
      c.k0 = g.offsets[c.e];
      c.klen = g.offsets[c.e + 1] - c.k0;
      c.ld = c.klen;
      c.rsA = make_rsrc(A + (long)c.k0 * g.M + (long)c.m0 * c.klen, (long)(g.M - c.m0) * c.klen);
      c.rsB = make_rsrc(B + (long)c.k0 * g.N + (long)c.n0 * c.klen, (long)(g.N - c.n0) * c.klen);
      c.rsB2 = c.rsB;
    }
    return c;
  };
  auto num_k = [&](const Tile& c) { return c.klen > 0 ? (c.klen + BK - 1) / BK : 0; };

  auto issue = [&](const Tile& c, int kt, int stage) {  // kt: K offset relative to c.k0
    char* sA = smem + stage * STAGE;
    char* sB = sA + SA;
    if constexpr (MODE == RAGGED_K) {  // both operands: rows of the segment's length
      const int ll[2] = {kc_lane_off(lane, 0, c.ld), kc_lane_off(lane, 1, c.ld)};
      load_kc<BM, NW>(sA, wave, ll, kt, c.ld, [&](int r8, int& r0) {
        r0 = r8;
        return c.rsA;
      });
      load_kc<BN, NW>(sB, wave, ll, kt, c.ld, [&](int r8, int& r0) {
        r0 = r8;
        return c.rsB;
      });
      return;
    }
    load_kc<BM, NW>(sA, wave, a_lane, kt, (int)g.lda, [&](int r8, int& r0) {
      r0 = r8;
      return c.rsA;
    });
    if constexpr (BSEL == BSEL_GLU) {
      load_kc<BN, NW>(sB, wave, b_lane, kt, (int)g.ldb, [&](int r8, int& r0) {
        const int p = r8 % WTN;
        r0 = (r8 / WTN) * (WTN / 2) + (p % (WTN / 2));
        return (p >= WTN / 2) ? c.rsB2 : c.rsB;
      });
    } else if constexpr (BSEL == BSEL_KSPLIT) {
      const bool second = kt >= g.split;
      load_kc<BN, NW>(sB, wave, b_lane, second ? kt - g.split : kt, (int)g.ldb, [&](int r8, int& r0) {
        r0 = r8;
        return second ? c.rsB2 : c.rsB;
      });
    } else {
      load_kc<BN, NW>(sB, wave, b_lane, kt, (int)g.ldb, [&](int r8, int& r0) {
        r0 = r8;
        return c.rsB;
      });
    }
  };

  // LDS scale pieces of a stage: [A 256 rows][B 256 rows][W3 256 rows (GLU)],
  // each the step's K chunk of consecutive rows (one wave, one 1 KiB load).
  auto issue_scales = [&](const Tile& c, int kt, int stage) {
    if (wave >= NSC) return;
    char* dst = smem + 2 * STAGE + stage * SCB + wave * 1024;
    if (wave == 0) {  // A rows m0.. of chunk (k0 + kt) / 128 (k0 = 0 on the ragged-M side)
      lds_load16(rsSA, dst, (int)(((c.k0 + kt) >> 7) * x.sa_step) + c.m0 * 4 + lane * 16);
    } else {
      int ktb = c.k0 + kt, row0 = c.n0;
      bool second = false;
      if constexpr (BSEL == BSEL_GLU) {
        second = wave == 2;  // W3 next to W1, the same hidden units
        row0 = c.n0 / 2;
      } else if constexpr (BSEL == BSEL_KSPLIT) {
        second = kt >= g.split;
        if (second) ktb -= g.split;
      }
      const long off = (long)(ktb >> 7) * x.sb_step + ((long)c.e * x.sb_row_es + row0) * 4;
      lds_load16(second ? rsSB2 : rsSB, dst, (int)off + lane * 16);
    }
  };
  // this lane's scale words of the step in `stage`, pre-shifted so that byte
  // 0 / byte 2 are the lane's blocks of slice 0 / slice 1
  auto lds_scales = [&](int stage, uint32_t(&sa)[TM], uint32_t(&sb)[TN]) {
    const char* sc = smem + 2 * STAGE + stage * SCB;
    const int l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = *(const uint32_t*)(sc + (wm * WTM + i * 32 + l32) * 4) >> (8 * half);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      int off;
      if constexpr (BSEL == BSEL_GLU)
        off = (j < TN / 2 ? 1024 : 2048) + (wn * (WTN / 2) + (j % (TN / 2)) * 32 + l32) * 4;
      else
        off = 1024 + (wn * WTN + j * 32 + l32) * 4;
      sb[j] = *(const uint32_t*)(sc + off) >> (8 * half);
    }
  };

  int t = t_begin + lb;
  Tile cur;
  uint32_t sa[TM], sb[TN];  // this step's scale words
  if (t < t_end) {
    cur = decode(t);
    if (num_k(cur) > 0) {
      issue(cur, 0, 0);
      issue_scales(cur, 0, 0);
    }
  }
  for (; t < t_end; t += nbx) {
    const int e = cur.e, m0 = cur.m0, m_end = cur.m_end, n0 = cur.n0;
    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    const int nk = num_k(cur);
    // Ragged M: the wave's 32-row subtiles wholly past the expert's last row
    // skip their MFMAs (see the bf16 kernel).
    int nv = TM;
    if constexpr (MODE == RAGGED_M) {
      const int rows = m_end - (m0 + wm * WTM);
      nv = rows <= 0 ? 0 : (rows >= WTM ? TM : (rows + 31) / 32);
    }
    for (int it = 0; it < nk; ++it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // stage it&1 and this step's scales are in; stage (it+1)&1 is free
      lds_scales(it & 1, sa, sb);
      if (it + 1 < nk) {
        issue_scales(cur, (it + 1) * BK, (it + 1) & 1);
        issue(cur, (it + 1) * BK, (it + 1) & 1);
      }
      const char* sA = smem + (it & 1) * STAGE;
      const char* sB = sA + SA;
      // Slice 0's fragments are read here; slice 1's are read under slice 0's
      // MFMAs, A fragment i as soon as row i's MFMAs are issued, B fragment j
      // after the last row's MFMA j (the registers of one slice, renamed a
      // little by the compiler, is all that fits next to the accumulators).
      v8i32_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = frag_mx(sA, wm * WTM + i * 32, 0, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[j] = frag_mx(sB, wn * WTN + j * 32, 0, lane);
      static_for<BK / 64>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        constexpr bool last = kk + 1 == BK / 64;
        __builtin_amdgcn_sched_barrier(0);
        static_for<TM>([&](auto I) {
          constexpr int i = decltype(I)::value;
          const bool row_ok = i < nv;  // uniform: only an expert's tail tile skips
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if (row_ok)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], af[i], acc[i][j], 0, 0, 2 * kk,
                                                                           (int)sb[j], 2 * kk, (int)sa[i]);
            if constexpr (!last && i == TM - 1) {
              __builtin_amdgcn_sched_barrier(0);
              bfr[j] = frag_mx(sB, wn * WTN + j * 32, kk + 1, lane);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          if constexpr (!last) {
            __builtin_amdgcn_sched_barrier(0);
            af[i] = frag_mx(sA, wm * WTM + i * 32, kk + 1, lane);
            __builtin_amdgcn_sched_barrier(0);
          }
        });
      });
    }

    __syncthreads();  // every wave is done with the last K stage
    {
      const int tn = t + nbx;
      if (tn < t_end) {
        const Tile nxt = decode(tn);
        if (num_k(nxt) > 0) {
          issue(nxt, 0, 0);
          issue_scales(nxt, 0, 0);
        }
        cur = nxt;
      }
    }
    constexpr int WLDS = STAGE / NW;
    epilogue<WTM, WTN, CSEL, EPI, WLDS, MODE == RAGGED_M>(g, acc, smem + STAGE + wave * WLDS, lane, wm, wn, e, m0, m_end, n0);
  }
}

template <int BM, int BN, int MODE, int BSEL, int CSEL, int EPI>
static void run_mx(const char* name, const Args& a, const MxArgs& x, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return;
  ProfScope ps(name, s);
  ggemm_mx_kernel<BM, BN, 2, 4, MODE, BSEL, CSEL, EPI><<<grid_for(max_tiles), 512, 0, s>>>(a, x);
}

}  // namespace gg

using namespace gg;

// Up projection + SwiGLU: xq [R,d] x (W1q | W3q) [E,h,d]; any of G, U, H may
// be null (not stored).
template <int BM>
static void mx_up_bm(const char* name, const MxFwd& p, void* gq, void* u, void* hb, hipStream_t s) {
  const int E = p.E, R = p.R, d = p.d, h = p.h;
  const int mt_max = cdiv(R, BM) + E;
  Args a{};
  a.A = (const uint16_t*)p.xq; a.lda = d;
  a.B = (const uint16_t*)p.w1q; a.B2 = (const uint16_t*)p.w3q; a.ldb = d; a.b_es = (long)h * d;
  a.C = gq; a.C2 = u; a.C3 = hb; a.ldc = h;
  a.N = 2 * h; a.K = d; a.split = h;
  a.offsets = p.offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
  a.tiles_n = cdiv(2L * h, 256);
  MxArgs x{};
  x.sA = p.xs; x.sa_step = 4L * R; x.sA_bytes = (long)R * (d / 32);
  x.sB = p.w1s; x.sB2 = p.w3s; x.sb_step = 4L * E * h; x.sb_row_es = h; x.sB_bytes = (long)E * h * (d / 32);
  run_mx<BM, 256, RAGGED_M, BSEL_GLU, CSEL_NONE, EPI_SWIGLU_FWD>(name, a, x, mt_max * a.tiles_n, s);
}

hipError_t launch_ggemm_recompute_gu_mx(const MxFwd& p, hipStream_t s) {
  if (small_rows(p.E, p.R)) mx_up_bm<128>("ggemm_mx_recompute_gu", p, p.g, p.u, nullptr, s);
  else mx_up_bm<256>("ggemm_mx_recompute_gu", p, p.g, p.u, nullptr, s);
  return hipGetLastError();
}

template <int BM>
static hipError_t mx_fwd_bm(const MxFwd& p, unsigned parts, hipStream_t s) {
  const int E = p.E, R = p.R, d = p.d, h = p.h;
  const int mt_max = cdiv(R, BM) + E;
  if (parts & MOE_FWD_UP) {
    mx_up_bm<BM>("ggemm_mx_up_swiglu", p, p.g, p.u, p.hbuf, s);
    // H -> rowwise MX (down GEMM) and columnwise per expert (wgrad down)
    ProfScope ps("mx_quantize_h", s);
    const hipError_t err = launch_mx_quantize(p.hbuf, true, h, R, h, nullptr, 1, p.offsets, p.off128, E, 0,
                                              (R + 127 * E + 31) / 32, p.hq, p.hs, p.hqT, p.hsT, p.rcap, s);
    if (err != hipSuccess) return err;
  }
  if (parts & MOE_FWD_DOWN) {  // down projection: hq [R,h] x W2q [E,d,h]
    Args a{};
    a.A = (const uint16_t*)p.hq; a.lda = h;
    a.B = (const uint16_t*)p.w2q; a.ldb = h; a.b_es = (long)d * h;
    a.C = p.yp; a.ldc = d;
    a.N = d; a.K = h;
    a.offsets = p.offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(d, 256);
    MxArgs x{};
    x.sA = p.hs; x.sa_step = 4L * R; x.sA_bytes = (long)R * (h / 32);
    x.sB = p.w2s; x.sb_step = 4L * E * d; x.sb_row_es = d; x.sB_bytes = (long)E * d * (h / 32);
    run_mx<BM, 256, RAGGED_M, BSEL_NONE, CSEL_NONE, EPI_BF16>("ggemm_mx_down", a, x, mt_max * a.tiles_n, s);
  }
  return hipGetLastError();
}

// Ragged-M MX GEMMs use 256 x 256 tiles (128-row tiles when experts average
// fewer than 192 rows): an fp8 K step does half a bf16 step's MFMA time per
// byte loaded, so the per-step costs need the larger tile.  The weight
// gradients (K-tail masking, more registers) use 128 x 256.
hipError_t launch_ggemm_fwd_mx(const MxFwd& p, unsigned parts, hipStream_t s) {
  if (small_rows(p.E, p.R)) return mx_fwd_bm<128>(p, parts, s);
  return mx_fwd_bm<256>(p, parts, s);
}

template <int BM>
static hipError_t mx_dgrad_bm(const MxBwd& p, unsigned parts, hipStream_t s) {
  const int E = p.E, R = p.R, d = p.d, h = p.h;
  const int mt_max = cdiv(R, BM) + E;
  if (parts & MOE_BWD_DGRAD_DOWN) {  // dgrad down + SwiGLU backward: dyq [R,d] x W2 blocked along d ([E*h, d])
    Args a{};
    a.A = (const uint16_t*)p.dyq; a.lda = d;
    a.B = (const uint16_t*)p.w2tq; a.ldb = d; a.b_es = (long)h * d;
    a.C = p.dgu; a.ldc = 2L * h;
    a.G = (const uint16_t*)p.g; a.U = (const uint16_t*)p.u; a.ldgu = h;
    a.N = h; a.K = d; a.split = h;
    a.offsets = p.offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(h, 256);
    MxArgs x{};
    x.sA = p.dys; x.sa_step = 4L * R; x.sA_bytes = (long)R * (d / 32);
    x.sB = p.w2ts; x.sb_step = 4L * E * h; x.sb_row_es = h; x.sB_bytes = (long)h * E * d / 32;
    run_mx<BM, 256, RAGGED_M, BSEL_NONE, CSEL_NONE, EPI_SWIGLU_BWD>("ggemm_mx_dgrad_down_swiglu", a, x,
                                                                    mt_max * a.tiles_n, s);
  }
  if (parts & MOE_BWD_DGRAD_DOWN) {
    ProfScope ps("mx_quantize_dgu", s);
    const hipError_t err = launch_mx_quantize(p.dgu, true, 2L * h, R, 2 * h, nullptr, 1, p.offsets, p.off128, E, 0,
                                              (R + 127 * E + 31) / 32, p.dguq, p.dgus, p.dguqT, p.dgusT, p.rcap, s);
    if (err != hipSuccess) return err;
  }
  if (parts & MOE_BWD_DGRAD_UP) {  // dgrad up: dguq [R,2h] x (W1 | W3) blocked along h ([E*d, h] each)
    Args a{};
    a.A = (const uint16_t*)p.dguq; a.lda = 2L * h;
    a.B = (const uint16_t*)p.w1tq; a.B2 = (const uint16_t*)p.w3tq; a.ldb = h; a.b_es = (long)d * h;
    a.C = p.dxp; a.ldc = d;
    a.N = d; a.K = 2 * h; a.split = h;
    a.offsets = p.offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(d, 256);
    MxArgs x{};
    x.sA = p.dgus; x.sa_step = 4L * R; x.sA_bytes = (long)R * (2 * h / 32);
    x.sB = p.w1ts; x.sB2 = p.w3ts; x.sb_step = 4L * E * d; x.sb_row_es = d; x.sB_bytes = (long)d * E * h / 32;
    run_mx<BM, 256, RAGGED_M, BSEL_KSPLIT, CSEL_NONE, EPI_BF16>("ggemm_mx_dgrad_up", a, x, mt_max * a.tiles_n, s);
  }
  return hipGetLastError();
}

// parts (MOE_BWD_* mask): DGRAD_DOWN also quantises dYp before its GEMM
// (unless MX_DY_READY) and dG|dU after it; MX_QUANT_DY quantises dYp alone,
// so WGRAD_DOWN may start as soon as that is done, WGRAD_UP once DGRAD_DOWN is.
hipError_t launch_ggemm_bwd_mx(const MxBwd& p, unsigned parts, hipStream_t s) {
  const int E = p.E, R = p.R, d = p.d, h = p.h;
  if ((parts & MOE_BWD_MX_QUANT_DY) || ((parts & MOE_BWD_DGRAD_DOWN) && !(parts & MOE_BWD_MX_DY_READY))) {
    // dYp -> rowwise (dgrad down) and columnwise per expert (wgrad down)
    ProfScope ps("mx_quantize_dy", s);
    // from the stored dYp, or straight from dy (row r: topk_w[src[r]] * dy[src[r] / k])
    const bool from_dy = p.dyp == nullptr;
    const hipError_t err =
        launch_mx_quantize(from_dy ? p.dy : p.dyp, true, d, R, d, from_dy ? p.src : nullptr, from_dy ? p.k : 1,
                           p.offsets, p.off128, E, 0, (R + 127 * E + 31) / 32, p.dyq, p.dys, p.dyqT, p.dysT, p.rcap, s,
                           from_dy ? p.topk_w : nullptr);
    if (err != hipSuccess) return err;
  }
  if (parts & (MOE_BWD_DGRAD_DOWN | MOE_BWD_DGRAD_UP)) {
    const hipError_t err = small_rows(E, R) ? mx_dgrad_bm<128>(p, parts, s) : mx_dgrad_bm<256>(p, parts, s);
    if (err != hipSuccess) return err;
  }
  if (!(parts & (MOE_BWD_WGRAD_DOWN | MOE_BWD_WGRAD_UP))) return hipGetLastError();
  const long sc = p.rcap / 32;
  if (parts & MOE_BWD_WGRAD_DOWN) {  // wgrad down: dW2[e] = dYp_e^T H_e over the expert's padded segment
    Args a{};
    a.A = (const uint16_t*)p.dyqT;  // expert-major columnwise copies: rows of each segment's length
    a.B = (const uint16_t*)p.hqT;
    a.C = p.dw2; a.ldc = h; a.c_es = (long)d * h;
    a.M = d; a.N = h;
    a.offsets = p.off128; a.kstep = 128; a.E = E; a.R = R;
    a.tiles_m = cdiv(d, 256); a.tiles_n = cdiv(h, 256);
    MxArgs x{};
    x.sA = p.dysT; x.sa_step = 4L * d; x.sA_bytes = (long)d * sc;
    x.sB = p.hsT; x.sb_step = 4L * h; x.sB_bytes = (long)h * sc;
    run_mx<256, 256, RAGGED_K, BSEL_NONE, CSEL_NONE, EPI_BF16>("ggemm_mx_wgrad_down", a, x, E * a.tiles_m * a.tiles_n,
                                                               s);
  }
  if (parts & MOE_BWD_WGRAD_UP) {  // wgrad up: [dW1; dW3][e] = [dG | dU]_e^T Xp_e
    Args a{};
    a.A = (const uint16_t*)p.dguqT;  // expert-major columnwise copies: rows of each segment's length
    a.B = (const uint16_t*)p.xqT;
    a.C = p.dw1; a.C2 = p.dw3; a.ldc = d; a.c_es = (long)h * d;
    a.M = 2 * h; a.N = d; a.split = h;
    a.offsets = p.off128; a.kstep = 128; a.E = E; a.R = R;
    a.tiles_m = cdiv(2L * h, 256); a.tiles_n = cdiv(d, 256);
    MxArgs x{};
    x.sA = p.dgusT; x.sa_step = 8L * h; x.sA_bytes = (long)2 * h * sc;
    x.sB = p.xsT; x.sb_step = 4L * d; x.sB_bytes = (long)d * sc;
    run_mx<256, 256, RAGGED_K, BSEL_NONE, CSEL_MSPLIT, EPI_BF16>("ggemm_mx_wgrad_up", a, x,
                                                                 E * a.tiles_m * a.tiles_n, s);
  }
  return hipGetLastError();
}

}  // namespace trg
