// Grouped bf16 GEMMs of the expert SwiGLU FFNs on gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  One launch per GEMM kind
// covers every expert: the many small per-expert products are batched into a
// single grouped GEMM call (Olmo-core 3 overview, "Routing and compute
// optimisation").
//
// CDNA4 design:
//  * Persistent, XCD-aware scheduler.  The grid is one workgroup per compute
//    unit.  The logical tile list (derived on the device from the expert
//    offsets, so the host never waits for routing) is cut into eight
//    contiguous ranges, one per XCD (workgroup i runs on XCD i % 8), and the
//    workgroups of an XCD walk their range together.  At any moment an XCD's
//    32 CUs work on neighbouring tiles that share A rows and B columns, so the
//    XCD's own L2 serves the re-reads.
//  * 512 threads = 8 waves in a 2 x 4 grid (two waves per SIMD, so one hides
//    the other's LDS latency); block tile BM x 256, K step 64.
//  * Operands move HBM -> LDS with buffer_load_dwordx4 ... lds (no register
//    staging).  A buffer resource bounds every operand: reads past the end of
//    an operand return zero, which also zero-fills the ragged K tail of the
//    weight-gradient GEMMs.
//  * LDS holds two stages.  An operand stored K-contiguous lands as
//    [rows][64] bf16 (128-byte rows) with 16-byte chunks XOR-swizzled by the
//    row pair (conflict-free for 64 banks); fragments are read with
//    ds_read_b128.  An operand stored
//    MN-contiguous (dgrad weights, both wgrad operands) lands as [64][BMN]
//    bf16 with chunks XOR-swizzled by the k row and is read with the gfx950
//    transpose read ds_read_b64_tr_b16, which hands each lane 4 k-consecutive
//    values of its column.  Either way every MFMA sees the same fragments.
//  * Fragments are double-buffered in registers: the reads for the next
//    16-wide k slice are in flight while the current slice's MFMAs issue; the
//    next K tile's HBM loads are in flight during the whole current tile.
//  * The MFMA is issued as (B fragment, A fragment): each lane then owns 4
//    consecutive output columns of one row.
//  * Epilogues (bf16 store, SwiGLU forward G/U/H, SwiGLU backward dG/dU from
//    dH, G, U) stage each wave's 32-row slabs in LDS and move whole row
//    segments with 16-byte loads and stores.
#include "ggemm_impl.h"

namespace trg {
namespace gg {

template <int BM, int BN, int WM, int WN, bool AKC, bool BKC, int MODE, int BSEL, int CSEL, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void ggemm_kernel(Args g) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int SA = BM * 128, SB = BN * 128;  // bytes per stage and operand
  constexpr int STAGE = SA + SB;
  static_assert(BM % 128 == 0 && BN % 128 == 0, "tile");
  static_assert(BSEL != BSEL_GLU || (TN % 2 == 0), "GLU pairs subtiles");
  static_assert(MODE == RAGGED_M || (!AKC && !BKC), "weight gradients read both operands MN-contiguous");
  // Light tail tiles (RmSched: at most 128 valid rows, 256-row tiles) run a
  // three-stage pipeline: they need only half the A stage, so three stages of
  // LSTAGE bytes fit, and two steps of prefetch hide the load latency their
  // few MFMAs cannot.  LPW: stage loads per wave per light step.
  constexpr bool LIGHT3 = MODE == RAGGED_M && BM == 256 && AKC;
  constexpr int LSA = 128 * 128, LSTAGE = LSA + SB;
  constexpr int LPW = (128 / 8) / NW + (BKC ? (BN / 8) / NW : (64 * BN * 2 / 1024) / NW);
  static_assert(!LIGHT3 || LPW == 6, "the light pipeline's vmcnt immediate");
  // (the weight gradients take the same 144 KB, for a larger epilogue area)
  constexpr int SMEM = LIGHT3 && 3 * LSTAGE > 2 * STAGE ? 3 * LSTAGE
                       : (MODE == RAGGED_K && BM == 256 ? 3 * (128 * 128 + SB) : 2 * STAGE);
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

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

  // Per-tile geometry and operand resources.
  struct Tile {
    int e, m0, m_end, n0, k0, k_end;
    bool light;  // a light tail (three-stage pipeline)
    __amdgpu_buffer_rsrc_t rsA, rsB, rsB2;
  };
  const long a_ldb = g.lda * 2, b_ldb = g.ldb * 2;
  auto decode = [&](int t) {
    Tile c;
    c.light = false;
    if constexpr (MODE == RAGGED_M) {
      int nt;
      rm_tile<BM>(pre, g.offsets, g.E, g.tiles_n, rms, t, c.e, c.m0, c.m_end, nt);
      c.light = LIGHT3 && t >= rms.nf;
      c.n0 = nt * BN;
      c.k0 = 0;
      c.k_end = g.K;
      // A: routed rows from m0 on, K-contiguous
      c.rsA = make_rsrc(g.A + (long)c.m0 * g.lda, (long)(g.R - c.m0) * a_ldb);
      if constexpr (BSEL == BSEL_GLU) {
        const long hh0 = c.n0 / 2;
        c.rsB = make_rsrc(g.B + (long)c.e * g.b_es + hh0 * g.ldb, (g.split - hh0) * b_ldb);
        c.rsB2 = make_rsrc(g.B2 + (long)c.e * g.b_es + hh0 * g.ldb, (g.split - hh0) * b_ldb);
      } else if constexpr (BKC) {
        c.rsB = make_rsrc(g.B + (long)c.e * g.b_es + (long)c.n0 * g.ldb, (long)(g.N - c.n0) * b_ldb);
        c.rsB2 = c.rsB;
      } else {
        // MN-contiguous B: X[k][n] inside the expert's block of b_es elements
        c.rsB = make_rsrc(g.B + (long)c.e * g.b_es + c.n0, (g.b_es - c.n0) * 2);
        c.rsB2 = (BSEL == BSEL_KSPLIT) ? make_rsrc(g.B2 + (long)c.e * g.b_es + c.n0, (g.b_es - c.n0) * 2) : c.rsB;
      }
    } else {
      const int per_e = g.tiles_m * g.tiles_n;
      c.e = t / per_e;
      const int r = t - c.e * per_e;
      const int mt = r / g.tiles_n, nt = r - mt * g.tiles_n;
      c.m0 = mt * BM;
      c.m_end = g.M;
      c.n0 = nt * BN;
      c.k0 = g.offsets[c.e];
      c.k_end = g.offsets[c.e + 1];
      // weight gradients: K = the expert's rows; rows past k_end read as zero
      const long nrows = c.k_end - c.k0;
      c.rsA = make_rsrc(g.A + (long)c.k0 * g.lda + c.m0, nrows * a_ldb - (long)c.m0 * 2);
      c.rsB = make_rsrc(g.B + (long)c.k0 * g.ldb + c.n0, nrows * b_ldb - (long)c.n0 * 2);
      c.rsB2 = c.rsB;
    }
    return c;
  };
  auto num_k = [&](const Tile& c) { return c.k_end > c.k0 ? (c.k_end - c.k0 + BK - 1) / BK : 0; };

  int a_lane[2], b_lane[2];
  if constexpr (AKC) {
    a_lane[0] = kc_lane_off(lane, 0, (int)a_ldb);
    a_lane[1] = kc_lane_off(lane, 1, (int)a_ldb);
  } else {
    a_lane[0] = mnc_lane_off<BM>(lane, 0, (int)a_ldb);
    a_lane[1] = mnc_lane_off<BM>(lane, 1, (int)a_ldb);
  }
  if constexpr (BKC) {
    b_lane[0] = kc_lane_off(lane, 0, (int)b_ldb);
    b_lane[1] = kc_lane_off(lane, 1, (int)b_ldb);
  } else {
    b_lane[0] = mnc_lane_off<BN>(lane, 0, (int)b_ldb);
    b_lane[1] = mnc_lane_off<BN>(lane, 1, (int)b_ldb);
  }
  auto issue = [&](const Tile& c, int kt, int stage) {  // kt: K offset relative to c.k0
    char* sA = smem + stage * STAGE;
    char* sB = sA + SA;
    if (LIGHT3 && c.light) {  // rows 0..127 of A and all of B, stage stride LSTAGE
      sA = smem + stage * LSTAGE;
      sB = sA + LSA;
      load_kc<128, NW>(sA, wave, a_lane, kt * 2, (int)a_ldb, [&](int r8, int& r0) {
        r0 = r8;
        return c.rsA;
      });
    } else if constexpr (AKC) {
      load_kc<BM, NW>(sA, wave, a_lane, kt * 2, (int)a_ldb, [&](int r8, int& r0) {
        r0 = r8;
        return c.rsA;
      });
    } else {
      load_mnc<BM, NW>(sA, wave, a_lane, c.rsA, kt, (int)a_ldb);
    }
    if constexpr (BKC) {
      if constexpr (BSEL == BSEL_GLU) {
        load_kc<BN, NW>(sB, wave, b_lane, kt * 2, (int)b_ldb, [&](int r8, int& r0) {
          // LDS rows of wave column `part`: first WTN/2 from W1, next WTN/2
          // from W3, both for the same hidden units
          const int p = r8 % WTN;
          r0 = (r8 / WTN) * (WTN / 2) + (p % (WTN / 2));
          return (p >= WTN / 2) ? c.rsB2 : c.rsB;
        });
      } else {
        load_kc<BN, NW>(sB, wave, b_lane, kt * 2, (int)b_ldb, [&](int r8, int& r0) {
          r0 = r8;
          return c.rsB;
        });
      }
    } else {
      if constexpr (BSEL == BSEL_KSPLIT) {
        if (kt >= g.split) load_mnc<BN, NW>(sB, wave, b_lane, c.rsB2, kt - g.split, (int)b_ldb);
        else load_mnc<BN, NW>(sB, wave, b_lane, c.rsB, kt, (int)b_ldb);
      } else {
        load_mnc<BN, NW>(sB, wave, b_lane, c.rsB, kt, (int)b_ldb);
      }
    }
  };

  // The first K step of a tile is loaded into stage 0 before the previous
  // tile's epilogue runs (the epilogue stages through stage 1), so a tile
  // boundary costs no full memory round trip.
  int t = t_begin + lb;
  Tile cur;
  if (t < t_end) {
    cur = decode(t);
    if (num_k(cur) > 0) issue(cur, 0, 0);
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
    // Ragged M: the wave's 32-row subtiles that lie wholly past the expert's
    // last row hold no output, so their MFMAs are skipped (an expert's last
    // row tile is often nearly empty: 8 rows of 256).  On a SIMD the two
    // waves' MFMAs share one matrix core, so the tail tile's time shrinks with
    // them.
    int nv = TM;
    if constexpr (MODE == RAGGED_M) {
      const int rows = m_end - (m0 + wm * WTM);
      nv = rows <= 0 ? 0 : (rows >= WTM ? TM : (rows + 31) / 32);
    }
    const bool light = LIGHT3 && cur.light;
    for (int it = 0; it < nk; ++it) {
      // light: step it+1's LPW loads per wave may stay in flight
      if (light && it > 0 && it + 1 < nk) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // this step's stage is complete; the stage read last step is free
      const char* sA;
      const char* sB;
      if (light) {
        if (it == 0) {
          if (nk > 1) issue(cur, BK, 1);
          if (nk > 2) issue(cur, 2 * BK, 2);
        } else if (it + 2 < nk) {
          issue(cur, (it + 2) * BK, (it + 2) % 3);
        }
        sA = smem + (it % 3) * LSTAGE;
        sB = sA + LSA;
      } else {
        if (it + 1 < nk) issue(cur, (it + 1) * BK, (it + 1) & 1);
        sA = smem + (it & 1) * STAGE;
        sB = sA + SA;
      }
      bf16x8_t af[2][TM], bfr[2][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = frag<BM, AKC>(sA, wm * WTM + i * 32, 0, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[0][j] = frag<BN, BKC>(sB, wn * WTN + j * 32, 0, lane);
      // Scheduling fences keep the next slice's reads ahead of this slice's
      // MFMAs (two fragment sets stay live instead of one re-used per MFMA).
      __builtin_amdgcn_sched_barrier(0);
      // Ragged K: an expert's last step may hold fewer than BK rows; its rows
      // past k_end read as zero, so when it holds at most half a step the
      // upper half's slices add nothing and are skipped (short segments: 85
      // rows per expert take two steps, the second a third full).  One
      // uniform test per step: per-slice tests slowed the full steps.
      const bool upper = MODE != RAGGED_K || cur.k_end - cur.k0 - it * BK > BK / 2;
      static_for<BK / 16>([&](auto KK) {
        constexpr int kk = decltype(KK)::value;
        constexpr int fb = kk & 1;  // fragment set of this slice
        if (kk >= BK / 32 && !upper) return;
        if constexpr (kk + 1 < BK / 16) {
          if (kk + 1 < BK / 32 || upper) {
#pragma unroll
            for (int i = 0; i < TM; ++i) af[fb ^ 1][i] = frag<BM, AKC>(sA, wm * WTM + i * 32, kk + 1, lane);
#pragma unroll
            for (int j = 0; j < TN; ++j) bfr[fb ^ 1][j] = frag<BN, BKC>(sB, wn * WTN + j * 32, kk + 1, lane);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if (i < nv)  // uniform: only an expert's tail tile skips
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[fb][j], af[fb][i], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      });
    }

    // ---------------- epilogue ----------------
    // Staged through stage 1 while the next tile's first K step streams into
    // stage 0.
    __syncthreads();  // every wave is done with the last K stage
    {
      const int tn = t + nbx;
      if (tn < t_end) {
        const Tile nxt = decode(tn);
        if (num_k(nxt) > 0) issue(nxt, 0, 0);
        cur = nxt;
      }
    }
    // LDS bytes per wave: inside stage 1; for the weight gradients everything
    // past stage 0 (which may already hold the next tile's first step), room
    // for 64-row slabs (ragged M measured no better with them)
    constexpr int WLDS = MODE == RAGGED_K ? (SMEM - STAGE) / NW / 256 * 256 : STAGE / NW;
    epilogue<WTM, WTN, CSEL, EPI, WLDS, MODE == RAGGED_M>(g, acc, smem + STAGE + wave * WLDS, lane, wm, wn, e, m0, m_end, n0);
  }
}

// 8 waves (two per SIMD) per 256-wide tile: while one wave of a SIMD waits
// on LDS the other issues MFMAs.
template <int BM, int BN, bool AKC, bool BKC, int MODE, int BSEL, int CSEL, int EPI>
static void run(const char* name, const Args& a, int max_tiles, hipStream_t s) {
  if (max_tiles <= 0) return;
  ProfScope ps(name, s);
  constexpr int WM = 2, WN = (BN >= 256 ? 4 : 2);
  ggemm_kernel<BM, BN, WM, WN, AKC, BKC, MODE, BSEL, CSEL, EPI><<<grid_for(max_tiles), 64 * WM * WN, 0, s>>>(a);
}

}  // namespace gg

// The grouped GEMMs need no scratch: every workgroup derives its schedule's
// prefixes from the expert offsets in its prologue.
size_t ggemm_ws_bytes(int E, int R, int d, int h) {
  (void)E; (void)R; (void)d; (void)h;
  return 0;
}

using namespace gg;

// Up projection with the SwiGLU epilogue (N covers W1 and W3 rows); any of
// G, U, H may be null (not stored).
template <int BM>
static void up_bm(const char* name, const void* xp, const void* w1, const void* w3, const int* offsets, int E, int R,
                  int d, int h, void* gq, void* u, void* hb, hipStream_t s) {
  const int mt_max = cdiv(R, BM) + E;
  Args a{};
  a.A = (const uint16_t*)xp; a.lda = d;
  a.B = (const uint16_t*)w1; a.B2 = (const uint16_t*)w3; a.ldb = d; a.b_es = (long)h * d;
  a.C = gq; a.C2 = u; a.C3 = hb; a.ldc = h;
  a.N = 2 * h; a.K = d; a.split = h;
  a.offsets = offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
  a.tiles_n = cdiv(2L * h, 256);
  run<BM, 256, true, true, RAGGED_M, BSEL_GLU, CSEL_NONE, EPI_SWIGLU_FWD>(name, a, mt_max * a.tiles_n, s);
}

template <int BM>
static void fwd_bm(const void* xp, const void* w1, const void* w3, const void* w2, const int* offsets, int E, int R,
                   int d, int h, void* gq, void* u, void* hb, void* yp, hipStream_t s) {
  const int mt_max = cdiv(R, BM) + E;
  up_bm<BM>("ggemm_up_swiglu", xp, w1, w3, offsets, E, R, d, h, gq, u, hb, s);
  {  // down projection
    Args a{};
    a.A = (const uint16_t*)hb; a.lda = h;
    a.B = (const uint16_t*)w2; a.ldb = h; a.b_es = (long)d * h;
    a.C = yp; a.ldc = d;
    a.N = d; a.K = h;
    a.offsets = offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(d, 256);
    run<BM, 256, true, true, RAGGED_M, BSEL_NONE, CSEL_NONE, EPI_BF16>("ggemm_down", a, mt_max * a.tiles_n, s);
  }
}

hipError_t launch_ggemm_fwd(const void* xp, const void* w1, const void* w3, const void* w2, const int* offsets,
                            int E, int R, int d, int h, bool bf16, void* g, void* u, void* hb, void* yp, void* ws,
                            hipStream_t s) {
  if (!bf16)
    return launch_ggemm_fwd_f32((const float*)xp, (const float*)w1, (const float*)w3, (const float*)w2, offsets, E,
                                R, d, h, (float*)g, (float*)u, (float*)hb, (float*)yp, s);
  (void)ws;
  if (small_rows(E, R))
    fwd_bm<128>(xp, w1, w3, w2, offsets, E, R, d, h, g, u, hb, yp, s);
  else
    fwd_bm<256>(xp, w1, w3, w2, offsets, E, R, d, h, g, u, hb, yp, s);
  return hipGetLastError();
}

hipError_t launch_ggemm_recompute_gu(const void* xp, const void* w1, const void* w3, const int* offsets, int E, int R,
                                     int d, int h, void* g, void* u, void* ws, hipStream_t s) {
  (void)ws;
  if (small_rows(E, R))
    up_bm<128>("ggemm_recompute_gu", xp, w1, w3, offsets, E, R, d, h, g, u, nullptr, s);
  else
    up_bm<256>("ggemm_recompute_gu", xp, w1, w3, offsets, E, R, d, h, g, u, nullptr, s);
  return hipGetLastError();
}

template <int BM>
static void dgrad_bm(const void* dyp, const void* g, const void* u, const void* w1, const void* w3, const void* w2,
                     const int* offsets, int E, int R, int d, int h, void* dgu, void* dxp, unsigned parts,
                     hipStream_t s) {
  const int mt_max = cdiv(R, BM) + E;
  if (parts & MOE_BWD_DGRAD_DOWN) {  // dgrad down + SwiGLU backward: dH = dYp W2[e] -> dG, dU
    Args a{};
    a.A = (const uint16_t*)dyp; a.lda = d;
    a.B = (const uint16_t*)w2; a.ldb = h; a.b_es = (long)d * h;
    a.C = dgu; a.ldc = 2L * h;
    a.G = (const uint16_t*)g; a.U = (const uint16_t*)u; a.ldgu = h;
    a.N = h; a.K = d; a.split = h;
    a.offsets = offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(h, 256);
    run<BM, 256, true, false, RAGGED_M, BSEL_NONE, CSEL_NONE, EPI_SWIGLU_BWD>("ggemm_dgrad_down_swiglu", a,
                                                                              mt_max * a.tiles_n, s);
  }
  if (parts & MOE_BWD_DGRAD_UP) {  // dgrad up: dXp = [dG | dU] [W1; W3]
    Args a{};
    a.A = (const uint16_t*)dgu; a.lda = 2L * h;
    a.B = (const uint16_t*)w1; a.B2 = (const uint16_t*)w3; a.ldb = d; a.b_es = (long)h * d;
    a.C = dxp; a.ldc = d;
    a.N = d; a.K = 2 * h; a.split = h;
    a.offsets = offsets; a.split_tails = split_tails(E, R); a.E = E; a.R = R;
    a.tiles_n = cdiv(d, 256);
    run<BM, 256, true, false, RAGGED_M, BSEL_KSPLIT, CSEL_NONE, EPI_BF16>("ggemm_dgrad_up", a, mt_max * a.tiles_n, s);
  }
}

hipError_t launch_ggemm_bwd(const void* dyp, const void* xp, const void* g, const void* u, const void* hb,
                            const void* w1, const void* w3, const void* w2, const int* offsets, int E, int R, int d,
                            int h, bool bf16, void* dgu, void* dxp, void* dw1, void* dw3, void* dw2, void* ws,
                            unsigned parts, hipStream_t s) {
  if (!bf16)
    return launch_ggemm_bwd_f32((const float*)dyp, (const float*)xp, (const float*)g, (const float*)u,
                                (const float*)hb, (const float*)w1, (const float*)w3, (const float*)w2, offsets, E,
                                R, d, h, (float*)dgu, (float*)dxp, (float*)dw1, (float*)dw3, (float*)dw2, s);
  (void)ws;
  if (parts & (MOE_BWD_DGRAD_DOWN | MOE_BWD_DGRAD_UP)) {
    if (small_rows(E, R))
      dgrad_bm<128>(dyp, g, u, w1, w3, w2, offsets, E, R, d, h, dgu, dxp, parts, s);
    else
      dgrad_bm<256>(dyp, g, u, w1, w3, w2, offsets, E, R, d, h, dgu, dxp, parts, s);
  }
  if (parts & MOE_BWD_WGRAD_DOWN) {  // wgrad down: dW2[e] = dYp_e^T H_e  (M = d, N = h, K = the expert's rows)
    Args a{};
    a.A = (const uint16_t*)dyp; a.lda = d;
    a.B = (const uint16_t*)hb; a.ldb = h;
    a.C = dw2; a.ldc = h; a.c_es = (long)d * h;
    a.M = d; a.N = h;
    a.offsets = offsets; a.kstep = BK; a.E = E; a.R = R;
    a.tiles_m = cdiv(d, 256); a.tiles_n = cdiv(h, 256);
    run<256, 256, false, false, RAGGED_K, BSEL_NONE, CSEL_NONE, EPI_BF16>("ggemm_wgrad_down", a,
                                                                          E * a.tiles_m * a.tiles_n, s);
  }
  if (parts & MOE_BWD_WGRAD_UP) {  // wgrad up: [dW1; dW3][e] = [dG | dU]_e^T Xp_e  (M = 2h, N = d)
    Args a{};
    a.A = (const uint16_t*)dgu; a.lda = 2L * h;
    a.B = (const uint16_t*)xp; a.ldb = d;
    a.C = dw1; a.C2 = dw3; a.ldc = d; a.c_es = (long)h * d;
    a.M = 2 * h; a.N = d; a.split = h;
    a.offsets = offsets; a.kstep = BK; a.E = E; a.R = R;
    a.tiles_m = cdiv(2L * h, 256); a.tiles_n = cdiv(d, 256);
    run<256, 256, false, false, RAGGED_K, BSEL_NONE, CSEL_MSPLIT, EPI_BF16>("ggemm_wgrad_up", a,
                                                                            E * a.tiles_m * a.tiles_n, s);
  }
  return hipGetLastError();
}

}  // namespace trg
