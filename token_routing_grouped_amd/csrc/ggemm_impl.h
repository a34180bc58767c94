// Shared pieces of the grouped GEMMs (bf16 and MXFP8): operand descriptors,
// HBM->LDS loaders, fragment reads, the staged epilogue, and the persistent
// scheduler's helpers.  See ggemm.hip for the design.
#pragma once

#include "common.h"
#include "kernels.h"
#include "prof.h"

namespace trg {
namespace gg {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

enum Mode { RAGGED_M = 1, RAGGED_K = 2 };
enum BSel { BSEL_NONE = 0, BSEL_GLU = 1, BSEL_KSPLIT = 2 };
enum CSel { CSEL_NONE = 0, CSEL_MSPLIT = 1 };
enum Epi { EPI_BF16 = 0, EPI_SWIGLU_FWD = 2, EPI_SWIGLU_BWD = 3 };

constexpr int BK = 64;
constexpr int kLdsBytes = 163840;  // gfx950 LDS per workgroup

// Per-wave epilogue staging area next to the two operand stages: what is
// left of the LDS, at most 16 KiB, in whole KiB.
constexpr int lds_epilogue_bytes(int stage, int nw) {
  const int r = (kLdsBytes - 2 * stage) / nw;
  return (r > 16384 ? 16384 : r) / 1024 * 1024;
}
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

struct Args {
  // Operand X[mn][k]: K-contiguous -> X[mn*ld + k]; MN-contiguous -> X[k*ld + mn]
  const uint16_t* A;
  long lda;
  const uint16_t* B;
  const uint16_t* B2;  // BSEL_GLU: W3 next to W1;  BSEL_KSPLIT: second K half
  long ldb, b_es;      // b_es: per-expert element stride of B
  void* C;
  void* C2;  // CSEL_MSPLIT: rows >= split;  SWIGLU_FWD: U
  void* C3;  // SWIGLU_FWD: H
  long ldc, c_es;
  const uint16_t* G;  // SWIGLU_BWD inputs
  const uint16_t* U;
  long ldgu;
  int M, N, K;  // RAGGED_K: M x N output per expert;  RAGGED_M: N, K
  int split;    // GLU: h;  KSPLIT: first K half;  MSPLIT: first M half
  const int* offsets;
  int split_tails;  // RAGGED_M, 256-row tiles: light tails scheduled apart (see RmSched)
  int kstep;        // RAGGED_K: K values per step (the work prefix's unit)
  int E, R;
  int tiles_m, tiles_n;
};

// Staged epilogue rows go out with store_nt16 when NT (the ragged-M GEMMs:
// 2-6% faster on dgrad-down and down at the small shape; the weight gradients
// measured no better, or slower, with it).  The SwiGLU-forward epilogue keeps
// the default policy: its staged stores gained nothing overall with the hint
// (the down projection that reads H next slowed by more), and its direct
// 8-byte stores rely on L2 merging partial lines (twice as slow with it).
TRG_DEV void store_row16(bool nt, void* p, uint4 v) {
  if (nt) store_nt16(p, v);
  else *(uint4*)p = v;
}

TRG_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const unsigned n = bytes <= 0 ? 0u : (bytes >= 0xFFFFFFFFL ? 0xFFFFFFFFu : (unsigned)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcFlags);
}

// 16 bytes per lane from the buffer at byte voff into LDS at lds (wave-uniform
// base; lane i lands at lds + 16 i).  Issued as inline assembly so that the
// compiler's wait insertion does not see an LDS write: it would otherwise
// hold every LDS read it cannot prove disjoint (the transpose reads) until all
// in-flight stage loads are done.  The kernels order the stages themselves
// (vmcnt(0) + barrier before a stage is read).  M0 is saved and restored.
TRG_DEV void lds_load16(__amdgpu_buffer_rsrc_t rs, char* lds, int voff) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)(lds_void_t*)lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voff), "s"(rs)
      : "memory");
}

// 4 bytes per lane from the buffer at byte voff (4-byte aligned) into LDS at
// lds + 4 * lane, the same way.
TRG_DEV void lds_load4(__amdgpu_buffer_rsrc_t rs, char* lds, int voff) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)(lds_void_t*)lds);
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(voff), "s"(rs)
      : "memory");
}

// K-contiguous operand: BMN rows of 64 bf16 (128-byte rows).  gfx950's LDS
// has 64 banks and serves ds_read_b128 16 lanes at a time; a fragment read
// hands those 16 lanes 16 consecutive rows at one logical chunk, so the 16-byte
// chunk slot of row r is swizzled as p = c ^ ((r >> 1) & 7): two rows share a
// 256-byte bank window and the XOR spreads the 8 row pairs over all 8 chunk
// positions.  Wave w fills 1 KiB blocks [w*P, (w+1)*P), P = BMN/8 / waves;
// block b holds rows 8b..8b+7.  The lane's part of the byte offset depends only on the
// block's parity.  row8(b) -> (resource, first row of block b inside that
// resource).
template <int BMN, int NW, class Row8>
TRG_DEV void load_kc(char* dst, int wave, const int (&lane_off)[2], int kbyte, int ld_bytes, Row8 row8) {
  constexpr int PER = BMN / 8 / NW;  // 1 KiB blocks per wave
  static_assert(PER >= 1 && (BMN / 8) % NW == 0, "blocks per wave");
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave * PER + i;
    int r0;
    const __amdgpu_buffer_rsrc_t rs = row8(blk * 8, r0);
    lds_load16(rs, dst + blk * 1024, lane_off[blk & 1] + r0 * ld_bytes + kbyte);
  }
}

TRG_DEV int kc_lane_off(int lane, int parity, int ld_bytes) {
  const int l8 = lane >> 3;  // row inside the block
  const int sw = (parity << 2) | (l8 >> 1);
  return l8 * ld_bytes + (((lane & 7) ^ sw) << 4);
}

// MN-contiguous operand: 64 k rows of BMN bf16 (row = BMN*2 bytes).  LDS
// chunk slot p of k row kr receives global chunk p ^ ((kr & 3) << 2).  A 1 KiB
// block covers 1024/ROWB k rows; the lane's offset inside a block depends only
// on the block's parity (BMN = 256) or not at all (BMN = 128).
template <int BMN>
TRG_DEV int mnc_lane_off(int lane, int parity, int ld_bytes) {
  constexpr int ROWB = BMN * 2;
  const int off = parity * 1024 + lane * 16;
  const int kr = off / ROWB;
  const int c = ((off % ROWB) >> 4) ^ ((kr & 3) << 2);
  return (kr - parity * (1024 / ROWB)) * ld_bytes + c * 16;
}

template <int BMN, int NW>
TRG_DEV void load_mnc(char* dst, int wave, const int (&lane_off)[2], __amdgpu_buffer_rsrc_t rs, int krow0,
                      int ld_bytes) {
  constexpr int ROWB = BMN * 2;
  constexpr int NBLK = 64 * ROWB / 1024;
  constexpr int RPB = 1024 / ROWB;  // k rows per block
  constexpr int PER = NBLK / NW;
  static_assert(PER >= 1 && NBLK % NW == 0, "blocks per wave");
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int blk = wave * PER + i;
    lds_load16(rs, dst + blk * 1024, lane_off[blk & 1] + (krow0 + blk * RPB) * ld_bytes);
  }
}

// Fragment of 8 k-consecutive values for MFMA lane `lane` (its row / column
// is base + (lane & 31), its k range kk*16 + (lane >> 5)*8 + [0, 8)).
TRG_DEV bf16x8_t frag_kc(const char* s, int base, int kk, int lane) {
  const int row = base + (lane & 31);
  const int c = kk * 2 + (lane >> 5);
  return *(const bf16x8_t*)(s + row * 128 + ((c ^ ((row >> 1) & 7)) << 4));
}

template <int BMN>
TRG_DEV bf16x8_t frag_mnc(const char* s, int base, int kk, int lane) {
  constexpr int ROWB = BMN * 2;
  // Transpose read: the 16 lanes of a group load a 4 (k) x 16 (column) block,
  // lane s of the group the 4 values of row s/4 starting at column 4*(s%4);
  // after the read lane s holds column s's 4 values, k ascending.
  const int g = lane >> 4, s16 = lane & 15;
  const int col = base + (g & 1) * 16 + (s16 & 3) * 4;
  const int kr = kk * 16 + (g >> 1) * 8 + (s16 >> 2);
  const int sw = (kr & 3) << 2;
  const int cb = ((col >> 3) ^ sw) << 4;
  const int within = (col & 7) * 2;
  const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s + kr * ROWB + cb + within));
  const bf16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(s + (kr + 4) * ROWB + cb + within));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int BMN, bool KC>
TRG_DEV bf16x8_t frag(const char* s, int base, int kk, int lane) {
  if constexpr (KC) return frag_kc(s, base, kk, lane);
  else return frag_mnc<BMN>(s, base, kk, lane);
}

// Epilogue of one output tile.  Each wave stages slabs of its tile (8 to 64
// rows, as many as its private LDS area `wl` of WLDS bytes holds) and writes
// whole row segments with 16-byte stores; the accumulator layout alone would scatter 8-byte pieces over
// 32 rows per store instruction.  Accumulator lane (lrow, lgrp) owns row lrow
// and, per 32-column subtile j and group q, columns j*32 + q*8 + lgrp + {0..3}.
// EPI_BF16 writes C (rows >= split go to C2 under CSEL_MSPLIT, plus e*c_es);
// EPI_SWIGLU_FWD treats the first TN/2 subtiles as G and the rest as U of the
// same hidden units and writes G, U and H = silu(G) * U (staged per 32-row
// subtile where the three fit, else directly from the accumulators, see
// below); EPI_SWIGLU_BWD treats the tile as dH and writes
// dG | dU from the stored G and U.
template <int WTN, int EPI, int WLDS>
constexpr int epilogue_slab_rows() {  // plain bf16: two or one whole 32-row subtiles when they fit; else 16 rows, else 8
  if (EPI == EPI_BF16 && 64 * (WTN * 2 + 16) <= WLDS) return 64;
  if (EPI == EPI_BF16 && 32 * (WTN * 2 + 16) <= WLDS) return 32;
  return (EPI == EPI_SWIGLU_BWD ? 2 * 16 * (WTN * 2 + 16) : 16 * (WTN * 2 + 16)) <= WLDS ? 16 : 8;
}

template <int WTM, int WTN, int CSEL, int EPI, int WLDS, bool NT>
TRG_DEV void epilogue(const Args& g, f32x16_t (&acc)[WTM / 32][WTN / 32], char* wl, int lane, int wm, int wn, int e,
                      int m0, int m_end, int n0) {
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int P = WTN * 2 + 16;       // staged row pitch (16-byte aligned)
  constexpr int SR = epilogue_slab_rows<WTN, EPI, WLDS>();  // slab rows: a part of an accumulator subtile
  constexpr int NPART = SR >= 32 ? 1 : 32 / SR;
  static_assert(EPI != EPI_SWIGLU_BWD || 2 * SR * P <= WLDS, "epilogue LDS");
  if constexpr (EPI == EPI_SWIGLU_FWD && 3 * 32 * (WTN + 16) <= WLDS) {
    // G, U and H of one 32-row subtile staged in LDS (the wave's WTN/2 hidden
    // units, row pitch PF), then written as 16-byte row pieces
    constexpr int PF = WTN + 16;
    constexpr int CPR = WTN / 16;  // 16-byte chunks per staged row
    const int lrow = lane & 31, lgrp = (lane >> 5) * 4;
    const int hh0 = n0 / 2 + wn * (WTN / 2);
    char* sG = wl;
    char* sU = wl + 32 * PF;
    char* sH = wl + 64 * PF;
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int ms = m0 + wm * WTM + i * 32;
      if (ms < m_end) {
        static_for<TN / 2>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            float gv[4], uv[4], hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              gv[r] = acc[i][j][q * 4 + r];
              uv[r] = acc[i][j + TN / 2][q * 4 + r];
              hv[r] = silu_f(gv[r]) * uv[r];
            }
            const int off = lrow * PF + (j * 32 + q * 8 + lgrp) * 2;
            *(uint2*)(sG + off) = make_uint2(pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3]));
            *(uint2*)(sU + off) = make_uint2(pack_bf2(uv[0], uv[1]), pack_bf2(uv[2], uv[3]));
            *(uint2*)(sH + off) = make_uint2(pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3]));
          });
        });
        __builtin_amdgcn_wave_barrier();
        // any of G, U, H may be absent: a memory-lean forward stores H only,
        // the backward's recompute G and U only (uniform branches)
        for (int c = lane; c < 32 * CPR; c += 64) {
          const int row = c / CPR, cc = c - row * CPR;
          const int m = ms + row, col = hh0 + cc * 8;
          if (m < m_end && col < g.split) {
            const long off = (long)m * g.ldc + col;
            const int so = row * PF + cc * 16;
            if (g.C) *(uint4*)((uint16_t*)g.C + off) = *(const uint4*)(sG + so);
            if (g.C2) *(uint4*)((uint16_t*)g.C2 + off) = *(const uint4*)(sU + so);
            if (g.C3) *(uint4*)((uint16_t*)g.C3 + off) = *(const uint4*)(sH + so);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();  // the staging area is rewritten next
    });
    return;
  }
  if constexpr (EPI == EPI_SWIGLU_FWD) {
    // G, U and H go out straight from the accumulators (8-byte pieces, merged
    // into whole lines by L2): measured faster than staging three arrays
    // through LDS.
    const int lrow = lane & 31, lgrp = (lane >> 5) * 4;
    const int hh0 = n0 / 2 + wn * (WTN / 2);
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const int m = m0 + wm * WTM + i * 32 + lrow;
      if (m >= m_end) return;
      static_for<TN / 2>([&](auto J) {
        constexpr int j = decltype(J)::value;
        static_for<4>([&](auto Q) {
          constexpr int q = decltype(Q)::value;
          const int c = hh0 + j * 32 + q * 8 + lgrp;
          if (c >= g.split) return;
          float gv[4], uv[4], hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            gv[r] = acc[i][j][q * 4 + r];
            uv[r] = acc[i][j + TN / 2][q * 4 + r];
            hv[r] = silu_f(gv[r]) * uv[r];
          }
          // any of G, U, H may be absent: a memory-lean forward stores H only,
          // the backward's recompute G and U only (uniform branches)
          const long off = (long)m * g.ldc + c;
          if (g.C) *(uint2*)((uint16_t*)g.C + off) = make_uint2(pack_bf2(gv[0], gv[1]), pack_bf2(gv[2], gv[3]));
          if (g.C2) *(uint2*)((uint16_t*)g.C2 + off) = make_uint2(pack_bf2(uv[0], uv[1]), pack_bf2(uv[2], uv[3]));
          if (g.C3) *(uint2*)((uint16_t*)g.C3 + off) = make_uint2(pack_bf2(hv[0], hv[1]), pack_bf2(hv[2], hv[3]));
        });
      });
    });
    return;
  }
  static_assert(SR * P <= WLDS, "epilogue LDS");
  const int lrow = lane & 31, lgrp = (lane >> 5) * 4;
  const int mw = m0 + wm * WTM;
  const int srow = lrow & (SR - 1);
  auto stage4 = [&](char* slab, int pitch, int col, float v0, float v1, float v2, float v3) {
    *(uint2*)(slab + srow * pitch + col * 2) = make_uint2(pack_bf2(v0, v1), pack_bf2(v2, v3));
  };
  // Slab rows -> memory: chunk c of COLS/8 16-byte chunks per row.
  auto store_rows = [&](const char* slab, int pitch, int cols, int ms, auto&& dst) {
    const int cpr = cols / 8;
    for (int c = lane; c < SR * cpr; c += 64) {
      const int row = c / cpr, cc = c - row * cpr;
      if (ms + row < m_end) dst(ms + row, cc * 8, *(const uint4*)(slab + row * pitch + cc * 16));
    }
  };
  if constexpr (EPI == EPI_BF16 && SR > 32) {
    // SUB whole 32-row subtiles per round: fewer LDS write -> read turns
    constexpr int SUB = SR / 32;
    static_assert(TM % SUB == 0, "subtiles per round");
    char* sC = wl;
    const int nw = n0 + wn * WTN;
    static_for<TM / SUB>([&](auto IS) {
      constexpr int i0 = decltype(IS)::value * SUB;
      const int ms = mw + i0 * 32;
      if (ms < m_end) {
        static_for<SUB>([&](auto S) {
          constexpr int sub = decltype(S)::value;
          static_for<TN>([&](auto J) {
            constexpr int j = decltype(J)::value;
            static_for<4>([&](auto Q) {
              constexpr int q = decltype(Q)::value;
              *(uint2*)(sC + (sub * 32 + lrow) * P + (j * 32 + q * 8 + lgrp) * 2) =
                  make_uint2(pack_bf2(acc[i0 + sub][j][q * 4 + 0], acc[i0 + sub][j][q * 4 + 1]),
                             pack_bf2(acc[i0 + sub][j][q * 4 + 2], acc[i0 + sub][j][q * 4 + 3]));
            });
          });
        });
        __builtin_amdgcn_wave_barrier();
        store_rows(sC, P, WTN, ms, [&](int m, int c, uint4 v) {
          if (nw + c < g.N) {
            uint16_t* Cb = (uint16_t*)g.C;
            int mr = m;
            if constexpr (CSEL == CSEL_MSPLIT) {
              if (m >= g.split) {
                Cb = (uint16_t*)g.C2;
                mr = m - g.split;
              }
            }
            store_row16(NT, Cb + (long)e * g.c_es + (long)mr * g.ldc + nw + c, v);
          }
        });
      }
      __builtin_amdgcn_wave_barrier();  // the slab area is rewritten next
    });
    return;
  }
  // SWIGLU_BWD: G and U of one slab, GUQ 16-byte pieces per lane, in flight
  // one slab ahead
  constexpr int GUQ = EPI == EPI_SWIGLU_BWD ? SR * (WTN / 8) / 64 : 1;
  static_assert(EPI != EPI_SWIGLU_BWD || SR * (WTN / 8) % 64 == 0, "slab pieces per lane");
  uint4 gq[GUQ], uq[GUQ];
  auto load_gu = [&](int ms) {
#pragma unroll
    for (int q = 0; q < GUQ; ++q) {
      const int c = lane + 64 * q, row = c / (WTN / 8), cc = c - row * (WTN / 8);
      const int m = ms + row, n = n0 + wn * WTN + cc * 8;
      gq[q] = make_uint4(0, 0, 0, 0);
      uq[q] = gq[q];
      if (m < m_end && n < g.N) {
        gq[q] = *(const uint4*)(g.G + (long)m * g.ldgu + n);
        uq[q] = *(const uint4*)(g.U + (long)m * g.ldgu + n);
      }
    }
  };
  if constexpr (EPI == EPI_SWIGLU_BWD) load_gu(mw);
  static_for<TM * NPART>([&](auto IH) {
    constexpr int i = decltype(IH)::value / NPART;
    constexpr int part = decltype(IH)::value % NPART;
    const int ms = mw + i * 32 + part * SR;
    const bool mine = (lrow / SR) == part;  // lane's row is in this part
    if (ms < m_end) {
      if constexpr (EPI == EPI_SWIGLU_BWD) {
        // dH = acc; G and U come in coalesced (this slab's loads were issued
        // during the previous slab), dG and dU go out the same way.
        char* sG = wl;
        char* sU = wl + SR * P;
#pragma unroll
        for (int q = 0; q < GUQ; ++q) {
          const int c = lane + 64 * q, row = c / (WTN / 8), cc = c - row * (WTN / 8);
          *(uint4*)(sG + row * P + cc * 16) = gq[q];
          *(uint4*)(sU + row * P + cc * 16) = uq[q];
        }
        if constexpr (decltype(IH)::value + 1 < TM * NPART) {
          constexpr int ni = (decltype(IH)::value + 1) / NPART, npart = (decltype(IH)::value + 1) % NPART;
          load_gu(mw + ni * 32 + npart * SR);
        }
        __builtin_amdgcn_wave_barrier();
        static_for<TN>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            if (!mine) return;
            const int off = srow * P + (j * 32 + q * 8 + lgrp) * 2;
            const uint2 gw = *(const uint2*)(sG + off);
            const uint2 uw = *(const uint2*)(sU + off);
            const float gg[4] = {bf_lo(gw.x), bf_hi(gw.x), bf_lo(gw.y), bf_hi(gw.y)};
            const float uu[4] = {bf_lo(uw.x), bf_hi(uw.x), bf_lo(uw.y), bf_hi(uw.y)};
            float dg[4], du[4];
            static_for<4>([&](auto Rr) {
              constexpr int r = decltype(Rr)::value;
              const float v = acc[i][j][q * 4 + r];
              const float sg = sigmoid_f(gg[r]);
              du[r] = v * gg[r] * sg;
              dg[r] = v * uu[r] * sg * (1.0f + gg[r] * (1.0f - sg));
            });
            *(uint2*)(sG + off) = make_uint2(pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]));
            *(uint2*)(sU + off) = make_uint2(pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]));
          });
        });
        __builtin_amdgcn_wave_barrier();
        const int nw = n0 + wn * WTN;
        uint16_t* D = (uint16_t*)g.C;
        store_rows(sG, P, WTN, ms, [&](int m, int c, uint4 v) {
          if (nw + c < g.N) store_row16(NT, D + (long)m * g.ldc + nw + c, v);
        });
        store_rows(sU, P, WTN, ms, [&](int m, int c, uint4 v) {
          if (nw + c < g.N) store_row16(NT, D + (long)m * g.ldc + g.split + nw + c, v);
        });
      } else {
        char* sC = wl;
        static_for<TN>([&](auto J) {
          constexpr int j = decltype(J)::value;
          static_for<4>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
            if (mine)
              stage4(sC, P, j * 32 + q * 8 + lgrp, acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1],
                     acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]);
          });
        });
        __builtin_amdgcn_wave_barrier();
        const int nw = n0 + wn * WTN;
        store_rows(sC, P, WTN, ms, [&](int m, int c, uint4 v) {
          if (nw + c < g.N) {
            uint16_t* Cb = (uint16_t*)g.C;
            int mr = m;
            if constexpr (CSEL == CSEL_MSPLIT) {
              if (m >= g.split) {
                Cb = (uint16_t*)g.C2;
                mr = m - g.split;
              }
            }
            store_row16(NT, Cb + (long)e * g.c_es + (long)mr * g.ldc + nw + c, v);
          }
        });
      }
      __builtin_amdgcn_wave_barrier();  // the slab area is rewritten next
    }
  });
}

// Per-expert prefixes of the persistent schedules, computed by every
// workgroup in its prologue from the expert offsets (E <= 1024) into LDS:
// one read of offsets and a block scan, instead of a separate launch per
// GEMM that the GEMM would wait for (a one-block kernel queued behind a
// persistent GEMM on another stream waits for whole tiles to drain).
// pre[0, E] (and pre[E+1, 2E+1] for two lists) receive the exclusive prefix
// of f0(e) (and f1(e)); pre[E] is the total.
template <int NT, class F>
TRG_DEV void block_prefix_1024(int n, F f, int* out, int* tmp) {
  constexpr int PER = 1024 / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int v[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    v[i] = e < n ? f(e) : 0;
    sum += v[i];
  }
  int x = sum;  // inclusive scan over the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const int t = tmp[w];
      tmp[w] = run;
      run += t;
    }
  }
  __syncthreads();
  int ex = tmp[wv] + x - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid * PER + i;
    if (e < n) out[e] = ex;
    ex += v[i];
  }
  if (tid == NT - 1) out[n] = ex;
  __syncthreads();  // tmp is reused by the next call
}

// Ragged-M tile prefixes (see RmSched): BM = 128, [E+1] 128-row tiles;
// BM = 256, [E+1] full-cost tiles then [E+1] light tails.
template <int BM, int NT>
TRG_DEV void rm_prefix(const int* offsets, int E, int split, int* pre, int* tmp) {
  auto cnt = [&](int e) { return offsets[e + 1] - offsets[e]; };
  if constexpr (BM == 128) {
    block_prefix_1024<NT>(E, [&](int e) { return (cnt(e) + 127) / 128; }, pre, tmp);
  } else {
    auto light = [&](int c) { const int tail = c & 255; return split && tail > 0 && tail <= 128; };
    block_prefix_1024<NT>(E, [&](int e) { const int c = cnt(e); return (c + 255) / 256 - (light(c) ? 1 : 0); },
                          pre, tmp);
    block_prefix_1024<NT>(E, [&](int e) { return light(cnt(e)) ? 1 : 0; }, pre + (E + 1), tmp);
  }
}

// Ragged-K work prefix (see wgrad_range): K steps of each expert's tiles plus
// kTileFixedSteps.
constexpr int kTileFixedSteps = 2;
template <int NT>
TRG_DEV void wgrad_prefix(const int* koff, int E, int kstep, int* pre, int* tmp) {
  block_prefix_1024<NT>(E, [&](int e) { return (koff[e + 1] - koff[e] + kstep - 1) / kstep + kTileFixedSteps; },
                        pre, tmp);
}

// Ragged-M schedule.  Every row tile has the same K, but an expert's last
// row tile is often nearly empty, and its MFMAs are skipped
// (subtiles past m_end): with 256-row tiles such a tail costs about half a
// tile.  toff holds the per-expert prefixes of rm_prefix:
//   BM = 128: [E+1] prefix of the experts' 128-row tiles;
//   BM = 256: [E+1] prefix of full-cost tiles (more than 128 valid rows: the
//             whole 256-row tiles and a tail of 129..255 rows), then [E+1]
//             prefix of light tails (1..128 rows).
// (Light tails are split out only where split_tails() says so; otherwise
// every row tile is in the first list and the second is empty.)
// Each XCD takes an eighth of the full-cost tiles (times the column tiles),
// in expert order, followed by an eighth of the light tails: its CUs walk the
// list round-robin, so the light tails land on the CUs that got one full
// tile fewer (8 experts of ~4096 rows: 1024 full-cost tiles, 4 per CU, and 16
// light tails, instead of 1040 tiles of which 16 CUs ran a fifth full one).
struct RmSched {
  int f0, nf, l0, nl;  // this XCD's full-cost list slice [f0, f0+nf) and light slice [l0, l0+nl)
};

template <int BM>
TRG_DEV RmSched rm_sched(const int* toff, int E, int tiles_n, int xcd) {
  RmSched r;
  const int F = toff[E] * tiles_n;
  const int L = BM == 256 ? toff[(E + 1) + E] * tiles_n : 0;
  const int fper = (F + 7) >> 3, lper = (L + 7) >> 3;
  r.f0 = min(F, xcd * fper);
  r.nf = min(F, r.f0 + fper) - r.f0;
  r.l0 = min(L, xcd * lper);
  r.nl = min(L, r.l0 + lper) - r.l0;
  return r;
}

// Position p of an XCD's walk -> expert, first row, row end and column tile.
template <int BM>
TRG_DEV void rm_tile(const int* toff, const int* offs, int E, int tiles_n, const RmSched& r, int p, int& e, int& m0,
                     int& m_end, int& nt) {
  const bool light = p >= r.nf;
  const int* pre = light ? toff + (E + 1) : toff;
  const int idx = light ? r.l0 + (p - r.nf) : r.f0 + p;
  const int mtg = idx / tiles_n;
  nt = idx - mtg * tiles_n;
  int lo = 0, hi = E;  // last expert with pre[e] <= mtg
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= mtg) lo = mid; else hi = mid;
  }
  e = lo;
  m_end = offs[lo + 1];
  m0 = light ? offs[lo] + ((m_end - offs[lo]) & ~255) : offs[lo] + (mtg - pre[lo]) * BM;
}

// Weight-gradient tiles differ in work: a tile's K loop runs over its
// expert's rows.  work[e] = sum over experts e' < e of one tile's work,
// ceil(rows_e' / K step) K steps plus kTileFixedSteps for the tile's prologue
// and epilogue; every expert has per_e tiles, expert-major.  The tile list is cut
// into the eight XCD ranges by count (as the ragged-M GEMMs are) unless that
// leaves one XCD more than 1.25x the mean work; then it is cut by work, so a
// skewed routing (one expert holding a sixth of the rows) does not leave
// seven XCDs idle while one works through the heavy experts.  By work, XCD x
// takes the tiles whose cumulative work starts in [x W / 8, (x + 1) W / 8).
// (The count cut stays the default because with about one tile per CU a cut
// one tile off the count costs a whole extra tile on some CU.)
TRG_DEV void wgrad_range(const int* work, int E, int per_e, int total, int xcd, int& t_begin, int& t_end) {
  const long W = (long)work[E] * per_e;
  const int per = (total + 7) >> 3;
  auto cum = [&](int t) -> long {  // work of tiles [0, t)
    if (t >= total) return W;
    const int e = t / per_e;
    return (long)work[e] * per_e + (long)(t - e * per_e) * (work[e + 1] - work[e]);
  };
  long wmax = 0;
  for (int x = 0; x < 8; ++x) {
    const long wx = cum(min(total, (x + 1) * per)) - cum(min(total, x * per));
    wmax = wx > wmax ? wx : wmax;
  }
  if (wmax * 8 * 4 <= W * 5) {
    t_begin = min(total, xcd * per);
    t_end = min(total, t_begin + per);
    return;
  }
  auto tile_at = [&](long target) -> int {  // first tile whose work starts at or after target
    if (target >= W) return total;
    int lo = 0, hi = E;  // last expert whose first tile starts at or before target
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long)work[mid] * per_e <= target) lo = mid; else hi = mid;
    }
    const long we = work[lo + 1] - work[lo];  // >= kTileFixedSteps > 0
    const long j = (target - (long)work[lo] * per_e + we - 1) / we;
    return lo * per_e + (int)(j < per_e ? j : per_e);
  };
  t_begin = tile_at(xcd * W / 8);
  t_end = xcd == 7 ? total : tile_at((xcd + 1) * W / 8);
}

// Light tails get their own place in the walk only where experts are large
// (R >= 2048 E): there an extra tile round is a large share of the kernel,
// while with a few hundred rows per expert moving every tail away from its
// expert's other tiles loses the weights' L2 reuse (wide shape: +3%).
inline int split_tails(int E, int R) { return (long)R >= 2048L * E ? 1 : 0; }

inline int cdiv(long a, long b) { return (int)((a + b - 1) / b); }

struct DevInfo {
  int cus = 0;
};
inline int grid_for(int tiles) {
  static DevInfo g_dev[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (g_dev[dev].cus == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_dev[dev].cus = n;
  }
  int grid = (g_dev[dev].cus + 7) / 8 * 8;  // a multiple of 8: whole XCD groups
  const int need = (tiles + 7) / 8 * 8;
  if (need < grid) grid = need;
  return grid < 8 ? 8 : grid;
}

// Row tile of the ragged-M GEMMs: 256 unless experts are small on average.
inline bool small_rows(int E, int R) { return R < 192L * E; }

}  // namespace gg
}  // namespace trg
