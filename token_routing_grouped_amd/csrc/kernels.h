// Internal launch entry points (host side) of the gfx950 kernels.  The C ABI
// in api.hip validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace trg {

// routing
size_t route_ws_bytes(int T, int E, int k);
// moe_route_noalloc: largest routing workspace its static scratch array holds
constexpr size_t kRouteScratchBytes = 4u << 20;
// device address of that array on the current device (resolved once per device)
hipError_t route_scratch(void** out);
hipError_t launch_route(const float* logits, int T, int E, int k, const int* forced, float* probs, int* idx,
                        float* w, int* counts, int* offsets, int* pos, int* src, int* off128, int* err_flag,
                        void* ws, hipStream_t s);

// dispatch / combine (bf16 = uint16_t storage, or float)
hipError_t launch_permute(const void* x, bool bf16, int T, int d, int k, const int* pos, void* xp, hipStream_t s);
hipError_t launch_gather_sum(const void* yp, const float* w, const int* pos, int T, int d, int k, bool bf16,
                             void* y, hipStream_t s);
hipError_t launch_combine_bwd(const void* dy, const void* yp, const float* w, const int* pos, int T, int d, int k,
                              bool bf16, void* dyp, float* dgate, hipStream_t s);

// router GEMMs
size_t router_bwd_ws_bytes(int T, int d, int E);
hipError_t launch_router_logits(const void* x, bool bf16, const void* wr, int T, int d, int E, float* logits,
                                hipStream_t s);
// dxp == nullptr: dx += dlogits wr.  Otherwise dx = sum_j dxp[pos[t,j]] +
// dlogits wr (the unpermute-sum folded in; dx is only written).  parts:
// kRouterDwr and / or kRouterDx (dlogits is computed for either).
constexpr unsigned kRouterDwr = 1, kRouterDx = 2;
hipError_t launch_router_bwd(const float* probs, const int* idx, const float* dgate, const float* aux_g,
                             const void* x, const void* wr, int T, int d, int E, int k, bool bf16, void* dx, void* dwr,
                             void* ws, hipStream_t s, const void* dxp = nullptr, const int* pos = nullptr,
                             unsigned parts = kRouterDwr | kRouterDx);
size_t balance_ws_bytes(int T, int E);
hipError_t launch_balance(const float* probs, const int* counts, int T, int E, int k, float alpha, float* stats,
                          float* aux_g, float* mean_probs, void* ws, hipStream_t s);

// grouped GEMMs
size_t ggemm_ws_bytes(int E, int R, int d, int h);
hipError_t launch_ggemm_fwd(const void* xp, const void* w1, const void* w3, const void* w2, const int* offsets,
                            int E, int R, int d, int h, bool bf16, void* g, void* u, void* hb, void* yp, void* ws,
                            hipStream_t s);
hipError_t launch_ggemm_bwd(const void* dyp, const void* xp, const void* g, const void* u, const void* hb,
                            const void* w1, const void* w3, const void* w2, const int* offsets, int E, int R, int d,
                            int h, bool bf16, void* dgu, void* dxp, void* dw1, void* dw3, void* dw2, void* ws, unsigned parts,
                            hipStream_t s);

// bf16 MFMA dense GEMM helpers used by the router (E >= 64)
hipError_t launch_dense_nt_f32out(const uint16_t* A, const uint16_t* B, float* C, int M, int N, int K,
                                  hipStream_t s);
hipError_t launch_router_dwr_mfma(const uint16_t* dL, const uint16_t* x, uint16_t* dwr, float* part, int T, int d,
                                  int E, hipStream_t s);
hipError_t launch_router_dx_mfma(const uint16_t* dL, const uint16_t* wr, uint16_t* dx, const uint16_t* dxp,
                                 const int* pos, int k, int T, int d, int E,
                                 hipStream_t s);
size_t router_dwr_mfma_part_bytes(int T, int d, int E);

// fp32 reference-shaped grouped GEMMs (small fp32 layers)
hipError_t launch_ggemm_fwd_f32(const float* xp, const float* w1, const float* w3, const float* w2,
                                const int* offsets, int E, int R, int d, int h, float* g, float* u, float* hb,
                                float* yp, hipStream_t s);
hipError_t launch_ggemm_bwd_f32(const float* dyp, const float* xp, const float* g, const float* u, const float* hb,
                                const float* w1, const float* w3, const float* w2, const int* offsets, int E, int R,
                                int d, int h, float* dgu, float* dxp, float* dw1, float* dw3, float* dw2,
                                hipStream_t s);

// MXFP8
hipError_t launch_mx_quantize(const void* in, bool bf16, long ld_in, int rows, int cols, const int* src, int gk,
                              const int* seg_off, const int* seg_off128, int nseg, int seg_rows, int max_blocks32,
                              uint8_t* q_row, uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, long ldc,
                              hipStream_t s, const float* gate = nullptr);
typedef moe_mx_fwd_args MxFwd;
typedef moe_mx_bwd_args MxBwd;
hipError_t launch_ggemm_recompute_gu(const void* xp, const void* w1, const void* w3, const int* offsets, int E, int R,
                                     int d, int h, void* g, void* u, void* ws, hipStream_t s);
hipError_t launch_ggemm_recompute_gu_mx(const MxFwd& p, hipStream_t s);
hipError_t launch_ggemm_fwd_mx(const MxFwd& p, unsigned parts, hipStream_t s);  // parts: MOE_FWD_* mask
hipError_t launch_ggemm_bwd_mx(const MxBwd& p, unsigned parts, hipStream_t s);

}  // namespace trg
