/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE expert-layer library.
 *
 * One GPU's share of an Olmo-core 3 style mixture-of-experts layer, forward and
 * backward:
 *
 *   router logits -> softmax / top-k with all routing metadata kept on the GPU
 *   -> rowwise dispatch of every routed token row straight into per-expert
 *   contiguous input buffers -> one grouped GEMM over all experts' SwiGLU FFNs
 *   -> gate-weighted combine; and the matching backward.
 *
 * Sources: "Olmo-core 3 open mixture-of-experts training infrastructure"
 * (agentlenshq.com), section "Routing and compute optimisation": routed tokens
 * are written directly into the experts' input buffers, routing metadata stays
 * on the GPU so the CPU is not a bottleneck, and many small per-expert matrix
 * products are batched into one larger grouped GEMM call.  The Thai
 * announcement (ai4bro.com, "Scaling and optimising MoE training") adds that
 * the CPU can queue work without waiting for data copies.  The same page set
 * names MXFP8 as the low-precision option ("Precision optimisation with
 * MXFP8").  The pages define no interface; the calls below are this library's.
 *
 * Conventions for every call
 * ---------------------------
 *  - All pointers are DEVICE pointers unless stated; the caller owns every
 *    buffer.  The library never allocates device memory: scratch comes from a
 *    caller workspace sized by the matching *_workspace_size() call (the one
 *    exception, moe_route_noalloc, uses a fixed static array of the library).
 *  - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null
 *    stream) and returns.  No call copies device data to the host and none
 *    synchronises a stream or the device.  Buffer sizes depend only on
 *    T, d, E, k, h (dropless: R = T*k routed rows).
 *  - Tensors are contiguous and row-major.  Shapes:
 *      x, y, dx [T,d]; wr, dwr [E,d]; logits, probs [T,E] f32;
 *      topk_idx, pos [T,k] i32; topk_w, dgate [T,k] f32;
 *      counts [E], offsets [E+1], off128 [E+1], src [R] i32;
 *      xp, yp, dyp, dxp [R,d]; g, u, hbuf [R,h]; dgu [R,2h] (dG | dU);
 *      w1, w3, dw1, dw3 [E,h,d]; w2, dw2 [E,d,h]   (output-major, K last).
 *  - dt selects the storage type of activations, weights and gradients:
 *    MOE_F32 or MOE_BF16.  Accumulation is always fp32.
 *  - Data pointers must be 16-byte aligned; row widths in bytes (d or h times
 *    the element size) must be multiples of 16.
 *  - Errors: a non-zero moe_status_t; moe_last_error_string() holds a message
 *    (thread-local).  Nothing throws across the ABI and nothing aborts.  After
 *    an error no work has been enqueued by that call, except MOE_ERR_HIP which
 *    reports a failed launch.
 *  - Results are bitwise reproducible run to run (no order-dependent float
 *    atomics) and independent of grid sizes.
 *  - Only gfx950 is supported (MOE_ERR_UNSUPPORTED otherwise).
 */
#ifndef TRG_MOE_H
#define TRG_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* bad size, null pointer, k > E, ...            */
  MOE_ERR_UNSUPPORTED = 2,  /* device is not gfx950, or dtype combination    */
  MOE_ERR_ALIGNMENT = 3,    /* pointer or row width not 16-byte aligned      */
  MOE_ERR_WORKSPACE = 4,    /* workspace null or smaller than required       */
  MOE_ERR_HIP = 5           /* a HIP launch or runtime call failed           */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2, MOE_E8M0 = 3 } moe_dtype_t;

/* Device-side data errors OR-ed into *err_flag by moe_route (forced routing). */
#define MOE_FLAG_INDEX_RANGE 1  /* a forced expert index outside [0, E)      */
#define MOE_FLAG_DUPLICATE 2    /* a token lists the same expert twice       */

/* Limits: 1 <= k <= min(E, 32); E <= 1024; T*k < 2^31. */

const char* moe_version(void);
const char* moe_last_error_string(void);

/*
 * Optional per-kernel timing for benchmarks (not part of the layer's math).
 * moe_prof_enable(1): every grouped-GEMM kernel and every other entry point
 * afterwards is bracketed by two HIP events recorded on its launch stream.
 * moe_prof_query(name): waits for the recorded events of launches called
 * `name` and returns their count and summed milliseconds (this call does
 * block the host).  moe_prof_names(): newline-separated names seen so far;
 * returns the size needed (including the NUL).  moe_prof_reset() frees all
 * recorded events.  moe_prof_only(name): from then on only launches called
 * `name` are bracketed (null or "": every launch, the default); the name is
 * copied.
 */
moe_status_t moe_prof_enable(int on);
moe_status_t moe_prof_only(const char* name);
moe_status_t moe_prof_reset(void);
moe_status_t moe_prof_query(const char* name, int* count, float* total_ms);
size_t moe_prof_names(char* buf, size_t n);

/*
 * moe_router_logits: logits[t,e] = sum_c x[t,c] * wr[e,c], fp32 accumulate,
 * fp32 output.  The router of the MoE block (the pages call the step routing;
 * its form -- a linear router followed by softmax / top-k -- is this
 * library's reading).  x [T,d], wr [E,d] of type dt; logits [T,E] f32.
 */
moe_status_t moe_router_logits(const void* x, int dt, const void* wr, int T, int d, int E,
                               float* logits, void* stream);

/*
 * moe_route: softmax + top-k + GPU-resident routing metadata ("Routing and
 * compute optimisation": routing metadata stays on the GPU).
 *   probs[t,:]  = softmax(logits[t,:]) (max-subtracted, fp32)
 *   topk_idx[t,j] = the j-th largest logit's expert; ties go to the lower
 *                 index.  If forced_idx [T,k] is non-null it is used instead
 *                 (random-routing stress modes); entries outside [0,E) are
 *                 clamped and flagged, duplicates flagged.
 *   topk_w[t,j] = probs[t, topk_idx[t,j]]  (not renormalised)
 *   counts[e]   = number of (t,j) routed to e; offsets = exclusive prefix sum
 *                 (offsets[E] = T*k); off128 (nullable) = prefix sum of counts
 *                 rounded up to multiples of 128 (MX column segments: each
 *                 starts on a 128-byte line of the columnwise copies).
 *   pos[t,j]    = row of (t,j) in the expert-contiguous buffer: offsets[e]
 *                 plus the number of entries (t',j') < (t,j) in (token, slot)
 *                 order routed to the same e.  src[pos[t,j]] = t*k + j.
 *   err_flag    = nullable int32; MOE_FLAG_* bits are OR-ed in on the device.
 * ws: moe_route_workspace_size(T,E,k) bytes.  Bit-exact for identical logits.
 */
size_t moe_route_workspace_size(int T, int E, int k);
moe_status_t moe_route(const float* logits, int T, int E, int k, const int32_t* forced_idx,
                       float* probs, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* pos, int32_t* src, int32_t* off128,
                       int32_t* err_flag, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_noalloc: moe_route for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results without ws / ws_bytes.  Its
 * scratch (the per-chunk expert counts) is a static device array of 4 MiB
 * inside the library, one per GPU, held until the process ends; routings that
 * need more (ceil(T*k/256) * E * 4 bytes: T*k above 2^18 rows at E = 1024,
 * above 2^21 at E = 128) are refused with MOE_ERR_WORKSPACE.  The call itself allocates nothing.
 * Every call on one GPU uses that GPU's array and leaves its contents behind
 * (each call writes every word it reads first), so calls that overlap on one
 * GPU -- concurrent streams, or threads enqueueing at once -- race; serialise
 * them or use moe_route.
 */
moe_status_t moe_route_noalloc(const float* logits, int T, int E, int k, const int32_t* forced_idx,
                               float* probs, int32_t* topk_idx, float* topk_w, int32_t* counts,
                               int32_t* offsets, int32_t* pos, int32_t* src, int32_t* off128,
                               int32_t* err_flag, void* stream);

/*
 * moe_permute: rowwise dispatch ("Routing and compute optimisation": routed
 * tokens are written directly into the experts' input buffers).  Token-major:
 * each x[t] row is read once and written to its k rows xp[pos[t,j]].
 */
moe_status_t moe_permute(const void* x, int dt, int T, int d, int k, const int32_t* pos,
                         void* xp, void* stream);

/*
 * moe_combine: y[t] = sum_j topk_w[t,j] * yp[pos[t,j]], fp32 accumulation in
 * slot order, one rounding to dt.  The inverse of the dispatch.
 */
moe_status_t moe_combine(const void* yp, const float* topk_w, const int32_t* pos, int T, int d,
                         int k, int dt, void* y, void* stream);

/*
 * moe_combine_bwd: dyp[pos[t,j]] = topk_w[t,j] * dy[t] (rounded to dt) and
 * dgate[t,j] = <dy[t], yp[pos[t,j]]> (fp32).  dyp may be null: then only dgate
 * is written (the MXFP8 backward quantises dYp straight from dy).
 */
moe_status_t moe_combine_bwd(const void* dy, const void* yp, const float* topk_w,
                             const int32_t* pos, int T, int d, int k, int dt, void* dyp,
                             float* dgate, void* stream);

/*
 * moe_unpermute_sum: dx[t] = sum_j dxp[pos[t,j]] (fp32 accumulation, one
 * rounding).  Adjoint of moe_permute.
 */
moe_status_t moe_unpermute_sum(const void* dxp, const int32_t* pos, int T, int d, int k, int dt,
                               void* dx, void* stream);

/*
 * moe_grouped_gemm_fwd: all experts' SwiGLU FFNs as grouped GEMMs over the
 * ragged expert segments [offsets[e], offsets[e+1]) of xp ("Routing and
 * compute optimisation": many small per-expert products batched into one
 * grouped GEMM).  One launch computes, for every expert at once,
 *   g = xp w1[e]^T, u = xp w3[e]^T, hbuf = silu(g) * u   (SwiGLU fused in the
 *   epilogue; g, u, hbuf stored in dt for the backward),
 * and a second launch yp = hbuf w2[e]^T.  The tile map is derived on the
 * device from offsets, by every workgroup in its prologue.  ws:
 * moe_grouped_gemm_workspace_size() bytes (0 in this version; ws may then be
 * null).
 * bf16 needs d and h to be multiples of 64 and R * max(d, 2h) * 2 < 2^31.
 * Memory-lean forward (bf16): g and/or u may be null, then they are not
 * stored; the backward recomputes them with moe_grouped_gemm_recompute_gu
 * (bit-identical to what this call would have stored), so only xp, hbuf and
 * yp have to live from the forward to the backward.
 */
size_t moe_grouped_gemm_workspace_size(int E, int R, int d, int h);
moe_status_t moe_grouped_gemm_fwd(const void* xp, const void* w1, const void* w3, const void* w2,
                                  const int32_t* offsets, int E, int R, int d, int h, int dt,
                                  void* g, void* u, void* hbuf, void* yp, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_bwd: backward of moe_grouped_gemm_fwd given dyp.
 *   dgrad down + SwiGLU backward (fused):  dH = dyp w2[e];  s = sigmoid(g);
 *     dU = dH * silu(g);  dG = dH * u * s * (1 + g (1 - s))  -> dgu [R,2h]
 *   wgrad down: dw2[e] = dyp_e^T hbuf_e   (K = the expert's rows)
 *   dgrad up:   dxp = dG w1[e] + dU w3[e]
 *   wgrad up:   dw1[e] = dG_e^T xp_e,  dw3[e] = dU_e^T xp_e
 * Weight gradients are accumulated in fp32 over the whole segment and rounded
 * once; an expert with no rows gets zero gradients.
 */
/*
 * moe_grouped_gemm_recompute_gu: the up projection of moe_grouped_gemm_fwd
 * alone, writing g = xp w1[e]^T and u = xp w3[e]^T (bf16, [R,h] each) and not
 * hbuf: the recompute of the memory-lean backward, which trades activation
 * memory for one more up projection.  Same arguments, layouts and workspace
 * as moe_grouped_gemm_fwd.
 */
moe_status_t moe_grouped_gemm_recompute_gu(const void* xp, const void* w1, const void* w3,
                                           const int32_t* offsets, int E, int R, int d, int h, int dt,
                                           void* g, void* u, void* ws, size_t ws_bytes, void* stream);

moe_status_t moe_grouped_gemm_bwd(const void* dyp, const void* xp, const void* g, const void* u,
                                  const void* hbuf, const void* w1, const void* w3,
                                  const void* w2, const int32_t* offsets, int E, int R, int d,
                                  int h, int dt, void* dgu, void* dxp, void* dw1, void* dw3,
                                  void* dw2, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm_bwd_parts: moe_grouped_gemm_bwd restricted to a subset of
 * its four GEMMs (bf16), so that a caller can run them on two streams:
 *   MOE_BWD_DGRAD_DOWN  dgu = SwiGLU-bwd(dyp W2[e], g, u)   needs dyp
 *   MOE_BWD_WGRAD_DOWN  dw2 = dyp^T hbuf per expert          needs dyp
 *   MOE_BWD_DGRAD_UP    dxp = dgu [W1; W3]                   needs dgu
 *   MOE_BWD_WGRAD_UP    dw1 | dw3 = dgu^T xp per expert      needs dgu
 * The pages report that overlapping streams does not always help
 * (Olmo-core 3 overview, "Empirical findings beyond raw speed"); this call is
 * what measures that here.  Calls that may run concurrently need separate
 * workspaces.  Same arguments as moe_grouped_gemm_bwd otherwise.
 */
enum {
  MOE_BWD_DGRAD_DOWN = 1,
  MOE_BWD_WGRAD_DOWN = 2,
  MOE_BWD_DGRAD_UP = 4,
  MOE_BWD_WGRAD_UP = 8,
  MOE_BWD_ALL = 15,
  /* MXFP8 parts only (moe_grouped_gemm_bwd_mx_parts): */
  MOE_BWD_MX_QUANT_DY = 16, /* make dYp's MX copies (nothing else unless other bits are set) */
  MOE_BWD_MX_DY_READY = 32  /* with MOE_BWD_DGRAD_DOWN: dYp's copies exist, do not remake them */
};
moe_status_t moe_grouped_gemm_bwd_parts(const void* dyp, const void* xp, const void* g, const void* u,
                                        const void* hbuf, const void* w1, const void* w3, const void* w2,
                                        const int32_t* offsets, int E, int R, int d, int h, int dt, void* dgu,
                                        void* dxp, void* dw1, void* dw3, void* dw2, unsigned parts, void* ws,
                                        size_t ws_bytes, void* stream);

/*
 * moe_router_bwd: gradient through the gates into the logits, wr and x.
 *   gh[t,e] = dgate[t,j] where e = topk_idx[t,j], else 0
 *   dlogits = probs * (gh - sum_e probs*gh)      (softmax backward)
 *   dwr = dlogits^T x;   dx += dlogits wr        (dx holds the expert-path
 *                                                 gradient on entry)
 * ws: moe_router_bwd_workspace_size(T,d,E) bytes.
 */
size_t moe_router_bwd_workspace_size(int T, int d, int E);
moe_status_t moe_router_bwd(const float* probs, const int32_t* topk_idx, const float* dgate,
                            const void* x, const void* wr, int T, int d, int E, int k, int dt,
                            void* dx, void* dwr, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_router_bwd_unpermute: moe_unpermute_sum and moe_router_bwd (or, with a
 * non-null aux_g, moe_router_bwd_aux) in one pass over dx, the input's whole
 * gradient: the adjoint of the dispatch (routed rows written straight into
 * the experts' buffers: Olmo-core 3 overview, "Routing and compute
 * optimisation") plus the gradient through the gates into x:
 *   dx[t] = sum_j dxp[pos[t,j]] + (dlogits wr)[t]
 * summed in fp32 (the slots in order, then the router term) and rounded once
 * to dt; dwr as moe_router_bwd.  dx is written, not read.
 *   dxp [T*k, d] dt, 16-byte aligned: the expert-path input gradient in
 *       expert order (moe_grouped_gemm_bwd's dxp); pos [T,k] from moe_route.
 *   Other arguments, workspace (moe_router_bwd_workspace_size) and errors as
 *   moe_router_bwd; aux_g may be null.
 */
moe_status_t moe_router_bwd_unpermute(const float* probs, const int32_t* topk_idx, const float* dgate,
                                      const float* aux_g, const void* x, const void* wr,
                                      const void* dxp, const int32_t* pos, int T, int d, int E, int k,
                                      int dt, void* dx, void* dwr, void* ws, size_t ws_bytes,
                                      void* stream);
/*
 * moe_router_bwd_unpermute_parts: moe_router_bwd_unpermute restricted to its
 * dwr part (MOE_ROUTER_DWR: needs dgate, not dxp) or its dx part
 * (MOE_ROUTER_DX: needs dxp), so that dwr can run on a second stream as soon
 * as the combine backward has written dgate.  Each part recomputes dlogits in
 * its own workspace: calls that may run concurrently need separate
 * workspaces.  A part's unused pointers may be null (dwr and x without
 * MOE_ROUTER_DWR; dx, wr, dxp and pos without MOE_ROUTER_DX).  Both parts
 * together equal moe_router_bwd_unpermute bit for bit.
 */
enum { MOE_ROUTER_DWR = 1, MOE_ROUTER_DX = 2 };
moe_status_t moe_router_bwd_unpermute_parts(const float* probs, const int32_t* topk_idx,
                                            const float* dgate, const float* aux_g, const void* x,
                                            const void* wr, const void* dxp, const int32_t* pos, int T,
                                            int d, int E, int k, int dt, void* dx, void* dwr, void* ws,
                                            size_t ws_bytes, unsigned parts, void* stream);

/*
 * Router balance step.  The pages warn that a routing balance score can
 * improve while the actual workload balance gets worse (token gerrymandering:
 * Olmo-core 3 overview, "Empirical findings beyond raw speed") but define no
 * score and no balance loss; the plain reading taken here:
 *   f_e = counts[e] / (T k),  P_e = (1/T) sum_t probs[t,e]
 *   score = E sum_e f_e P_e                 (1 when both are uniform)
 *   loss  = alpha * score                   (auxiliary load-balance loss)
 *   actual balance = max_e counts[e] / (T k / E)
 *   aux_g[e] = d loss / d probs[t,e] = alpha E f_e / T   (every t)
 *
 * moe_balance: probs [T,E] f32 and counts [E] i32 as written by moe_route;
 *   0 <= alpha (finite).  Writes stats[4] f32 = {score, loss, max/mean load,
 *   min/mean load}; aux_g [E] f32 and mean_probs [E] f32 (= P) if non-null.
 *   Deterministic (fixed-order sums).  ws: moe_balance_workspace_size(T, E)
 *   bytes.  Everything stays on the device.
 * moe_router_bwd_aux: moe_router_bwd with the balance loss: aux_g[e] (from
 *   moe_balance) is added to every token's gate-gradient row before the
 *   softmax backward, so dlogits, dwr and dx carry both terms.
 */
size_t moe_balance_workspace_size(int T, int E);
moe_status_t moe_balance(const float* probs, const int32_t* counts, int T, int E, int k, float alpha,
                         float* stats, float* aux_g, float* mean_probs, void* ws, size_t ws_bytes,
                         void* stream);
moe_status_t moe_router_bwd_aux(const float* probs, const int32_t* topk_idx, const float* dgate,
                                const float* aux_g, const void* x, const void* wr, int T, int d, int E,
                                int k, int dt, void* dx, void* dwr, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * ---------------------------------------------------------------------------
 * MXFP8 path ("Precision optimisation with MXFP8": MXFP8 cuts both compute and
 * the traffic between experts).  Encoding (OCP microscaling): E4M3FN elements
 * and one E8M0 scale byte per 32 consecutive values along a GEMM's reduction
 * dimension; s = clamp(floor(log2(amax)) - 8, -127, 127) taken from the
 * exponent bits (s = -127 for an all-zero block), scale byte s + 127,
 * elements E4M3FN(v / 2^s) rounded to nearest even and saturated to +-448,
 * sign of zero kept.  Layouts:
 *   rowwise      q [rows, cols] u8 (blocks along cols)
 *   columnwise   blocks of 32 consecutive rows inside each row segment, the
 *                last block of a segment zero-padded, stored expert-major:
 *                each segment's copy is the transpose of its padded rows, a
 *                contiguous [cols, len] block (row c = column c of the
 *                segment), so a GEMM over one expert reads rows len bytes
 *                apart.  With seg_off the copy of segment e starts at byte
 *                off128[e] * cols and len = off128[e+1] - off128[e] (a buffer
 *                of cols * ldc bytes); with fixed segments (the weights: S =
 *                rows/seg_rows segments) q is [S*cols, ldc], row e*cols + c
 *                holding column c of segment e
 *   scales       K-chunk major: for an MX matrix of n rows (rowwise: rows;
 *                columnwise: cols) with K values per row (rowwise: cols;
 *                columnwise: ldc), the scale of block b (K values 32b ..
 *                32b+31) of row r is byte (b/4 * n + r) * 4 + b%4, i.e.
 *                [ceil(K/128)][n][4] bytes: the four scales of a 128-wide
 *                K chunk of a row form one dword, and one chunk's dwords of
 *                consecutive rows are contiguous (a GEMM K step of 128 reads
 *                its tile's scales in one piece)
 * ---------------------------------------------------------------------------
 *
 * mx_quantize: quantise `rows` rows of a [*, cols] matrix `in` (dt = MOE_BF16
 * or MOE_F32, row stride cols) to either or both layouts in one pass.
 *   gather_src (nullable): logical row r is in[gather_src[r] / gather_k]
 *     (pass moe_route's src and k to quantise the routed rows of x straight
 *     from x: the rowwise dispatch and the quantisation in one step).
 *   seg_off / seg_off128 (nullable, [nseg+1]): row segments and their padded
 *     starts: multiples of 32, each padded segment at least as long as its
 *     segment and at most 127 rows longer (moe_route's offsets / off128); if null, segments of seg_rows rows
 *     (rows a multiple of seg_rows, or seg_rows = rows), each padded to 32.
 *   q_row/s_row (nullable): rowwise output; s_row holds ceil(cols/128) * rows
 *     * 4 bytes.  q_col/s_col (nullable): columnwise output; ldc a multiple of
 *     32.  With seg_off, ldc >= rows + 127*nseg is the padded row capacity:
 *     q_col holds cols * ldc bytes, s_col ceil(ldc/128) * cols * 4.  With
 *     fixed segments, ldc >= round32(seg_rows) is the row stride: q_col holds
 *     rows/seg_rows * cols rows of ldc, s_col ceil(ldc/128) * rows/seg_rows *
 *     cols * 4 bytes.
 * cols must be a multiple of 32.  Bit-exact and deterministic.
 */
moe_status_t mx_quantize(const void* in, int dt, int rows, int cols, const int32_t* gather_src, int gather_k,
                         const int32_t* seg_off, const int32_t* seg_off128, int nseg, int seg_rows, uint8_t* q_row,
                         uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int ldc, void* stream);

/*
 * MXFP8 grouped GEMMs of the expert FFNs: the same SwiGLU forward and backward
 * as moe_grouped_gemm_fwd / _bwd, with every GEMM operand quantised along its
 * own reduction dimension and multiplied on gfx950's scaled matrix cores
 * (fp32 accumulation, bf16 outputs).  d and h must be multiples of 128; rcap
 * (padded row capacity of every columnwise copy: a copy of n columns holds
 * n * rcap bytes, expert-major as mx_quantize writes it) a multiple of 128 and
 * >= R + 127*E;
 * off128 as moe_route writes it (segment starts on multiples of 128).  Scale
 * arrays are in the K-chunk-major layout above; with d, h and rcap multiples
 * of 128 each holds exactly (values)/32 bytes, e.g. xs = R*d/32.
 * The caller quantises x (mx_quantize with gather) and the weights; the calls
 * quantise H, dYp and dG|dU themselves (both layouts, from the stored bf16
 * values).  ws: moe_grouped_gemm_workspace_size() bytes.
 */
typedef struct {
  int E, R, d, h, rcap;
  const int32_t* offsets;                 /* [E+1] expert row offsets          */
  const int32_t* off128;                   /* [E+1] 128-padded segment starts   */
  const uint8_t* xq; const uint8_t* xs;   /* [R,d], [R,d/32] routed x, rowwise */
  const uint8_t* w1q; const uint8_t* w1s; /* [E,h,d], [E,h,d/32] rowwise       */
  const uint8_t* w3q; const uint8_t* w3s; /* [E,h,d], [E,h,d/32] rowwise       */
  const uint8_t* w2q; const uint8_t* w2s; /* [E,d,h], [E,d,h/32] rowwise       */
  void* g; void* u; void* hbuf;           /* out: [R,h] bf16                   */
  uint8_t* hq; uint8_t* hs;               /* out: [R,h], [R,h/32] rowwise H    */
  uint8_t* hqT; uint8_t* hsT;             /* out: h*rcap (expert-major), [h,rcap/32] */
  void* yp;                               /* out: [R,d] bf16                   */
  void* ws; size_t ws_bytes;
} moe_mx_fwd_args;

typedef struct {
  int E, R, d, h, rcap;
  const int32_t* offsets;
  const int32_t* off128;
  const void* dyp;                          /* [R,d] bf16 (moe_combine_bwd)         */
  uint8_t* dyq; uint8_t* dys;               /* out: [R,d], [R,d/32] rowwise dYp     */
  uint8_t* dyqT; uint8_t* dysT;             /* out: d*rcap (expert-major), [d,rcap/32] */
  const void* g; const void* u;             /* [R,h] bf16 from the forward          */
  const uint8_t* hqT; const uint8_t* hsT;   /* columnwise H from the forward        */
  const uint8_t* xqT; const uint8_t* xsT;   /* d*rcap columnwise routed x (expert-major) */
  const uint8_t* w1tq; const uint8_t* w1ts; /* [E*d,h], [E*d,h/32]: W1 blocked on h,
                                               expert-major (mx_quantize, seg_rows h) */
  const uint8_t* w3tq; const uint8_t* w3ts; /* same for W3                          */
  const uint8_t* w2tq; const uint8_t* w2ts; /* [E*h,d], [E*h,d/32]: W2 blocked on d,
                                               expert-major (seg_rows d)            */
  void* dgu;                                /* out: [R,2h] bf16 (dG | dU)           */
  uint8_t* dguq; uint8_t* dgus;             /* out: [R,2h], [R,2h/32]               */
  uint8_t* dguqT; uint8_t* dgusT;           /* out: 2h*rcap (expert-major), [2h,rcap/32] */
  void* dxp;                                /* out: [R,d] bf16                      */
  void* dw1; void* dw3; void* dw2;          /* out: weight gradients, bf16          */
  void* ws; size_t ws_bytes;
  /* dYp's MX copies straight from dy, without dyp: when dyp is null, row r of
   * dYp is taken as bf16(topk_w[src[r]] * dy[src[r] / k]), exactly what
   * moe_combine_bwd would have stored (it may then be called with dyp = null,
   * for dgate only).  dy [T,d] bf16, topk_w [T,k] f32 and src [R] i32 as
   * moe_route wrote them; unused when dyp is given. */
  const void* dy; const float* topk_w; const int32_t* src; int k;
} moe_mx_bwd_args;

moe_status_t moe_grouped_gemm_fwd_mx(const moe_mx_fwd_args* args, void* stream);
moe_status_t moe_grouped_gemm_bwd_mx(const moe_mx_bwd_args* args, void* stream);
/*
 * moe_grouped_gemm_fwd_mx_parts: moe_grouped_gemm_fwd_mx in two halves, so
 * that a caller making the weights' MX copies on another stream can start the
 * up projection once W1's and W3's copies exist and wait for W2's only before
 * the down projection.  MOE_FWD_UP: the up projection with its SwiGLU
 * epilogue (g, u, hbuf) and H's MX copies (hq/hs, hqT/hsT); reads xq/xs,
 * w1q/w1s, w3q/w3s.  MOE_FWD_DOWN: the down projection (yp) from H's rowwise
 * copy and w2q/w2s; needs the up part done.  Both bits: moe_grouped_gemm_fwd_mx.
 * Same arguments and checks as moe_grouped_gemm_fwd_mx; parts must be a
 * non-empty subset of MOE_FWD_ALL (else MOE_ERR_INVALID_ARG).
 */
enum {
  MOE_FWD_UP = 1,
  MOE_FWD_DOWN = 2,
  MOE_FWD_ALL = 3
};
moe_status_t moe_grouped_gemm_fwd_mx_parts(const moe_mx_fwd_args* args, unsigned parts, void* stream);
/*
 * moe_grouped_gemm_bwd_mx_parts: moe_grouped_gemm_bwd_mx restricted to a
 * subset (MOE_BWD_* mask) of its four GEMMs, for two streams as with
 * moe_grouped_gemm_bwd_parts.  MOE_BWD_DGRAD_DOWN also makes dYp's MX copies
 * (dyq/dys, dyqT/dysT) before its GEMM, unless MOE_BWD_MX_DY_READY is set
 * (an earlier MOE_BWD_MX_QUANT_DY call made them), and dG|dU's (dguq/dgus,
 * dguqT/dgusT) after it.  MOE_BWD_WGRAD_DOWN needs dYp's copies (either
 * way), MOE_BWD_WGRAD_UP and MOE_BWD_DGRAD_UP need the dgrad-down part done.
 * Calls that may run concurrently need separate workspaces.  Same arguments
 * and checks as moe_grouped_gemm_bwd_mx.
 */
moe_status_t moe_grouped_gemm_bwd_mx_parts(const moe_mx_bwd_args* args, unsigned parts, void* stream);
/*
 * Memory-lean MXFP8: moe_grouped_gemm_fwd_mx accepts g = u = null (not
 * stored); moe_grouped_gemm_recompute_gu_mx then runs the MX up projection
 * alone from xq/xs and the weights' forward copies, writing g and u only, so
 * the forward-to-backward state is the fp8 copies (xq, xqT, hqT) and yp.
 */
moe_status_t moe_grouped_gemm_recompute_gu_mx(const moe_mx_fwd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TRG_MOE_H */
