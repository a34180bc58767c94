// C ABI of the MoE expert-layer library: argument validation, workspace
// checks, error reporting, and the launches.  Every entry point only enqueues
// work on the caller's stream; none copies device data to the host or
// synchronises (the routing metadata never leaves the GPU).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"
#include "prof.h"

// ---- optional HIP-event timing of individual launches -----------------------
namespace trg {
namespace {
std::atomic<bool> g_prof{false};
std::mutex g_prof_mu;
struct ProfRec {
  std::string name;
  hipEvent_t b, e;
};
std::vector<ProfRec> g_prof_done;
std::vector<std::pair<std::string, hipEvent_t>> g_prof_open;
std::string g_prof_only;  // empty: every launch; else only launches of this name

bool prof_selected(const char* name) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  return g_prof_only.empty() || g_prof_only == name;
}
}  // namespace

bool prof_on() { return g_prof.load(std::memory_order_relaxed); }

// Timing-only events: without the default system-scope fence, recording one
// does not write back and invalidate the caches between the launches it
// brackets (timestamps are read after a device synchronisation).
hipError_t prof_event(hipEvent_t* ev) { return hipEventCreateWithFlags(ev, hipEventDisableSystemFence); }

void prof_begin(const char* name, hipStream_t s) {
  if (!prof_selected(name)) return;
  hipEvent_t ev;
  if (prof_event(&ev) != hipSuccess) return;
  (void)hipEventRecord(ev, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_open.emplace_back(name, ev);
}

void prof_end(const char* name, hipStream_t s) {
  if (!prof_selected(name)) return;
  hipEvent_t ev;
  if (prof_event(&ev) != hipSuccess) return;
  (void)hipEventRecord(ev, s);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (size_t i = g_prof_open.size(); i-- > 0;) {
    if (g_prof_open[i].first == name) {
      g_prof_done.push_back({name, g_prof_open[i].second, ev});
      g_prof_open.erase(g_prof_open.begin() + (long)i);
      return;
    }
  }
  (void)hipEventDestroy(ev);
}
}  // namespace trg

namespace {

thread_local std::string g_err;

moe_status_t fail(moe_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status_t ok() {
  g_err.clear();
  return MOE_OK;
}

// gfx950 check, cached per device.
constexpr int kMaxDev = 64;
int g_arch_ok[kMaxDev];  // 0 unknown, 1 ok, -1 not gfx950
std::mutex g_arch_mu;

moe_status_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDev) return fail(MOE_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDeviceProperties failed");
    g_arch_ok[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  if (g_arch_ok[dev] != 1) return fail(MOE_ERR_UNSUPPORTED, "this library is built for gfx950 only");
  return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

moe_status_t check_ptrs(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ps) {
  for (auto& p : ps) {
    if (p.second == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s: %s is null", fn, p.first);
    if (!aligned16(p.second)) return fail(MOE_ERR_ALIGNMENT, "%s: %s is not 16-byte aligned", fn, p.first);
  }
  return MOE_OK;
}

// Nullable pointers (not stored when null) must still be 16-byte aligned when
// given: the epilogues write them in 16-byte pieces.
moe_status_t check_optional_aligned(const char* fn, std::initializer_list<std::pair<const char*, const void*>> ps) {
  for (auto& p : ps)
    if (p.second != nullptr && !aligned16(p.second))
      return fail(MOE_ERR_ALIGNMENT, "%s: %s is not 16-byte aligned", fn, p.first);
  return MOE_OK;
}

moe_status_t check_dt(const char* fn, int dt) {
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: dt must be MOE_F32 or MOE_BF16", fn);
  return MOE_OK;
}

int esize(int dt) { return dt == MOE_F32 ? 4 : 2; }

moe_status_t check_row(const char* fn, const char* name, long n, int dt) {
  if (n <= 0) return fail(MOE_ERR_INVALID_ARG, "%s: %s must be positive", fn, name);
  if ((n * esize(dt)) % 16 != 0)
    return fail(MOE_ERR_ALIGNMENT, "%s: %s * element size must be a multiple of 16 bytes", fn, name);
  return MOE_OK;
}

moe_status_t check_tk(const char* fn, int T, int k) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  if (k < 1 || k > 32) return fail(MOE_ERR_INVALID_ARG, "%s: k must be in [1, 32]", fn);
  if ((long)T * k >= (1L << 31)) return fail(MOE_ERR_INVALID_ARG, "%s: T*k must be < 2^31", fn);
  return MOE_OK;
}

moe_status_t hip_status(const char* fn, hipError_t e) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
  return ok();
}

#define TRY(x)                      \
  do {                              \
    moe_status_t _st = (x);         \
    if (_st != MOE_OK) return _st;  \
  } while (0)

}  // namespace

extern "C" {

const char* moe_version(void) { return "trg-moe 0.1 (gfx950)"; }

const char* moe_last_error_string(void) { return g_err.c_str(); }

moe_status_t moe_prof_enable(int on) {
  trg::g_prof.store(on != 0);
  return ok();
}

moe_status_t moe_prof_only(const char* name) {
  std::lock_guard<std::mutex> lk(trg::g_prof_mu);
  trg::g_prof_only = name ? name : "";
  return ok();
}

moe_status_t moe_prof_reset(void) {
  std::lock_guard<std::mutex> lk(trg::g_prof_mu);
  for (auto& r : trg::g_prof_done) {
    (void)hipEventDestroy(r.b);
    (void)hipEventDestroy(r.e);
  }
  for (auto& o : trg::g_prof_open) (void)hipEventDestroy(o.second);
  trg::g_prof_done.clear();
  trg::g_prof_open.clear();
  return ok();
}

moe_status_t moe_prof_query(const char* name, int* count, float* total_ms) {
  if (!name || !count || !total_ms) return fail(MOE_ERR_INVALID_ARG, "moe_prof_query: null argument");
  std::lock_guard<std::mutex> lk(trg::g_prof_mu);
  int n = 0;
  float tot = 0.f;
  for (auto& r : trg::g_prof_done) {
    if (r.name != name) continue;
    if (hipEventSynchronize(r.e) != hipSuccess) return fail(MOE_ERR_HIP, "moe_prof_query: event wait failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.b, r.e) != hipSuccess) return fail(MOE_ERR_HIP, "moe_prof_query: elapsed failed");
    tot += ms;
    ++n;
  }
  *count = n;
  *total_ms = tot;
  return ok();
}

size_t moe_prof_names(char* buf, size_t n) {
  std::lock_guard<std::mutex> lk(trg::g_prof_mu);
  std::string all;
  for (auto& r : trg::g_prof_done) {
    std::string key = r.name + "\n";
    if (all.find(key) == std::string::npos && ("\n" + all).find("\n" + key) == std::string::npos) all += key;
  }
  if (buf && n > 0) {
    size_t m = all.size() < n - 1 ? all.size() : n - 1;
    memcpy(buf, all.data(), m);
    buf[m] = 0;
  }
  return all.size() + 1;
}

moe_status_t moe_router_logits(const void* x, int dt, const void* wr, int T, int d, int E, float* logits,
                               void* stream) {
  const char* fn = "moe_router_logits";
  TRY(check_dt(fn, dt));
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "%s: T must be >= 0", fn);
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  TRY(check_row(fn, "d", d, dt));
  if (!(dt == MOE_BF16 && E >= 64 && E % 8 == 0) && E > 64)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E > 64 needs bf16 storage and E %% 8 == 0", fn);
  TRY(check_ptrs(fn, {{"x", x}, {"wr", wr}, {"logits", logits}}));
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_router_logits(x, dt == MOE_BF16, wr, T, d, E, logits, (hipStream_t)stream));
}

size_t moe_route_workspace_size(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  return trg::route_ws_bytes(T, E, k);
}

moe_status_t moe_route(const float* logits, int T, int E, int k, const int32_t* forced_idx, float* probs,
                       int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* pos,
                       int32_t* src, int32_t* off128, int32_t* err_flag, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_route";
  TRY(check_tk(fn, T, k));
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k (%d) > E (%d)", fn, k, E);
  if (T > 0)
    TRY(check_ptrs(fn, {{"logits", logits}, {"probs", probs}, {"topk_idx", topk_idx}, {"topk_w", topk_w},
                        {"pos", pos}, {"src", src}}));
  TRY(check_ptrs(fn, {{"counts", counts}, {"offsets", offsets}}));
  const size_t need = trg::route_ws_bytes(T, E, k);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_route(logits, T, E, k, forced_idx, probs, topk_idx, topk_w, counts, offsets, pos,
                                          src, off128, err_flag, ws, (hipStream_t)stream));
}

moe_status_t moe_route_noalloc(const float* logits, int T, int E, int k, const int32_t* forced_idx, float* probs,
                               int32_t* topk_idx, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* pos,
                               int32_t* src, int32_t* off128, int32_t* err_flag, void* stream) {
  const char* fn = "moe_route_noalloc";
  TRY(check_tk(fn, T, k));
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k (%d) > E (%d)", fn, k, E);
  const size_t need = trg::route_ws_bytes(T, E, k);
  if (need > trg::kRouteScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "%s: this routing needs %zu bytes of scratch (ceil(T*k/256) * E * 4), more than the %zu the library "
                "holds; use moe_route with a workspace",
                fn, need, trg::kRouteScratchBytes);
  if (T > 0)
    TRY(check_ptrs(fn, {{"logits", logits}, {"probs", probs}, {"topk_idx", topk_idx}, {"topk_w", topk_w},
                        {"pos", pos}, {"src", src}}));
  TRY(check_ptrs(fn, {{"counts", counts}, {"offsets", offsets}}));
  TRY(check_device());
  void* scratch = nullptr;
  const hipError_t err = trg::route_scratch(&scratch);
  if (err != hipSuccess) return fail(MOE_ERR_HIP, "%s: scratch address: %s", fn, hipGetErrorString(err));
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_route(logits, T, E, k, forced_idx, probs, topk_idx, topk_w, counts, offsets, pos,
                                          src, off128, err_flag, scratch, (hipStream_t)stream));
}

moe_status_t moe_permute(const void* x, int dt, int T, int d, int k, const int32_t* pos, void* xp, void* stream) {
  const char* fn = "moe_permute";
  TRY(check_dt(fn, dt));
  TRY(check_tk(fn, T, k));
  TRY(check_row(fn, "d", d, dt));
  if (T == 0) return ok();
  TRY(check_ptrs(fn, {{"x", x}, {"pos", pos}, {"xp", xp}}));
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_permute(x, dt == MOE_BF16, T, d, k, pos, xp, (hipStream_t)stream));
}

moe_status_t moe_combine(const void* yp, const float* topk_w, const int32_t* pos, int T, int d, int k, int dt,
                         void* y, void* stream) {
  const char* fn = "moe_combine";
  TRY(check_dt(fn, dt));
  TRY(check_tk(fn, T, k));
  TRY(check_row(fn, "d", d, dt));
  if (T == 0) return ok();
  TRY(check_ptrs(fn, {{"yp", yp}, {"topk_w", topk_w}, {"pos", pos}, {"y", y}}));
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_gather_sum(yp, topk_w, pos, T, d, k, dt == MOE_BF16, y, (hipStream_t)stream));
}

moe_status_t moe_combine_bwd(const void* dy, const void* yp, const float* topk_w, const int32_t* pos, int T, int d,
                             int k, int dt, void* dyp, float* dgate, void* stream) {
  const char* fn = "moe_combine_bwd";
  TRY(check_dt(fn, dt));
  TRY(check_tk(fn, T, k));
  TRY(check_row(fn, "d", d, dt));
  if (T == 0) return ok();
  TRY(check_ptrs(fn, {{"dy", dy}, {"yp", yp}, {"topk_w", topk_w}, {"pos", pos}, {"dgate", dgate}}));
  TRY(check_optional_aligned(fn, {{"dyp", dyp}}));
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_combine_bwd(dy, yp, topk_w, pos, T, d, k, dt == MOE_BF16, dyp, dgate,
                                                (hipStream_t)stream));
}

moe_status_t moe_unpermute_sum(const void* dxp, const int32_t* pos, int T, int d, int k, int dt, void* dx,
                               void* stream) {
  const char* fn = "moe_unpermute_sum";
  TRY(check_dt(fn, dt));
  TRY(check_tk(fn, T, k));
  TRY(check_row(fn, "d", d, dt));
  if (T == 0) return ok();
  TRY(check_ptrs(fn, {{"dxp", dxp}, {"pos", pos}, {"dx", dx}}));
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_gather_sum(dxp, nullptr, pos, T, d, k, dt == MOE_BF16, dx, (hipStream_t)stream));
}

static moe_status_t check_ggemm_dims(const char* fn, int E, int R, int d, int h, int dt) {
  TRY(check_dt(fn, dt));
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (R < 0) return fail(MOE_ERR_INVALID_ARG, "%s: R must be >= 0", fn);
  TRY(check_row(fn, "d", d, dt));
  TRY(check_row(fn, "h", h, dt));
  if (dt == MOE_BF16 && (h % 64 != 0 || d % 64 != 0))
    return fail(MOE_ERR_INVALID_ARG, "%s: bf16 path needs d %% 64 == 0 and h %% 64 == 0", fn);
  // operand byte offsets inside one grouped GEMM are 32-bit
  const long widest = 2L * h > d ? 2L * h : (long)d;
  if ((long)R * widest * esize(dt) >= (1L << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: R * max(d, 2h) * element size must be < 2^31 bytes", fn);
  return MOE_OK;
}

size_t moe_grouped_gemm_workspace_size(int E, int R, int d, int h) {
  if (E < 1) return 0;
  return trg::ggemm_ws_bytes(E, R, d, h);
}

moe_status_t moe_grouped_gemm_fwd(const void* xp, const void* w1, const void* w3, const void* w2,
                                  const int32_t* offsets, int E, int R, int d, int h, int dt, void* g, void* u,
                                  void* hbuf, void* yp, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_gemm_fwd";
  TRY(check_ggemm_dims(fn, E, R, d, h, dt));
  TRY(check_ptrs(fn, {{"w1", w1}, {"w3", w3}, {"w2", w2}, {"offsets", offsets}}));
  if ((g == nullptr || u == nullptr) && dt != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "%s: the memory-lean forward (g or u null) needs bf16", fn);
  if (R == 0) return ok();
  TRY(check_ptrs(fn, {{"xp", xp}, {"hbuf", hbuf}, {"yp", yp}}));
  TRY(check_optional_aligned(fn, {{"g", g}, {"u", u}}));
  const size_t need = trg::ggemm_ws_bytes(E, R, d, h);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_fwd(xp, w1, w3, w2, offsets, E, R, d, h, dt == MOE_BF16, g, u, hbuf, yp, ws,
                                              (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm_recompute_gu(const void* xp, const void* w1, const void* w3, const int32_t* offsets,
                                           int E, int R, int d, int h, int dt, void* g, void* u, void* ws,
                                           size_t ws_bytes, void* stream) {
  const char* fn = "moe_grouped_gemm_recompute_gu";
  TRY(check_ggemm_dims(fn, E, R, d, h, dt));
  if (dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: needs bf16", fn);
  TRY(check_ptrs(fn, {{"w1", w1}, {"w3", w3}, {"offsets", offsets}}));
  if (R == 0) return ok();
  TRY(check_ptrs(fn, {{"xp", xp}, {"g", g}, {"u", u}}));
  const size_t need = trg::ggemm_ws_bytes(E, R, d, h);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_recompute_gu(xp, w1, w3, offsets, E, R, d, h, g, u, ws, (hipStream_t)stream));
}

static moe_status_t ggemm_bwd_impl(const char* fn, const void* dyp, const void* xp, const void* g, const void* u,
                                   const void* hbuf, const void* w1, const void* w3, const void* w2,
                                   const int32_t* offsets, int E, int R, int d, int h, int dt, void* dgu, void* dxp,
                                   void* dw1, void* dw3, void* dw2, unsigned parts, void* ws, size_t ws_bytes,
                                   void* stream) {
  TRY(check_ggemm_dims(fn, E, R, d, h, dt));
  if (parts == 0 || (parts & ~(unsigned)MOE_BWD_ALL) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: parts must be a non-empty subset of MOE_BWD_ALL", fn);
  if (dt != MOE_BF16 && parts != MOE_BWD_ALL)
    return fail(MOE_ERR_UNSUPPORTED, "%s: a subset of the backward GEMMs needs bf16", fn);
  TRY(check_ptrs(fn, {{"w1", w1}, {"w3", w3}, {"w2", w2}, {"offsets", offsets}, {"dw1", dw1}, {"dw3", dw3},
                      {"dw2", dw2}}));
  if (R > 0)
    TRY(check_ptrs(fn, {{"dyp", dyp}, {"xp", xp}, {"g", g}, {"u", u}, {"hbuf", hbuf}, {"dgu", dgu}, {"dxp", dxp}}));
  const size_t need = trg::ggemm_ws_bytes(E, R, d, h);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_bwd(dyp, xp, g, u, hbuf, w1, w3, w2, offsets, E, R, d, h, dt == MOE_BF16,
                                              dgu, dxp, dw1, dw3, dw2, ws, parts, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm_bwd(const void* dyp, const void* xp, const void* g, const void* u, const void* hbuf,
                                  const void* w1, const void* w3, const void* w2, const int32_t* offsets, int E, int R,
                                  int d, int h, int dt, void* dgu, void* dxp, void* dw1, void* dw3, void* dw2,
                                  void* ws, size_t ws_bytes, void* stream) {
  return ggemm_bwd_impl("moe_grouped_gemm_bwd", dyp, xp, g, u, hbuf, w1, w3, w2, offsets, E, R, d, h, dt, dgu, dxp,
                        dw1, dw3, dw2, MOE_BWD_ALL, ws, ws_bytes, stream);
}

moe_status_t moe_grouped_gemm_bwd_parts(const void* dyp, const void* xp, const void* g, const void* u,
                                        const void* hbuf, const void* w1, const void* w3, const void* w2,
                                        const int32_t* offsets, int E, int R, int d, int h, int dt, void* dgu,
                                        void* dxp, void* dw1, void* dw3, void* dw2, unsigned parts, void* ws,
                                        size_t ws_bytes, void* stream) {
  return ggemm_bwd_impl("moe_grouped_gemm_bwd_parts", dyp, xp, g, u, hbuf, w1, w3, w2, offsets, E, R, d, h, dt, dgu,
                        dxp, dw1, dw3, dw2, parts, ws, ws_bytes, stream);
}

size_t moe_router_bwd_workspace_size(int T, int d, int E) {
  if (T < 0 || d < 1 || E < 1) return 0;
  return trg::router_bwd_ws_bytes(T, d, E);
}

static moe_status_t router_bwd_impl(const char* fn, const float* probs, const int32_t* topk_idx, const float* dgate,
                                    const float* aux_g, const void* x, const void* wr, int T, int d, int E, int k,
                                    int dt, void* dx, void* dwr, void* ws, size_t ws_bytes, void* stream,
                                    const void* dxp = nullptr, const int32_t* pos = nullptr, bool fused = false,
                                    unsigned parts = MOE_ROUTER_DWR | MOE_ROUTER_DX) {
  TRY(check_dt(fn, dt));
  TRY(check_tk(fn, T, k));
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k (%d) > E (%d)", fn, k, E);
  TRY(check_row(fn, "d", d, dt));
  if (!(dt == MOE_BF16 && E >= 64 && E % 8 == 0) && E > 64)
    return fail(MOE_ERR_UNSUPPORTED, "%s: E > 64 needs bf16 storage and E %% 8 == 0", fn);
  if (parts == 0 || (parts & ~(unsigned)(MOE_ROUTER_DWR | MOE_ROUTER_DX)) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: parts must be a non-empty subset of MOE_ROUTER_DWR | MOE_ROUTER_DX", fn);
  const bool p_dwr = parts & MOE_ROUTER_DWR, p_dx = parts & MOE_ROUTER_DX;
  if (p_dwr) TRY(check_ptrs(fn, {{"dwr", dwr}}));
  if (T > 0) {
    TRY(check_ptrs(fn, {{"probs", probs}, {"topk_idx", topk_idx}, {"dgate", dgate}}));
    if (p_dwr) TRY(check_ptrs(fn, {{"x", x}}));
    if (p_dx) TRY(check_ptrs(fn, {{"wr", wr}, {"dx", dx}}));
    if (fused && p_dx) TRY(check_ptrs(fn, {{"dxp", dxp}, {"pos", pos}}));
  }
  const size_t need = trg::router_bwd_ws_bytes(T, d, E);
  if (ws == nullptr || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (!aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_router_bwd(probs, topk_idx, dgate, aux_g, x, wr, T, d, E, k, dt == MOE_BF16, dx,
                                               dwr, ws, (hipStream_t)stream, fused ? dxp : nullptr, pos, parts));
}

moe_status_t moe_router_bwd_unpermute(const float* probs, const int32_t* topk_idx, const float* dgate,
                                      const float* aux_g, const void* x, const void* wr, const void* dxp,
                                      const int32_t* pos, int T, int d, int E, int k, int dt, void* dx, void* dwr,
                                      void* ws, size_t ws_bytes, void* stream) {
  return router_bwd_impl("moe_router_bwd_unpermute", probs, topk_idx, dgate, aux_g, x, wr, T, d, E, k, dt, dx, dwr,
                         ws, ws_bytes, stream, dxp, pos, true);
}

moe_status_t moe_router_bwd_unpermute_parts(const float* probs, const int32_t* topk_idx, const float* dgate,
                                            const float* aux_g, const void* x, const void* wr, const void* dxp,
                                            const int32_t* pos, int T, int d, int E, int k, int dt, void* dx,
                                            void* dwr, void* ws, size_t ws_bytes, unsigned parts, void* stream) {
  return router_bwd_impl("moe_router_bwd_unpermute_parts", probs, topk_idx, dgate, aux_g, x, wr, T, d, E, k, dt, dx,
                         dwr, ws, ws_bytes, stream, dxp, pos, true, parts);
}

moe_status_t moe_router_bwd(const float* probs, const int32_t* topk_idx, const float* dgate, const void* x,
                            const void* wr, int T, int d, int E, int k, int dt, void* dx, void* dwr, void* ws,
                            size_t ws_bytes, void* stream) {
  return router_bwd_impl("moe_router_bwd", probs, topk_idx, dgate, nullptr, x, wr, T, d, E, k, dt, dx, dwr, ws,
                         ws_bytes, stream);
}

moe_status_t moe_router_bwd_aux(const float* probs, const int32_t* topk_idx, const float* dgate, const float* aux_g,
                                const void* x, const void* wr, int T, int d, int E, int k, int dt, void* dx, void* dwr,
                                void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_router_bwd_aux";
  if (T > 0) TRY(check_ptrs(fn, {{"aux_g", aux_g}}));
  return router_bwd_impl(fn, probs, topk_idx, dgate, aux_g, x, wr, T, d, E, k, dt, dx, dwr, ws, ws_bytes, stream);
}

size_t moe_balance_workspace_size(int T, int E) {
  if (T < 0 || E < 1) return 0;
  return trg::balance_ws_bytes(T, E);
}

moe_status_t moe_balance(const float* probs, const int32_t* counts, int T, int E, int k, float alpha, float* stats,
                         float* aux_g, float* mean_probs, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "moe_balance";
  TRY(check_tk(fn, T, k));
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (k > E) return fail(MOE_ERR_INVALID_ARG, "%s: k (%d) > E (%d)", fn, k, E);
  if (!(alpha >= 0.0f) || alpha > 1e30f) return fail(MOE_ERR_INVALID_ARG, "%s: alpha must be finite and >= 0", fn);
  TRY(check_ptrs(fn, {{"counts", counts}, {"stats", stats}}));
  if (T > 0) TRY(check_ptrs(fn, {{"probs", probs}}));
  const size_t need = trg::balance_ws_bytes(T, E);
  if (ws == nullptr || ws_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_balance(probs, counts, T, E, k, alpha, stats, aux_g, mean_probs, ws,
                                            (hipStream_t)stream));
}

moe_status_t mx_quantize(const void* in, int dt, int rows, int cols, const int32_t* gather_src, int gather_k,
                         const int32_t* seg_off, const int32_t* seg_off128, int nseg, int seg_rows, uint8_t* q_row,
                         uint8_t* s_row, uint8_t* q_col, uint8_t* s_col, int ldc, void* stream) {
  const char* fn = "mx_quantize";
  TRY(check_dt(fn, dt));
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "%s: rows must be >= 0", fn);
  if (cols <= 0 || cols % 32 != 0) return fail(MOE_ERR_INVALID_ARG, "%s: cols must be a positive multiple of 32", fn);
  if (!q_row && !q_col) return fail(MOE_ERR_INVALID_ARG, "%s: nothing to write (q_row and q_col are null)", fn);
  if ((q_row == nullptr) != (s_row == nullptr)) return fail(MOE_ERR_INVALID_ARG, "%s: q_row and s_row go together", fn);
  if ((q_col == nullptr) != (s_col == nullptr)) return fail(MOE_ERR_INVALID_ARG, "%s: q_col and s_col go together", fn);
  if (gather_src && gather_k < 1) return fail(MOE_ERR_INVALID_ARG, "%s: gather_k must be >= 1", fn);
  long padded, col_rows;  // padded rows in all; rows one columnwise row holds
  if (seg_off) {
    if (!seg_off128) return fail(MOE_ERR_INVALID_ARG, "%s: seg_off128 is required with seg_off", fn);
    if (nseg < 1 || nseg > 65536) return fail(MOE_ERR_INVALID_ARG, "%s: nseg must be in [1, 65536]", fn);
    padded = ((long)rows + 127L * nseg + 31) / 32 * 32;
    col_rows = (long)rows + 127L * nseg;
  } else {
    if (seg_rows < 1 || (seg_rows != rows && (seg_rows % 32 != 0 || rows % seg_rows != 0)))
      return fail(MOE_ERR_INVALID_ARG, "%s: seg_rows must equal rows, or be a multiple of 32 dividing rows", fn);
    const long seg32 = ((long)seg_rows + 31) / 32 * 32;
    padded = rows == 0 ? 0 : ((long)rows + seg_rows - 1) / seg_rows * seg32;
    col_rows = seg32;  // expert-major: one segment per columnwise row
  }
  if (q_col && (ldc % 32 != 0 || ldc < col_rows))
    return fail(MOE_ERR_INVALID_ARG, "%s: ldc must be a multiple of 32 and cover the padded rows", fn);
  if (padded >= (1L << 31) || (long)rows * cols >= (1L << 31) * 16L)
    return fail(MOE_ERR_UNSUPPORTED, "%s: problem too large", fn);
  if (rows == 0) return ok();
  TRY(check_ptrs(fn, {{"in", in}}));
  for (auto p : {std::make_pair("q_row", (const void*)q_row), std::make_pair("q_col", (const void*)q_col)})
    if (p.second && !aligned16(p.second)) return fail(MOE_ERR_ALIGNMENT, "%s: %s is not 16-byte aligned", fn, p.first);
  TRY(check_device());
  trg::ProfScope ps(fn, (hipStream_t)stream);
  return hip_status(fn, trg::launch_mx_quantize(in, dt == MOE_BF16, cols, rows, cols, gather_src, gather_k, seg_off,
                                                seg_off128, nseg, seg_rows, (int)(padded / 32), q_row, s_row, q_col,
                                                s_col, ldc, (hipStream_t)stream));
}

static moe_status_t check_mx_dims(const char* fn, int E, int R, int d, int h, int rcap, const void* ws,
                                  size_t ws_bytes) {
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID_ARG, "%s: E must be in [1, 1024]", fn);
  if (R < 0) return fail(MOE_ERR_INVALID_ARG, "%s: R must be >= 0", fn);
  if (d <= 0 || h <= 0 || d % 128 != 0 || h % 128 != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: d and h must be positive multiples of 128", fn);
  if (rcap % 128 != 0 || (long)rcap < (long)R + 127L * E)
    return fail(MOE_ERR_INVALID_ARG, "%s: rcap must be a multiple of 128 and >= R + 127*E", fn);
  const long widest = 2L * h > d ? 2L * h : (long)d;
  if ((long)R * widest * 2 >= (1L << 31) || (long)widest * rcap >= (1L << 31))
    return fail(MOE_ERR_UNSUPPORTED, "%s: operands larger than 2^31 bytes", fn);
  const size_t need = trg::ggemm_ws_bytes(E, R, d, h);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, ws_bytes);
  if (ws && !aligned16(ws)) return fail(MOE_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  return MOE_OK;
}

static moe_status_t ggemm_fwd_mx_impl(const char* fn, const moe_mx_fwd_args* a, unsigned parts, void* stream) {
  if (!a) return fail(MOE_ERR_INVALID_ARG, "%s: args is null", fn);
  if (parts == 0 || (parts & ~(unsigned)MOE_FWD_ALL) != 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: parts must be a non-empty subset of MOE_FWD_ALL", fn);
  TRY(check_mx_dims(fn, a->E, a->R, a->d, a->h, a->rcap, a->ws, a->ws_bytes));
  TRY(check_ptrs(fn, {{"offsets", a->offsets}, {"off128", a->off128}, {"w1q", a->w1q}, {"w1s", a->w1s},
                      {"w3q", a->w3q}, {"w3s", a->w3s}, {"w2q", a->w2q}, {"w2s", a->w2s}}));
  if (a->R == 0) return ok();
  TRY(check_ptrs(fn, {{"xq", a->xq}, {"xs", a->xs}, {"hbuf", a->hbuf}, {"hq", a->hq}, {"hs", a->hs},
                      {"hqT", a->hqT}, {"hsT", a->hsT}, {"yp", a->yp}}));
  TRY(check_optional_aligned(fn, {{"g", a->g}, {"u", a->u}}));
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_fwd_mx(*a, parts, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm_fwd_mx(const moe_mx_fwd_args* a, void* stream) {
  return ggemm_fwd_mx_impl("moe_grouped_gemm_fwd_mx", a, MOE_FWD_ALL, stream);
}

moe_status_t moe_grouped_gemm_fwd_mx_parts(const moe_mx_fwd_args* a, unsigned parts, void* stream) {
  return ggemm_fwd_mx_impl("moe_grouped_gemm_fwd_mx_parts", a, parts, stream);
}

moe_status_t moe_grouped_gemm_recompute_gu_mx(const moe_mx_fwd_args* a, void* stream) {
  const char* fn = "moe_grouped_gemm_recompute_gu_mx";
  if (!a) return fail(MOE_ERR_INVALID_ARG, "%s: args is null", fn);
  TRY(check_mx_dims(fn, a->E, a->R, a->d, a->h, a->rcap, a->ws, a->ws_bytes));
  TRY(check_ptrs(fn, {{"offsets", a->offsets}, {"w1q", a->w1q}, {"w1s", a->w1s}, {"w3q", a->w3q}, {"w3s", a->w3s}}));
  if (a->R == 0) return ok();
  TRY(check_ptrs(fn, {{"xq", a->xq}, {"xs", a->xs}, {"g", a->g}, {"u", a->u}}));
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_recompute_gu_mx(*a, (hipStream_t)stream));
}

static moe_status_t ggemm_bwd_mx_impl(const char* fn, const moe_mx_bwd_args* a, unsigned parts, void* stream) {
  if (!a) return fail(MOE_ERR_INVALID_ARG, "%s: args is null", fn);
  const unsigned mx_all = MOE_BWD_ALL | MOE_BWD_MX_QUANT_DY | MOE_BWD_MX_DY_READY;
  if ((parts & ~mx_all) != 0 || (parts & (MOE_BWD_ALL | MOE_BWD_MX_QUANT_DY)) == 0)
    return fail(MOE_ERR_INVALID_ARG, "%s: parts must be a non-empty subset of MOE_BWD_ALL | MOE_BWD_MX_QUANT_DY "
                "(with MOE_BWD_MX_DY_READY only beside MOE_BWD_DGRAD_DOWN)", fn);
  if ((parts & MOE_BWD_MX_DY_READY) && (!(parts & MOE_BWD_DGRAD_DOWN) || (parts & MOE_BWD_MX_QUANT_DY)))
    return fail(MOE_ERR_INVALID_ARG, "%s: MOE_BWD_MX_DY_READY goes with MOE_BWD_DGRAD_DOWN and without "
                "MOE_BWD_MX_QUANT_DY", fn);
  TRY(check_mx_dims(fn, a->E, a->R, a->d, a->h, a->rcap, a->ws, a->ws_bytes));
  TRY(check_ptrs(fn, {{"offsets", a->offsets}, {"off128", a->off128}, {"w1tq", a->w1tq}, {"w1ts", a->w1ts},
                      {"w3tq", a->w3tq}, {"w3ts", a->w3ts}, {"w2tq", a->w2tq}, {"w2ts", a->w2ts}, {"dw1", a->dw1},
                      {"dw3", a->dw3}, {"dw2", a->dw2}}));
  TRY(check_ptrs(fn, {{"dyq", a->dyq}, {"dys", a->dys}, {"dyqT", a->dyqT}, {"dysT", a->dysT}, {"hqT", a->hqT},
                      {"hsT", a->hsT}, {"xqT", a->xqT}, {"xsT", a->xsT}, {"dguqT", a->dguqT}, {"dgusT", a->dgusT}}));
  if (a->R > 0) {
    TRY(check_ptrs(fn, {{"g", a->g}, {"u", a->u}, {"dgu", a->dgu}, {"dguq", a->dguq}, {"dgus", a->dgus},
                        {"dxp", a->dxp}}));
    if (a->dyp == nullptr) {  // dYp's MX copies from dy, topk_w and src
      TRY(check_ptrs(fn, {{"dy", a->dy}, {"topk_w", a->topk_w}, {"src", a->src}}));
      if (a->k < 1 || a->k > 32 || a->R % a->k != 0)
        return fail(MOE_ERR_INVALID_ARG, "%s: k must be in [1, 32] and divide R when dyp is null", fn);
    } else {
      TRY(check_ptrs(fn, {{"dyp", a->dyp}}));
    }
  }
  TRY(check_device());
  return hip_status(fn, trg::launch_ggemm_bwd_mx(*a, parts, (hipStream_t)stream));
}

moe_status_t moe_grouped_gemm_bwd_mx(const moe_mx_bwd_args* a, void* stream) {
  return ggemm_bwd_mx_impl("moe_grouped_gemm_bwd_mx", a, MOE_BWD_ALL, stream);
}

moe_status_t moe_grouped_gemm_bwd_mx_parts(const moe_mx_bwd_args* a, unsigned parts, void* stream) {
  return ggemm_bwd_mx_impl("moe_grouped_gemm_bwd_mx_parts", a, parts, stream);
}

}  // extern "C"
