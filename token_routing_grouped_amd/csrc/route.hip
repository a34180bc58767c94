// GPU-resident routing: softmax / top-k, expert histogram, prefix sum and
// stable positions.  Nothing here leaves the device (Olmo-core 3 overview,
// "Routing and compute optimisation": routing metadata is kept on the GPU so
// the CPU never waits on it).
//
// Four launches, all deterministic (integer LDS atomics only, order-free):
//   route_topk   one wave per token: max, sum of exp, k rounds of wave argmax
//   route_count  one wave per chunk of 256 flattened (t, j) entries -> per-chunk
//                per-expert counts
//   route_scan   one workgroup: per-expert exclusive scan over chunks, counts,
//                offsets, off128
//   route_rank   one wave per chunk: rank of each entry among equal experts in
//                (token, slot) order via LDS match masks + popcount
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace trg {

constexpr int kChunk = 256;  // flattened (t, j) entries per rank/count chunk

// Lexicographic (value desc, index asc) comparison used for top-k.
TRG_DEV bool better(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }

template <int EPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int T, int E,
                                                         int k, const int* __restrict__ forced,
                                                         float* __restrict__ probs, int* __restrict__ idx_out,
                                                         float* __restrict__ w_out, int* __restrict__ err_flag) {
  const int lane = threadIdx.x & 63;
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;  // the whole wave leaves together
  const float* L = logits + (long)t * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    float x = e < E ? L[e] : -INFINITY;
    v[i] = (x != x) ? -INFINITY : x;  // NaN never wins a slot
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < EPL; ++i) m = fmaxf(m, v[i]);
  m = wave_max(m);
  float ex[EPL], s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    ex[i] = e < E ? expf(v[i] - m) : 0.f;
    s += ex[i];
  }
  s = wave_sum(s);
  float p[EPL];
  float* P = probs + (long)t * E;
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    int e = lane + 64 * i;
    p[i] = ex[i] / s;
    if (e < E) P[e] = p[i];
  }

  if (forced != nullptr) {
    // Given indices: validate, clamp into range, flag problems.
    int fe = lane < k ? forced[(long)t * k + lane] : 0;
    int flags = 0;
    if (lane < k && (fe < 0 || fe >= E)) {
      flags |= 1;
      fe = fe < 0 ? 0 : E - 1;
    }
    for (int j = 0; j < k; ++j) {
      int other = __shfl(fe, j, 64);
      if (lane < k && j < lane && other == fe) flags |= 2;
    }
    // gate = p of expert fe, owned by lane fe % 64, slot fe / 64
    float w = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      float c = __shfl(p[i], fe & 63, 64);
      if ((fe >> 6) == i) w = c;
    }
    if (lane < k) {
      idx_out[(long)t * k + lane] = fe;
      w_out[(long)t * k + lane] = w;
      if (flags && err_flag) atomicOr(err_flag, flags);
    }
    return;
  }

  unsigned chosen = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      int e = lane + 64 * i;
      if (e < E && !((chosen >> i) & 1u) && better(v[i], e, bv, be)) {
        bv = v[i];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oe = __shfl_xor(be, o, 64);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // be is now uniform across the wave
    float w = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if ((be >> 6) == i && (be & 63) == lane) chosen |= 1u << i;
      float c = __shfl(p[i], be & 63, 64);
      if ((be >> 6) == i) w = c;
    }
    if (lane == 0) {
      idx_out[(long)t * k + j] = be;
      w_out[(long)t * k + j] = w;
    }
  }
}

// The same for E <= LPT <= 32: a wave takes 64 / LPT tokens, LPT lanes each
// (lane sl of a token's group holds expert sl), so few experts do not leave
// most of a wave idle.  The shuffles stay inside a token's group.  The results
// are those of the one-token-per-wave kernel bit for bit: there the butterfly
// steps wider than LPT only combine with lanes holding no expert (max with
// -inf, sum with +0), and the remaining steps are these, in the same order;
// the arg-max is exact in any order.  A group past T runs on token T - 1's
// logits and writes nothing.
template <int LPT>
__global__ __launch_bounds__(256) void route_topk_packed_kernel(const float* __restrict__ logits, int T, int E,
                                                                int k, const int* __restrict__ forced,
                                                                float* __restrict__ probs, int* __restrict__ idx_out,
                                                                float* __restrict__ w_out, int* __restrict__ err_flag) {
  constexpr int TPW = 64 / LPT;  // tokens per wave
  const int lane = threadIdx.x & 63, sl = lane & (LPT - 1);
  const int t0 = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6) * TPW + lane / LPT;
  const bool valid = t0 < T;
  const int t = valid ? t0 : T - 1;
  const bool has_e = sl < E;
  float v = has_e ? logits[(long)t * E + sl] : -INFINITY;
  if (v != v) v = -INFINITY;  // NaN never wins a slot
  float m = v;
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, LPT));
  const float ex = has_e ? expf(v - m) : 0.f;
  float s = ex;
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, LPT);
  const float p = ex / s;
  if (valid && has_e) probs[(long)t * E + sl] = p;

  if (forced != nullptr) {
    int fe = sl < k ? forced[(long)t * k + sl] : 0;
    int flags = 0;
    if (sl < k && (fe < 0 || fe >= E)) {
      flags |= 1;
      fe = fe < 0 ? 0 : E - 1;
    }
    for (int j = 0; j < k; ++j) {
      const int other = __shfl(fe, j, LPT);
      if (sl < k && j < sl && other == fe) flags |= 2;
    }
    const float w = __shfl(p, fe, LPT);
    if (valid && sl < k) {
      idx_out[(long)t * k + sl] = fe;
      w_out[(long)t * k + sl] = w;
      if (flags && err_flag) atomicOr(err_flag, flags);
    }
    return;
  }

  bool chosen = false;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
    if (has_e && !chosen) {
      bv = v;
      be = sl;
    }
#pragma unroll
    for (int o = LPT / 2; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, LPT);
      const int oe = __shfl_xor(be, o, LPT);
      if (better(ov, oe, bv, be)) {
        bv = ov;
        be = oe;
      }
    }
    // be is now uniform across the token's group
    if (be == sl) chosen = true;
    const float w = __shfl(p, be & (LPT - 1), LPT);
    if (valid && sl == 0) {
      idx_out[(long)t * k + j] = be;
      w_out[(long)t * k + j] = w;
    }
  }
}

// Per-chunk expert histogram.  4 waves per block, one chunk per wave.
__global__ __launch_bounds__(256) void route_count_kernel(const int* __restrict__ idx, int R, int E, int nchunks,
                                                          int* __restrict__ chunk_cnt) {
  extern __shared__ int hist[];  // [4][E]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int chunk = blockIdx.x * 4 + w;
  int* hw = hist + w * E;
  for (int e = lane; e < E; e += 64) hw[e] = 0;
  __syncthreads();
  if (chunk < nchunks) {
#pragma unroll
    for (int r = 0; r < kChunk / 64; ++r) {
      long i = (long)chunk * kChunk + r * 64 + lane;
      if (i < R) atomicAdd(&hw[idx[i]], 1);
    }
  }
  __syncthreads();
  if (chunk < nchunks)
    for (int e = lane; e < E; e += 64) chunk_cnt[(long)chunk * E + e] = hw[e];
}

// One block of 1024 threads.  Thread (e, j) = tid / TPE, tid % TPE with TPE =
// 1024 / (E rounded up to a power of two) threads per expert owns a contiguous
// range of chunks of expert e.  Threads are ordered expert-major, so one
// exclusive block scan of the per-thread chunk sums gives every thread the
// absolute row of its first entry: the counts of all lower experts plus the
// same expert's earlier chunks.  A second scan over the experts' counts
// rounded up to 128 rows gives off128.  Finally each thread rewrites its chunks' counts as
// absolute starting rows.  Up to kScanReg chunks per thread are loaded at once
// and kept in registers for the rewrite (one round of loads in flight instead
// of a dependent round per 8 chunks, and no second read).
__global__ __launch_bounds__(1024) void route_scan_kernel(int* __restrict__ chunk_cnt, int nchunks, int E,
                                                          int* __restrict__ counts, int* __restrict__ offsets,
                                                          int* __restrict__ off128) {
  __shared__ int tmp[1024];
  __shared__ int off_s[1025];
  const int tid = threadIdx.x;
  int epow = 1;
  while (epow < E) epow <<= 1;
  const int tpe = 1024 / epow;
  const int e = tid / tpe, j = tid - e * tpe;
  const int per = (nchunks + tpe - 1) / tpe;
  const int cb = j * per, ce = min(nchunks, cb + per);
  const bool mine = e < E;
  constexpr int kScanReg = 64;
  const bool inreg = per <= kScanReg;  // uniform over the block
  int vr[kScanReg];
  int sum = 0;
  if (mine && inreg) {
#pragma unroll
    for (int u = 0; u < kScanReg; ++u) vr[u] = cb + u < ce ? chunk_cnt[(long)(cb + u) * E + e] : 0;
#pragma unroll
    for (int u = 0; u < kScanReg; ++u) sum += vr[u];
  } else if (mine) {
    int c = cb;
    for (; c + 8 <= ce; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = chunk_cnt[(long)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    for (; c < ce; ++c) sum += chunk_cnt[(long)c * E + e];
  }
  int total;
  const int base = block_excl_scan_1024(mine ? sum : 0, tmp, &total);
  if (mine && j == 0) off_s[e] = base;
  if (tid == 0) off_s[E] = total;
  __syncthreads();
  const int cnt_e = mine ? off_s[e + 1] - off_s[e] : 0;
  int total128;
  const int o128 = block_excl_scan_1024((mine && j == 0) ? (cnt_e + 127) & ~127 : 0, tmp, &total128);
  if (mine && j == 0) {
    counts[e] = cnt_e;
    offsets[e] = off_s[e];
    if (off128) off128[e] = o128;
  }
  if (tid == 0) {
    offsets[E] = total;
    if (off128) off128[E] = total128;
  }
  if (mine && inreg) {
    int run = base;
#pragma unroll
    for (int u = 0; u < kScanReg; ++u) {
      if (cb + u < ce) chunk_cnt[(long)(cb + u) * E + e] = run;
      run += vr[u];
    }
  } else if (mine) {
    int run = base;
    int c = cb;
    for (; c + 8 <= ce; c += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = chunk_cnt[(long)(c + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        chunk_cnt[(long)(c + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; c < ce; ++c) {
      const int v = chunk_cnt[(long)c * E + e];
      chunk_cnt[(long)c * E + e] = run;
      run += v;
    }
  }
}

// One wave per chunk.  Entries are visited in flattened (t, j) order, 64 at a
// time; the rank among equal experts is the popcount of the lower lanes in
// that expert's match mask, plus the running count carried between rounds.
__global__ __launch_bounds__(64) void route_rank_kernel(const int* __restrict__ idx, int R, int E,
                                                        const int* __restrict__ chunk_base, int* __restrict__ pos,
                                                        int* __restrict__ src) {
  extern __shared__ unsigned long long lds_rank[];  // masks [E] then run [E] (int)
  unsigned long long* mask = lds_rank;
  int* run = (int*)(lds_rank + E);
  const int lane = threadIdx.x;
  const int chunk = blockIdx.x;
  for (int e = lane; e < E; e += 64) {
    mask[e] = 0ull;
    run[e] = chunk_base[(long)chunk * E + e];
  }
  __syncthreads();
#pragma unroll 1
  for (int r = 0; r < kChunk / 64; ++r) {
    long i = (long)chunk * kChunk + r * 64 + lane;
    bool valid = i < R;
    int e = valid ? idx[i] : 0;
    if (valid) atomicOr(&mask[e], 1ull << lane);
    __syncthreads();
    unsigned long long mm = valid ? mask[e] : 0ull;
    int rank = __popcll(mm & ((1ull << lane) - 1ull));
    int p = valid ? run[e] + rank : 0;
    __syncthreads();
    if (valid && rank == 0) {
      run[e] += __popcll(mm);
      mask[e] = 0ull;
    }
    __syncthreads();
    if (valid) {
      pos[i] = p;
      src[p] = (int)i;
    }
  }
}

// ---- scratch for the entry point that allocates nothing (moe_route_noalloc)
// The per-chunk counts live in this file-scope device array instead of a
// caller workspace.  Every GPU that loads the library holds its own copy until
// the process ends; host code never uses the symbol itself (on the host it is
// only a stand-in), but the per-device address hipGetSymbolAddress returns.
static __device__ __align__(256) int scratch[kRouteScratchBytes / sizeof(int)];

namespace {
constexpr int kMaxScratchDev = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDev];  // device address of `scratch` per device, once resolved
}  // namespace

hipError_t route_scratch(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxScratchDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

size_t route_ws_bytes(int T, int E, int k) {
  long R = (long)T * k;
  long nchunks = (R + kChunk - 1) / kChunk;
  return (size_t)(nchunks * E * sizeof(int));
}

hipError_t launch_route(const float* logits, int T, int E, int k, const int* forced, float* probs, int* idx,
                        float* w, int* counts, int* offsets, int* pos, int* src, int* off128, int* err_flag,
                        void* ws, hipStream_t s) {
  long R = (long)T * k;
  int nchunks = (int)((R + kChunk - 1) / kChunk);
  int* chunk_cnt = (int*)ws;
  if (R == 0) {  // no tokens: counts and offsets are all zero
    route_scan_kernel<<<1, 1024, 0, s>>>(chunk_cnt, 0, E, counts, offsets, off128);
    return hipGetLastError();
  }
  dim3 g1((T + 3) / 4);
  if (E <= 8)
    route_topk_packed_kernel<8><<<(T + 31) / 32, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 16)
    route_topk_packed_kernel<16><<<(T + 15) / 16, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 32)
    route_topk_packed_kernel<32><<<(T + 7) / 8, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 64)
    route_topk_kernel<1><<<g1, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 128)
    route_topk_kernel<2><<<g1, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 256)
    route_topk_kernel<4><<<g1, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else if (E <= 512)
    route_topk_kernel<8><<<g1, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  else
    route_topk_kernel<16><<<g1, 256, 0, s>>>(logits, T, E, k, forced, probs, idx, w, err_flag);
  route_count_kernel<<<(nchunks + 3) / 4, 256, 4 * E * sizeof(int), s>>>(idx, (int)R, E, nchunks, chunk_cnt);
  route_scan_kernel<<<1, 1024, 0, s>>>(chunk_cnt, nchunks, E, counts, offsets, off128);
  route_rank_kernel<<<nchunks, 64, E * (sizeof(unsigned long long) + sizeof(int)), s>>>(idx, (int)R, E, chunk_cnt,
                                                                                        pos, src);
  return hipGetLastError();
}

}  // namespace trg
