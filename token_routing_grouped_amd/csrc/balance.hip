// Router balance step: the auxiliary load-balance loss and a report of the
// routing balance score against the actual expert load.
//
// The pages point out that a routing balance score can improve while the
// actual workload balance gets worse (token gerrymandering: Olmo-core 3
// overview, "Empirical findings beyond raw speed"); they define neither.  The
// reading taken:
//   f_e = counts[e] / (T k),  P_e = (1/T) sum_t probs[t, e]
//   score = E sum_e f_e P_e,   loss = alpha score,
//   actual = max_e counts[e] / (T k / E)
//   g_e = d loss / d probs[t, e] = alpha E f_e / T   (same for every token; the
//   router backward adds it to each token's gate-gradient row)
//
// Deterministic two-pass reduction: pass 1 sums fixed chunks of kBalChunk
// tokens per expert (a fixed tree inside each chunk), pass 2 adds the chunk
// sums in chunk order and forms the outputs.
#include "common.h"
#include "kernels.h"

namespace trg {

constexpr int kBalChunk = 256;  // tokens per partial sum

// Grid: (ceil(T / kBalChunk), ceil(E / 64)).  Block: 64 experts x 4 token
// lanes; lane group q sums tokens q, q+4, ... of the chunk, then the four
// partial sums are added in a fixed order.
__global__ __launch_bounds__(256) void balance_partial_kernel(const float* __restrict__ probs, int T, int E,
                                                              float* __restrict__ part) {
  __shared__ float acc[4][64];
  const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int e = blockIdx.y * 64 + el;
  const int t0 = blockIdx.x * kBalChunk, t1 = min(T, t0 + kBalChunk);
  float s = 0.f;
  if (e < E)
    for (int t = t0 + q; t < t1; t += 4) s += probs[(long)t * E + e];
  acc[q][el] = s;
  __syncthreads();
  if (q == 0 && e < E) part[(long)blockIdx.x * E + e] = (acc[0][el] + acc[1][el]) + (acc[2][el] + acc[3][el]);
}

// One block of up to 1024 threads, one expert per thread (E <= 1024).
//   stats[0] = score, stats[1] = loss, stats[2] = max / mean load,
//   stats[3] = min / mean load
__global__ __launch_bounds__(1024) void balance_final_kernel(const float* __restrict__ part, int nchunk,
                                                             const int* __restrict__ counts, int T, int E, int k,
                                                             float alpha, float* __restrict__ stats,
                                                             float* __restrict__ aux_g,
                                                             float* __restrict__ mean_probs) {
  __shared__ float fp[1024];
  __shared__ int cmax[1024], cmin[1024];
  const int e = threadIdx.x;
  float P = 0.f, f = 0.f;
  int c = 0;
  if (e < E) {
    for (int i = 0; i < nchunk; ++i) P += part[(long)i * E + e];
    P = T > 0 ? P / (float)T : 0.f;
    c = counts[e];
    f = T > 0 ? (float)c / ((float)T * (float)k) : 0.f;
    if (aux_g) aux_g[e] = T > 0 ? alpha * (float)E * f / (float)T : 0.f;
    if (mean_probs) mean_probs[e] = P;
  }
  fp[e] = e < E ? f * P : 0.f;
  cmax[e] = e < E ? c : INT_MIN;
  cmin[e] = e < E ? c : INT_MAX;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {  // fixed-order tree
    if (e < w) {
      fp[e] += fp[e + w];
      cmax[e] = max(cmax[e], cmax[e + w]);
      cmin[e] = min(cmin[e], cmin[e + w]);
    }
    __syncthreads();
  }
  if (e == 0) {
    const float score = (float)E * fp[0];
    const float mean = T > 0 ? (float)T * (float)k / (float)E : 0.f;
    stats[0] = score;
    stats[1] = alpha * score;
    stats[2] = mean > 0.f ? (float)cmax[0] / mean : 0.f;
    stats[3] = mean > 0.f ? (float)cmin[0] / mean : 0.f;
  }
}

size_t balance_ws_bytes(int T, int E) {
  const size_t nchunk = T > 0 ? (size_t)(T + kBalChunk - 1) / kBalChunk : 1;
  return nchunk * (size_t)E * sizeof(float);
}

hipError_t launch_balance(const float* probs, const int* counts, int T, int E, int k, float alpha, float* stats,
                          float* aux_g, float* mean_probs, void* ws, hipStream_t s) {
  float* part = (float*)ws;
  const int nchunk = T > 0 ? (T + kBalChunk - 1) / kBalChunk : 0;
  if (nchunk > 0) balance_partial_kernel<<<dim3(nchunk, (E + 63) / 64), 256, 0, s>>>(probs, T, E, part);
  balance_final_kernel<<<1, 1024, 0, s>>>(part, nchunk, counts, T, E, k, alpha, stats, aux_g, mean_probs);
  return hipGetLastError();
}

}  // namespace trg
