// Rowwise dispatch and its inverses: permute, combine (gate-weighted gather
// sum), unpermute-sum, and the combine backward.  All HBM-bound row moves in
// 16-byte vectors, one workgroup per token row: each x[t] is read once and
// written to its k expert rows (Olmo-core 3 overview, "Routing and compute
// optimisation": routed tokens go straight into the experts' input buffers).
#include "common.h"
#include "kernels.h"

namespace trg {

constexpr int kMaxK = 32;

template <class T>
__global__ __launch_bounds__(256) void permute_kernel(const T* __restrict__ x, int d, int k,
                                                      const int* __restrict__ pos, T* __restrict__ xp) {
  const int t = blockIdx.x;
  const int nv = d / Elt<T>::kVec;
  const uint4* xr = (const uint4*)(x + (long)t * d);
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    uint4 val = xr[v];
    for (int j = 0; j < k; ++j) {
      int p = pos[(long)t * k + j];
      ((uint4*)(xp + (long)p * d))[v] = val;
    }
  }
}

// y[t] = sum_j w[t,j] * yp[pos[t,j]] (w == nullptr: weights of one), fp32
// accumulation in slot order, one rounding.
// GATED: the combine (rows weighted by their gates); otherwise the
// unpermute-sum (plain sum).  Output rows use the default store policy: the
// non-temporal hint measured slower for the combine and, once the grouped
// GEMMs' schedule changed, no faster for the unpermute-sum (wide 87 -> 80 us
// without it).
template <class T, bool GATED>
__global__ __launch_bounds__(256) void gather_sum_kernel(const T* __restrict__ yp, const float* __restrict__ w,
                                                         const int* __restrict__ pos, int d, int k,
                                                         T* __restrict__ y) {
  constexpr int V = Elt<T>::kVec;
  const int t = blockIdx.x;
  const int nv = d / V;
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      int p = pos[(long)t * k + j];
      const float wj = GATED ? w[(long)t * k + j] : 1.0f;
      float f[V];
      unpack16<T>(((const uint4*)(yp + (long)p * d))[v], f);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(wj, f[i], acc[i]);
    }
    ((uint4*)(y + (long)t * d))[v] = pack16<T>(acc);
  }
}

// dyp[pos[t,j]] = w[t,j] * dy[t];  dgate[t,j] = <dy[t], yp[pos[t,j]]>.
template <class T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(const T* __restrict__ dy, const T* __restrict__ yp,
                                                          const float* __restrict__ w, const int* __restrict__ pos,
                                                          int d, int k, T* __restrict__ dyp,
                                                          float* __restrict__ dgate) {
  constexpr int V = Elt<T>::kVec;
  __shared__ float red[4][kMaxK];
  const int t = blockIdx.x;
  const int nv = d / V;
  float part[kMaxK];
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) part[j] = 0.f;
  for (int v = threadIdx.x; v < nv; v += blockDim.x) {
    float f[V];
    unpack16<T>(((const uint4*)(dy + (long)t * d))[v], f);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      if (j < k) {
        int p = pos[(long)t * k + j];
        float wj = w[(long)t * k + j];
        float o[V], g[V];
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = wj * f[i];
        if (dyp != nullptr) ((uint4*)(dyp + (long)p * d))[v] = pack16<T>(o);  // null: dgate only
        unpack16<T>(((const uint4*)(yp + (long)p * d))[v], g);
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < V; ++i) s = fmaf(f[i], g[i], s);
        part[j] += s;
      }
    }
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < kMaxK; ++j) {
    if (j < k) {
      float s = wave_sum(part[j]);
      if (lane == 0) red[wv][j] = s;
    }
  }
  __syncthreads();
  if (threadIdx.x < k) {
    int j = threadIdx.x;
    dgate[(long)t * k + j] = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
  }
}

hipError_t launch_permute(const void* x, bool bf16, int T, int d, int k, const int* pos, void* xp, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    permute_kernel<uint16_t><<<T, 256, 0, s>>>((const uint16_t*)x, d, k, pos, (uint16_t*)xp);
  else
    permute_kernel<float><<<T, 256, 0, s>>>((const float*)x, d, k, pos, (float*)xp);
  return hipGetLastError();
}

hipError_t launch_gather_sum(const void* yp, const float* w, const int* pos, int T, int d, int k, bool bf16,
                             void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const bool gated = w != nullptr;
  if (bf16) {
    if (gated) gather_sum_kernel<uint16_t, true><<<T, 256, 0, s>>>((const uint16_t*)yp, w, pos, d, k, (uint16_t*)y);
    else gather_sum_kernel<uint16_t, false><<<T, 256, 0, s>>>((const uint16_t*)yp, w, pos, d, k, (uint16_t*)y);
  } else {
    if (gated) gather_sum_kernel<float, true><<<T, 256, 0, s>>>((const float*)yp, w, pos, d, k, (float*)y);
    else gather_sum_kernel<float, false><<<T, 256, 0, s>>>((const float*)yp, w, pos, d, k, (float*)y);
  }
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void* dy, const void* yp, const float* w, const int* pos, int T, int d, int k,
                              bool bf16, void* dyp, float* dgate, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16)
    combine_bwd_kernel<uint16_t><<<T, 256, 0, s>>>((const uint16_t*)dy, (const uint16_t*)yp, w, pos, d, k,
                                                   (uint16_t*)dyp, dgate);
  else
    combine_bwd_kernel<float><<<T, 256, 0, s>>>((const float*)dy, (const float*)yp, w, pos, d, k, (float*)dyp,
                                                dgate);
  return hipGetLastError();
}

}  // namespace trg
