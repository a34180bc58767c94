// fp32 grouped GEMMs for layers stored in float32 (small layers).  One thread
// per output element, fp32 accumulation in index order; the expert of a routed
// row is found by binary search in the offsets.  Same contracts as the bf16
// matrix-core path; throughput is not a goal here.
#include "common.h"
#include "kernels.h"

namespace trg {

// Last expert e with offsets[e] <= r (skips empty experts).
TRG_DEV int expert_of_row(const int* __restrict__ off, int E, int r) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void f32_up_kernel(const float* __restrict__ xp, const float* __restrict__ w1,
                              const float* __restrict__ w3, const int* __restrict__ off, int E, int R, int d, int h,
                              float* __restrict__ G, float* __restrict__ U, float* __restrict__ H) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * h) return;
  const int r = (int)(i / h), j = (int)(i % h);
  const int e = expert_of_row(off, E, r);
  const float* x = xp + (long)r * d;
  const float* a = w1 + ((long)e * h + j) * d;
  const float* b = w3 + ((long)e * h + j) * d;
  float g = 0.f, u = 0.f;
  for (int c = 0; c < d; ++c) {
    g = fmaf(x[c], a[c], g);
    u = fmaf(x[c], b[c], u);
  }
  G[i] = g;
  U[i] = u;
  H[i] = silu_f(g) * u;
}

__global__ void f32_down_kernel(const float* __restrict__ H, const float* __restrict__ w2,
                                const int* __restrict__ off, int E, int R, int d, int h, float* __restrict__ yp) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * d) return;
  const int r = (int)(i / d), c = (int)(i % d);
  const int e = expert_of_row(off, E, r);
  const float* hr = H + (long)r * h;
  const float* w = w2 + ((long)e * d + c) * h;
  float s = 0.f;
  for (int j = 0; j < h; ++j) s = fmaf(hr[j], w[j], s);
  yp[i] = s;
}

__global__ void f32_dgrad_down_kernel(const float* __restrict__ dyp, const float* __restrict__ w2,
                                      const float* __restrict__ G, const float* __restrict__ U,
                                      const int* __restrict__ off, int E, int R, int d, int h,
                                      float* __restrict__ dgu) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * h) return;
  const int r = (int)(i / h), j = (int)(i % h);
  const int e = expert_of_row(off, E, r);
  const float* dy = dyp + (long)r * d;
  const float* w = w2 + (long)e * d * h + j;
  float dh = 0.f;
  for (int c = 0; c < d; ++c) dh = fmaf(dy[c], w[(long)c * h], dh);
  const float g = G[i], u = U[i], s = sigmoid_f(g);
  dgu[(long)r * 2 * h + j] = dh * u * s * (1.0f + g * (1.0f - s));
  dgu[(long)r * 2 * h + h + j] = dh * g * s;
}

__global__ void f32_dgrad_up_kernel(const float* __restrict__ dgu, const float* __restrict__ w1,
                                    const float* __restrict__ w3, const int* __restrict__ off, int E, int R, int d,
                                    int h, float* __restrict__ dxp) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)R * d) return;
  const int r = (int)(i / d), c = (int)(i % d);
  const int e = expert_of_row(off, E, r);
  const float* dg = dgu + (long)r * 2 * h;
  const float* a = w1 + (long)e * h * d + c;
  const float* b = w3 + (long)e * h * d + c;
  float s = 0.f;
  for (int j = 0; j < h; ++j) s = fmaf(dg[j], a[(long)j * d], s);
  for (int j = 0; j < h; ++j) s = fmaf(dg[h + j], b[(long)j * d], s);
  dxp[i] = s;
}

__global__ void f32_wgrad_down_kernel(const float* __restrict__ dyp, const float* __restrict__ H,
                                      const int* __restrict__ off, int E, int d, int h, float* __restrict__ dw2) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)E * d * h) return;
  const int e = (int)(i / ((long)d * h));
  const int c = (int)((i / h) % d), j = (int)(i % h);
  float s = 0.f;
  for (int r = off[e]; r < off[e + 1]; ++r) s = fmaf(dyp[(long)r * d + c], H[(long)r * h + j], s);
  dw2[i] = s;
}

__global__ void f32_wgrad_up_kernel(const float* __restrict__ dgu, const float* __restrict__ xp,
                                    const int* __restrict__ off, int E, int d, int h, float* __restrict__ dw1,
                                    float* __restrict__ dw3) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)E * 2 * h * d) return;
  const int e = (int)(i / (2L * h * d));
  const int m = (int)((i / d) % (2 * h)), c = (int)(i % d);
  float s = 0.f;
  for (int r = off[e]; r < off[e + 1]; ++r) s = fmaf(dgu[(long)r * 2 * h + m], xp[(long)r * d + c], s);
  if (m < h)
    dw1[((long)e * h + m) * d + c] = s;
  else
    dw3[((long)e * h + (m - h)) * d + c] = s;
}

static inline unsigned blocks_for(long n) { return (unsigned)((n + 255) / 256); }

hipError_t launch_ggemm_fwd_f32(const float* xp, const float* w1, const float* w3, const float* w2,
                                const int* offsets, int E, int R, int d, int h, float* g, float* u, float* hb,
                                float* yp, hipStream_t s) {
  if (R == 0) return hipSuccess;
  f32_up_kernel<<<blocks_for((long)R * h), 256, 0, s>>>(xp, w1, w3, offsets, E, R, d, h, g, u, hb);
  f32_down_kernel<<<blocks_for((long)R * d), 256, 0, s>>>(hb, w2, offsets, E, R, d, h, yp);
  return hipGetLastError();
}

hipError_t launch_ggemm_bwd_f32(const float* dyp, const float* xp, const float* g, const float* u, const float* hb,
                                const float* w1, const float* w3, const float* w2, const int* offsets, int E, int R,
                                int d, int h, float* dgu, float* dxp, float* dw1, float* dw3, float* dw2,
                                hipStream_t s) {
  if (R > 0) {
    f32_dgrad_down_kernel<<<blocks_for((long)R * h), 256, 0, s>>>(dyp, w2, g, u, offsets, E, R, d, h, dgu);
    f32_dgrad_up_kernel<<<blocks_for((long)R * d), 256, 0, s>>>(dgu, w1, w3, offsets, E, R, d, h, dxp);
  }
  f32_wgrad_down_kernel<<<blocks_for((long)E * d * h), 256, 0, s>>>(dyp, hb, offsets, E, d, h, dw2);
  f32_wgrad_up_kernel<<<blocks_for((long)E * 2 * h * d), 256, 0, s>>>(dgu, xp, offsets, E, d, h, dw1, dw3);
  return hipGetLastError();
}

}  // namespace trg
