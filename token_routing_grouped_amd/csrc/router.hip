// Router GEMMs and the softmax backward.
//   logits = x Wr^T;  dlogits = p * (g - <p, g>);  dWr = dlogits^T x;
//   dx += dlogits Wr.
// For few experts (E < 64) these are skinny and HBM-bound on x, so they run on
// the vector ALUs: one wave per token row for the logits, column-parallel
// partial sums over token chunks (reduced in a fixed order) for dWr, and one
// workgroup per token row for dx.  For E >= 64 (bf16, E % 8 == 0) the three
// products are real GEMMs and go to the matrix-core kernels.
#include "common.h"
#include "kernels.h"

namespace trg {

template <class T, int EB>
__global__ __launch_bounds__(256) void router_logits_valu_kernel(const T* __restrict__ x, const T* __restrict__ wr,
                                                                 int Tn, int d, int E, float* __restrict__ logits) {
  constexpr int V = Elt<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= Tn) return;
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  const uint4* xr = (const uint4*)(x + (long)t * d);
  const int nv = d / V;
  for (int v = lane; v < nv; v += 64) {
    float f[V];
    unpack16<T>(xr[v], f);
    // Groups of 8 expert rows: the loads are issued unconditionally (row
    // index clamped to a valid row) so they are all in flight together; only
    // the FMAs depend on e < E.
#pragma unroll
    for (int e0 = 0; e0 < EB; e0 += 8) {
      if (e0 >= E) break;
      uint4 wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[q] = ((const uint4*)(wr + (long)min(e0 + q, E - 1) * d))[v];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (e0 + q < E) {
          float w[V];
          unpack16<T>(wv[q], w);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[e0 + q] = fmaf(f[i], w[i], acc[e0 + q]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if (e < E) {
      const float s = wave_sum(acc[e]);
      if (lane == 0) logits[(long)t * E + e] = s;
    }
  }
}

// Softmax backward through the gates.  One wave per token.
template <int EPL>
__global__ __launch_bounds__(256) void router_dl_kernel(const float* __restrict__ probs, const int* __restrict__ idx,
                                                        const float* __restrict__ dgate,
                                                        const float* __restrict__ aux_g, int Tn, int E, int k,
                                                        float* __restrict__ dL, uint16_t* __restrict__ dLb) {
  const int lane = threadIdx.x & 63;
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= Tn) return;
  float p[EPL], gh[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    p[i] = e < E ? probs[(long)t * E + e] : 0.f;
    gh[i] = 0.f;
  }
  // the balance loss's probability gradient (the same for every token), added
  // before the gates' own (disjoint slots are written below)
  float ga[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) ga[i] = (aux_g != nullptr && lane + 64 * i < E) ? aux_g[lane + 64 * i] : 0.f;
  for (int j = 0; j < k; ++j) {
    const int ej = idx[(long)t * k + j];
    const float gj = dgate[(long)t * k + j];
#pragma unroll
    for (int i = 0; i < EPL; ++i)
      if (lane + 64 * i == ej) gh[i] = gj;
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) gh[i] += ga[i];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < EPL; ++i) s = fmaf(p[i], gh[i], s);
  s = wave_sum(s);
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      const float v = p[i] * (gh[i] - s);
      dL[(long)t * E + e] = v;
      if (dLb) dLb[(long)t * E + e] = f2bf(v);
    }
  }
}

constexpr int kDwrChunk = 128;  // tokens per dWr partial sum

// dWr partial sums over one chunk of kDwrChunk tokens.  Thread layout: 32
// column groups of CV = 64/EB consecutive columns x 8 token lanes (the token
// lanes of a group are neighbouring lanes of one wave, reduced with shuffles),
// so each wave load covers whole 128-byte row pieces of x.  The op is bound by
// HBM, so a workgroup issues every load of its chunk (the chunk's dlogits and
// each thread's NT rows of x) before the first wait; with 128-token chunks a
// typical shape has several workgroups per CU in flight.
template <class T, int EB, bool ELEM>
__global__ __launch_bounds__(256) void router_dwr_partial_kernel(const float* __restrict__ dL, const T* __restrict__ x,
                                                                 int Tn, int d, int E, float* __restrict__ part) {
  constexpr int CV = 64 / EB;           // columns per thread; EB * CV = 64 accumulators
  constexpr int NT = kDwrChunk / 8;     // rows per thread
  struct alignas(CV * sizeof(T)) Vec { T v[CV]; };
  __shared__ float sdl[kDwrChunk][EB];
  const int tl = threadIdx.x & 7, cg = threadIdx.x >> 3;
  const int c0 = blockIdx.x * (32 * CV) + cg * CV;
  const int chunk = blockIdx.y;
  const int t0 = chunk * kDwrChunk;
  const int nt = min(kDwrChunk, Tn - t0);
  // Raw rows, converted at the FMAs.  No branch around the loads (a branch
  // makes the compiler wait for each load before the next is issued): rows
  // past the chunk and column groups past d load a valid address and are
  // zeroed by a select.  ELEM (a column group may straddle d: fp32 with
  // d % CV != 0) loads element by element instead.
  Vec xr[NT];
  if constexpr (!ELEM) {
    const bool col_ok = c0 + CV <= d;
    const int cl = col_ok ? c0 : 0;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int tt = tl + 8 * j;
      xr[j] = *(const Vec*)(x + (long)(t0 + min(tt, nt - 1)) * d + cl);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int tt = tl + 8 * j;
#pragma unroll
      for (int v = 0; v < CV; ++v) xr[j].v[v] = (tt < nt && c0 + v < d) ? x[(long)(t0 + tt) * d + c0 + v] : T(0);
    }
  }
  // dlogits of the chunk -> LDS (zero past the chunk's end and for e >= E;
  // loaded from a clamped valid index, then selected, again without a branch)
  float dv[kDwrChunk * EB / 256];
#pragma unroll
  for (int q = 0; q < kDwrChunk * EB / 256; ++q) {
    const int i = threadIdx.x + 256 * q, tt = i / EB, e = i % EB;
    dv[q] = dL[(long)(t0 + min(tt, nt - 1)) * E + min(e, E - 1)];
  }
#pragma unroll
  for (int q = 0; q < kDwrChunk * EB / 256; ++q) {
    const int i = threadIdx.x + 256 * q;
    if (!(i / EB < nt && i % EB < E)) dv[q] = 0.f;
  }
  if constexpr (!ELEM) {
    const bool col_ok = c0 + CV <= d;
#pragma unroll
    for (int j = 0; j < NT; ++j)
      if (!(col_ok && tl + 8 * j < nt))
#pragma unroll
        for (int v = 0; v < CV; ++v) xr[j].v[v] = T(0);
  }
#pragma unroll
  for (int q = 0; q < kDwrChunk * EB / 256; ++q) {
    const int i = threadIdx.x + 256 * q;
    sdl[i / EB][i % EB] = dv[q];
  }
  __syncthreads();
  float acc[EB][CV];
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int v = 0; v < CV; ++v) acc[e][v] = 0.f;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int tt = tl + 8 * j;
#pragma unroll
    for (int v = 0; v < CV; ++v) {
      const float xv = Elt<T>::ld(&xr[j].v[v]);
#pragma unroll
      for (int e = 0; e < EB; ++e) acc[e][v] = fmaf(sdl[tt][e], xv, acc[e][v]);
    }
  }
  // sum the 8 token lanes (fixed order; every lane of the group ends with the
  // same sums), then lane tl writes experts tl, tl + 8, ...: CV contiguous
  // floats per expert row
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int v = 0; v < CV; ++v) {
      float a = acc[e][v];
      a += __shfl_xor(a, 1, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 4, 64);
      acc[e][v] = a;
    }
  const bool cols_full = c0 + CV <= d;
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if ((e & 7) != tl || e >= E) continue;
    float* dst = part + ((long)chunk * E + e) * d + c0;
    if (cols_full) {
      if constexpr (CV % 4 == 0) {
#pragma unroll
        for (int v = 0; v < CV; v += 4) *(float4*)(dst + v) = make_float4(acc[e][v], acc[e][v + 1], acc[e][v + 2], acc[e][v + 3]);
      } else {
#pragma unroll
        for (int v = 0; v < CV; ++v) dst[v] = acc[e][v];
      }
    } else {
#pragma unroll
      for (int v = 0; v < CV; ++v)
        if (c0 + v < d) dst[v] = acc[e][v];
    }
  }
}

// out[i] = sum over the nch chunk partials in chunk order (8 loads in flight).
template <class T>
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float* __restrict__ part, int nch, long n,
                                                        T* __restrict__ out) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= nch; c += 8) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = part[(long)(c + q) * n + i];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; c < nch; ++c) s += part[(long)c * n + i];
  Elt<T>::st(out + i, s);
}

// dx[t] += sum_e dL[t, e] Wr[e] for TPB = 4 tokens per workgroup: the Wr
// row pieces a thread loads serve all TPB token rows.  With dxp the
// expert-path term is summed here instead of read from dx (the unpermute-sum
// folded in): dx[t] = sum_j dxp[pos[t, j]] + sum_e dL[t, e] Wr[e], the slots
// summed in order in fp32 as the unpermute-sum does, then the router term,
// one rounding.
constexpr int kDxTokens = 4;
template <class T, int EB>
__global__ __launch_bounds__(256) void router_dx_valu_kernel(const float* __restrict__ dL, const T* __restrict__ wr,
                                                             int Tn, int d, int E, T* __restrict__ dx,
                                                             const T* __restrict__ dxp, const int* __restrict__ pos,
                                                             int k) {
  constexpr int V = Elt<T>::kVec;
  constexpr int TPB = kDxTokens;
  __shared__ float sdl[TPB][EB];
  __shared__ int spos[TPB][32];  // the tokens' slot positions (k <= 32; rows past Tn: row Tn - 1's)
  const int t0 = blockIdx.x * TPB;
  for (int i = threadIdx.x; i < TPB * EB; i += 256) {
    const int u = i / EB, e = i % EB;
    sdl[u][e] = (t0 + u < Tn && e < E) ? dL[(long)(t0 + u) * E + e] : 0.f;
  }
  if (dxp != nullptr)
    for (int i = threadIdx.x; i < TPB * k; i += 256) {
      const int u = i / k, j = i % k;
      spos[u][j] = pos[(long)min(t0 + u, Tn - 1) * k + j];
    }
  __syncthreads();
  const int nv = d / V;
  for (int v = threadIdx.x; v < nv; v += 256) {
    // the expert-path gradient rows (rows past Tn read row Tn - 1 and are
    // never written), added after the router term
    float base[TPB][V];
    if (dxp == nullptr) {
#pragma unroll
      for (int u = 0; u < TPB; ++u) unpack16<T>(((const uint4*)(dx + (long)min(t0 + u, Tn - 1) * d))[v], base[u]);
    } else {  // slot j's rows of all TPB tokens loaded together
#pragma unroll
      for (int u = 0; u < TPB; ++u)
#pragma unroll
        for (int i = 0; i < V; ++i) base[u][i] = 0.f;
      for (int j = 0; j < k; ++j) {
        uint4 rv[TPB];
#pragma unroll
        for (int u = 0; u < TPB; ++u)
          rv[u] = ((const uint4*)(dxp + (long)spos[u][j] * d))[v];
#pragma unroll
        for (int u = 0; u < TPB; ++u) {
          float f[V];
          unpack16<T>(rv[u], f);
#pragma unroll
          for (int i = 0; i < V; ++i) base[u][i] += f[i];
        }
      }
    }
    float acc[TPB][V];
#pragma unroll
    for (int u = 0; u < TPB; ++u)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[u][i] = 0.f;
    // groups of 8 expert rows, loaded unconditionally (clamped row index) so
    // that they are in flight together; the FMAs depend on e < E
#pragma unroll
    for (int e0 = 0; e0 < EB; e0 += 8) {
      if (e0 >= E) break;
      uint4 wv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) wv[q] = ((const uint4*)(wr + (long)min(e0 + q, E - 1) * d))[v];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (e0 + q < E) {
          float w[V];
          unpack16<T>(wv[q], w);
#pragma unroll
          for (int u = 0; u < TPB; ++u)
#pragma unroll
            for (int i = 0; i < V; ++i) acc[u][i] = fmaf(sdl[u][e0 + q], w[i], acc[u][i]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TPB; ++u) {
      if (t0 + u < Tn) {
#pragma unroll
        for (int i = 0; i < V; ++i) acc[u][i] += base[u][i];
        ((uint4*)(dx + (long)(t0 + u) * d))[v] = pack16<T>(acc[u]);
      }
    }
  }
}

template <class T>
__global__ __launch_bounds__(256) void zero_fill_kernel(T* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = T(0);
}

static inline bool router_uses_mfma(bool bf16, int E) { return bf16 && E >= 64 && E % 8 == 0; }
static inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

size_t router_bwd_ws_bytes(int T, int d, int E) {
  const size_t dl = align256((size_t)T * E * sizeof(float));
  const size_t dlb = align256((size_t)T * E * sizeof(uint16_t));
  const size_t valu = align256((size_t)((T + kDwrChunk - 1) / kDwrChunk) * E * d * sizeof(float));
  const size_t mf = align256(router_dwr_mfma_part_bytes(T, d, E));
  return dl + dlb + (valu > mf ? valu : mf);
}

template <class T, int EB>
static void logits_valu(const void* x, const void* wr, int Tn, int d, int E, float* out, hipStream_t s) {
  router_logits_valu_kernel<T, EB><<<(Tn + 3) / 4, 256, 0, s>>>((const T*)x, (const T*)wr, Tn, d, E, out);
}

template <class T>
static void logits_valu_any(const void* x, const void* wr, int Tn, int d, int E, float* out, hipStream_t s) {
  if (E <= 8) logits_valu<T, 8>(x, wr, Tn, d, E, out, s);
  else if (E <= 16) logits_valu<T, 16>(x, wr, Tn, d, E, out, s);
  else if (E <= 32) logits_valu<T, 32>(x, wr, Tn, d, E, out, s);
  else logits_valu<T, 64>(x, wr, Tn, d, E, out, s);
}

hipError_t launch_router_logits(const void* x, bool bf16, const void* wr, int T, int d, int E, float* logits,
                                hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (router_uses_mfma(bf16, E))
    return launch_dense_nt_f32out((const uint16_t*)x, (const uint16_t*)wr, logits, T, E, d, s);
  if (E > 64) return hipErrorInvalidValue;
  if (bf16) logits_valu_any<uint16_t>(x, wr, T, d, E, logits, s);
  else logits_valu_any<float>(x, wr, T, d, E, logits, s);
  return hipGetLastError();
}

template <class T, int EB>
static void bwd_valu(const float* dL, const void* x, const void* wr, int Tn, int d, int E, void* dx, void* dwr,
                     float* part, hipStream_t s, const void* dxp, const int* pos, int k, unsigned parts) {
  // dx first: in a step whose weight gradients run on a second stream this
  // pass (the larger one) fills the CUs those GEMMs free as they finish, and
  // the dWr sum, which no later kernel of the step reads, comes last.  The
  // two outputs are independent.
  if (parts & kRouterDx)
    router_dx_valu_kernel<T, EB><<<(Tn + kDxTokens - 1) / kDxTokens, 256, 0, s>>>(dL, (const T*)wr, Tn, d, E, (T*)dx,
                                                                                  (const T*)dxp, pos, k);
  if (parts & kRouterDwr) {
    const int nch = (Tn + kDwrChunk - 1) / kDwrChunk;
    constexpr int CV = 64 / EB;
    constexpr int cols_per_block = 32 * CV;
    dim3 grid((d + cols_per_block - 1) / cols_per_block, nch);
    if (d % CV == 0) router_dwr_partial_kernel<T, EB, false><<<grid, 256, 0, s>>>(dL, (const T*)x, Tn, d, E, part);
    else router_dwr_partial_kernel<T, EB, true><<<grid, 256, 0, s>>>(dL, (const T*)x, Tn, d, E, part);
    const long n = (long)E * d;
    chunk_sum_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(part, nch, n, (T*)dwr);
  }
}

template <class T>
static void bwd_valu_any(const float* dL, const void* x, const void* wr, int Tn, int d, int E, void* dx, void* dwr,
                         float* part, hipStream_t s, const void* dxp, const int* pos, int k, unsigned parts) {
  if (E <= 8) bwd_valu<T, 8>(dL, x, wr, Tn, d, E, dx, dwr, part, s, dxp, pos, k, parts);
  else if (E <= 16) bwd_valu<T, 16>(dL, x, wr, Tn, d, E, dx, dwr, part, s, dxp, pos, k, parts);
  else if (E <= 32) bwd_valu<T, 32>(dL, x, wr, Tn, d, E, dx, dwr, part, s, dxp, pos, k, parts);
  else bwd_valu<T, 64>(dL, x, wr, Tn, d, E, dx, dwr, part, s, dxp, pos, k, parts);
}

hipError_t launch_router_bwd(const float* probs, const int* idx, const float* dgate, const float* aux_g,
                             const void* x, const void* wr, int T, int d, int E, int k, bool bf16, void* dx, void* dwr,
                             void* ws, hipStream_t s, const void* dxp, const int* pos, unsigned parts) {
  const bool mf = router_uses_mfma(bf16, E);
  if (!mf && E > 64) return hipErrorInvalidValue;
  char* p = (char*)ws;
  float* dL = (float*)p;
  p += align256((size_t)T * E * sizeof(float));
  uint16_t* dLb = (uint16_t*)p;
  p += align256((size_t)T * E * sizeof(uint16_t));
  float* part = (float*)p;
  if (T == 0) {  // no tokens: dWr is zero (a fill kernel, not a memset node)
    if (!(parts & kRouterDwr)) return hipSuccess;
    const long n = (long)E * d;
    if (bf16) zero_fill_kernel<uint16_t><<<(unsigned)((n + 255) / 256), 256, 0, s>>>((uint16_t*)dwr, n);
    else zero_fill_kernel<float><<<(unsigned)((n + 255) / 256), 256, 0, s>>>((float*)dwr, n);
    return hipGetLastError();
  }
  const dim3 gw((T + 3) / 4);
  uint16_t* dlb_out = mf ? dLb : nullptr;
  if (E <= 64) router_dl_kernel<1><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 128) router_dl_kernel<2><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 256) router_dl_kernel<4><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else if (E <= 512) router_dl_kernel<8><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  else router_dl_kernel<16><<<gw, 256, 0, s>>>(probs, idx, dgate, aux_g, T, E, k, dL, dlb_out);
  if (mf) {
    // dx first, as on the vector path (bwd_valu): with the weight gradients on a
    // second stream the fused dx GEMM fills the CUs they free
    if (parts & kRouterDx) {
      hipError_t err =
          launch_router_dx_mfma(dLb, (const uint16_t*)wr, (uint16_t*)dx, (const uint16_t*)dxp, pos, k, T, d, E, s);
      if (err != hipSuccess) return err;
    }
    if (parts & kRouterDwr)
      return launch_router_dwr_mfma(dLb, (const uint16_t*)x, (uint16_t*)dwr, part, T, d, E, s);
    return hipGetLastError();
  }
  if (bf16) bwd_valu_any<uint16_t>(dL, x, wr, T, d, E, dx, dwr, part, s, dxp, pos, k, parts);
  else bwd_valu_any<float>(dL, x, wr, T, d, E, dx, dwr, part, s, dxp, pos, k, parts);
  return hipGetLastError();
}

}  // namespace trg
