// KV-drift probe: how far the K and V rows a step recomputes moved away from the
// values the cache held before the step.
//
// The pages measure the drift of the KV cache between consecutive denoising
// steps as the cosine distance of the value vectors, and report that it tracks
// the largest entropy among the tokens decoded in the step before (EntropyCache
// explainer, Arabic technical summary, section 2, key observations; Italian
// summary, section 2, observation 1). The probe measures exactly that quantity
// on the rows a step recomputes: for row i of layer l,
//   dist = 1 - <old, new> / (|old| |new|),
// with old = the cached vector before the step and new = the vector the step
// writes, for K and for V; per layer the mean and the max over the rows. A row
// whose old or new vector has zero norm (the never-written cache of a first
// step) is left out; a layer with no row left reports NaN.
//
// Three kernels: copy the rows' cached K/V before the layer's QKV GEMM
// overwrites them; per-row distances after it; per (layer, K/V) mean and max
// over the rows in a fixed order (deterministic).
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;

// old_k[i] = k_cache[rows[i]], old_v likewise (one workgroup per row)
template <typename T>
__global__ void __launch_bounds__(kThreads)
drift_gather_kernel(const T* __restrict__ kc, const T* __restrict__ vc, const int32_t* __restrict__ rows,
                    int L, int d, T* __restrict__ ok, T* __restrict__ ov) {
  const int i = blockIdx.x;
  const int p = rows[i];
  T* dk = ok + (int64_t)i * d;
  T* dv = ov + (int64_t)i * d;
  if (p < 0 || p >= L) {
    for (int j = threadIdx.x; j < d; j += kThreads) dk[j] = dv[j] = from_f<T>(0.f);
    return;
  }
  const T* sk = kc + (int64_t)p * d;
  const T* sv = vc + (int64_t)p * d;
  for (int j = threadIdx.x; j < d; j += kThreads) {
    dk[j] = sk[j];
    dv[j] = sv[j];
  }
}

__device__ __forceinline__ float block_sum(float x, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kThreads / 64; ++k) t += red[k];
  return t;
}

// dist[c * n + i] (c = 0: K, 1: V) for row i: 1 - cos(old, cache[rows[i]]), NaN if a norm is 0
template <typename T>
__global__ void __launch_bounds__(kThreads)
drift_rows_kernel(const T* __restrict__ ok, const T* __restrict__ ov, const T* __restrict__ kc,
                  const T* __restrict__ vc, const int32_t* __restrict__ rows, int n, int L, int d,
                  float* __restrict__ dist) {
  __shared__ float red[kThreads / 64];
  const int i = blockIdx.x;
  const int p = rows[i];
  for (int c = 0; c < 2; ++c) {
    const T* o = (c == 0 ? ok : ov) + (int64_t)i * d;
    float dot = 0.f, n0 = 0.f, n1 = 0.f;
    if (p >= 0 && p < L) {
      const T* nw = (c == 0 ? kc : vc) + (int64_t)p * d;
      for (int j = threadIdx.x; j < d; j += kThreads) {
        const float a = to_f(o[j]), b = to_f(nw[j]);
        dot = fmaf(a, b, dot);
        n0 = fmaf(a, a, n0);
        n1 = fmaf(b, b, n1);
      }
    }
    dot = block_sum(dot, red);
    n0 = block_sum(n0, red);
    n1 = block_sum(n1, red);
    if (threadIdx.x == 0)
      dist[(int64_t)c * n + i] = (n0 > 0.f && n1 > 0.f) ? 1.0f - dot / (sqrtf(n0) * sqrtf(n1)) : NAN;
  }
}

// out[4 l + 2 c + {0, 1}] = mean, max over the n valid (non-NaN) distances of (layer l, c)
__global__ void __launch_bounds__(kThreads)
drift_reduce_kernel(const float* __restrict__ dist, int n, int64_t layer_stride, float* __restrict__ out) {
  __shared__ float rs[kThreads], rm[kThreads];
  __shared__ int rc[kThreads];
  const int l = blockIdx.x, c = blockIdx.y;
  const float* x = dist + l * layer_stride + (int64_t)c * n;
  float s = 0.f, m = -INFINITY;
  int cnt = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const float v = x[i];
    if (v != v) continue;
    s += v;
    m = fmaxf(m, v);
    ++cnt;
  }
  rs[threadIdx.x] = s;
  rm[threadIdx.x] = m;
  rc[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      rs[threadIdx.x] += rs[threadIdx.x + w];
      rm[threadIdx.x] = fmaxf(rm[threadIdx.x], rm[threadIdx.x + w]);
      rc[threadIdx.x] += rc[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[4 * l + 2 * c] = rc[0] ? rs[0] / rc[0] : NAN;
    out[4 * l + 2 * c + 1] = rc[0] ? rm[0] : NAN;
  }
}

}  // namespace

ec_status drift_gather(ec_dtype dt, const void* kc, const void* vc, const int32_t* rows, int n, int L, int d,
                       void* ok, void* ov, hipStream_t s) {
  if (n == 0) return EC_OK;
  if (dt == EC_BF16)
    drift_gather_kernel<bf16><<<n, kThreads, 0, s>>>((const bf16*)kc, (const bf16*)vc, rows, L, d, (bf16*)ok,
                                                     (bf16*)ov);
  else
    drift_gather_kernel<float><<<n, kThreads, 0, s>>>((const float*)kc, (const float*)vc, rows, L, d,
                                                      (float*)ok, (float*)ov);
  EC_CHECK_LAUNCH("drift_gather_kernel");
  return EC_OK;
}

ec_status drift_rows(ec_dtype dt, const void* ok, const void* ov, const void* kc, const void* vc,
                     const int32_t* rows, int n, int L, int d, float* dist, hipStream_t s) {
  if (n == 0) return EC_OK;
  if (dt == EC_BF16)
    drift_rows_kernel<bf16><<<n, kThreads, 0, s>>>((const bf16*)ok, (const bf16*)ov, (const bf16*)kc,
                                                   (const bf16*)vc, rows, n, L, d, dist);
  else
    drift_rows_kernel<float><<<n, kThreads, 0, s>>>((const float*)ok, (const float*)ov, (const float*)kc,
                                                    (const float*)vc, rows, n, L, d, dist);
  EC_CHECK_LAUNCH("drift_rows_kernel");
  return EC_OK;
}

ec_status drift_reduce(const float* dist, int n_layers, int n, int64_t layer_stride, float* out, hipStream_t s) {
  drift_reduce_kernel<<<dim3(n_layers, 2), kThreads, 0, s>>>(dist, n, layer_stride, out);
  EC_CHECK_LAUNCH("drift_reduce_kernel");
  return EC_OK;
}

}  // namespace ec
