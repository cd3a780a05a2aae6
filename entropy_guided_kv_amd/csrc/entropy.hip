// Fused softmax entropy / argmax / confidence reduction over the vocabulary.
//
// The decision signal of EntropyCache is E_{t+1}, the largest softmax entropy
// (nats) among the newly decoded tokens' distributions; it costs O(V) per row
// and does not depend on sequence length or depth (EntropyCache explainer,
// Arabic technical summary, section 2, "Decode and evaluate entropy").
//
// With m the row max, Z = sum exp(x - m) and S = sum (x - m) exp(x - m), the
// entropy is ln Z - S/Z, the confidence max_j p_j = 1/Z and the argmax the
// first index holding m. Partial states over disjoint slices merge exactly:
//   m = max(ma, mb); Z = Za e^(ma-m) + Zb e^(mb-m);
//   S = (Sa + (ma-m) Za) e^(ma-m) + (Sb + (mb-m) Zb) e^(mb-m).
//
// Kernel 1 (grid: slices x rows, 256 threads): each workgroup owns one slice
// of one row and reads it exactly once from HBM with 16-byte loads, all issued
// up front (U vectors per thread held in registers; consecutive lanes read
// consecutive vectors). The slice max and first argmax come from a wavefront
// shuffle + LDS reduction; then every element is exponentiated once against
// the slice max (exp2 of (x - max) * log2 e) and Z, S are summed the same
// way. No per-element rescaling and no data reread.
// Kernel 2 (grid: rows, one wavefront each): merges the slices of a row in a
// fixed order (deterministic) and writes entropy / argmax / confidence.
// Kernel 3 (one workgroup, only when E is requested): max over selected rows.
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kU = 4;  // 16-byte vectors per thread per slice
constexpr float kNegInf = -INFINITY;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct Part {
  float m, z, s;  // s in natural units: sum (x - m) e^(x - m)
  int idx;
  int nan;
  int pad[3];
};

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<bf16> {
  static constexpr int E = 8;
  __device__ static void unpack(const v4u& u, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(u[k] << 16);
      x[2 * k + 1] = __uint_as_float(u[k] & 0xffff0000u);
    }
  }
};
template <> struct Vec<float> {
  static constexpr int E = 4;
  __device__ static void unpack(const v4u& u, float* x) {
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(u[k]);
  }
};

// (value, index) max with the lower index on ties
__device__ __forceinline__ void vmax(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(kThreads)
entropy_slice_kernel(const T* __restrict__ logits, int V, int64_t stride, int chunk,
                     Part* __restrict__ parts) {
  constexpr int E = Vec<T>::E;
  constexpr int NV = kU * E;  // values per thread
  const int split = blockIdx.x, row = blockIdx.y, splits = gridDim.x;
  const T* base = logits + (int64_t)row * stride;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;

  float x[NV];
  int j0[kU];
  if (VEC) {
    const int hiv = lo + ((hi - lo) / E) * E;  // end of the whole vectors
    v4u u[kU];
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      j0[k] = lo + (tid + k * kThreads) * E;
      if (j0[k] < hiv) u[k] = *reinterpret_cast<const v4u*>(base + j0[k]);
    }
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      if (j0[k] < hiv) {
        Vec<T>::unpack(u[k], x + k * E);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = j0[k] + e;
          x[k * E + e] = (j >= hiv && j < hi) ? to_f(base[j]) : kNegInf;  // ragged row end
        }
      }
    }
  } else {
#pragma unroll
    for (int k = 0; k < kU; ++k) {
      j0[k] = lo + (tid + k * kThreads) * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = j0[k] + e;
        x[k * E + e] = j < hi ? to_f(base[j]) : kNegInf;
      }
    }
  }

  // ---- slice max and first argmax
  float mv = kNegInf;
  int mi = 0x7fffffff;
  int nan = 0;
#pragma unroll
  for (int k = 0; k < kU; ++k)
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float v = x[k * E + e];
      nan |= (v != v);
      if (v > mv) {  // strict: first index within the thread (indices increase with k, e)
        mv = v;
        mi = j0[k] + e;
      }
    }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(mv, o);
    const int i2 = __shfl_xor(mi, o);
    vmax(mv, mi, v2, i2);
    nan |= __shfl_xor(nan, o);
  }
  __shared__ float sm[kThreads / 64];
  __shared__ int si[kThreads / 64], sn[kThreads / 64];
  __shared__ float sz[kThreads / 64], ss[kThreads / 64];
  if (lane == 0) {
    sm[wave] = mv;
    si[wave] = mi;
    sn[wave] = nan;
  }
  __syncthreads();
  mv = sm[0];
  mi = si[0];
  nan = sn[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) {
    vmax(mv, mi, sm[w], si[w]);
    nan |= sn[w];
  }

  // ---- Z and S against the slice max (log2 domain, one exp2 per element)
  float z = 0.f, s2 = 0.f;
  if (mv != kNegInf) {
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const float t = (x[q] - mv) * kLog2e;  // exactly 0 at the max
      const float e = exp2f(t);
      z += e;
      s2 += e > 0.f ? t * e : 0.f;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    z += __shfl_xor(z, o);
    s2 += __shfl_xor(s2, o);
  }
  if (lane == 0) {
    sz[wave] = z;
    ss[wave] = s2;
  }
  __syncthreads();
  if (tid == 0) {
    float zt = 0.f, st = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      zt += sz[w];
      st += ss[w];
    }
    Part p;
    p.m = mv;
    p.z = zt;
    p.s = st * kLn2;
    p.idx = mi;
    p.nan = nan;
    parts[(int64_t)row * splits + split] = p;
  }
}

// One wavefront per row: merge the row's slices (lane l takes slices l, l+64, ...).
__global__ void __launch_bounds__(64)
entropy_merge_kernel(const Part* __restrict__ parts, int splits, float* __restrict__ H,
                     int32_t* __restrict__ amax, float* __restrict__ conf) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const Part* pr = parts + (int64_t)row * splits;
  float mv = kNegInf;
  int mi = 0x7fffffff, nan = 0;
  for (int s = lane; s < splits; s += 64) {
    vmax(mv, mi, pr[s].m, pr[s].idx);
    nan |= pr[s].nan;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v2 = __shfl_xor(mv, o);
    const int i2 = __shfl_xor(mi, o);
    vmax(mv, mi, v2, i2);
    nan |= __shfl_xor(nan, o);
  }
  float z = 0.f, s = 0.f;
  if (mv != kNegInf) {
    for (int q = lane; q < splits; q += 64) {
      const Part p = pr[q];
      if (p.m == kNegInf) continue;
      const float d = p.m - mv, f = __expf(d);
      z += p.z * f;
      s += (p.s + d * p.z) * f;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    z += __shfl_xor(z, o);
    s += __shfl_xor(s, o);
  }
  if (lane == 0) {
    const bool bad = nan || mv == kNegInf;
    H[row] = bad ? NAN : __logf(z) - s / z;
    conf[row] = bad ? NAN : 1.0f / z;
    amax[row] = mi == 0x7fffffff ? 0 : mi;
  }
}

// E = max entropy over the selected rows (NaN if any selected row is NaN).
__global__ void __launch_bounds__(kThreads)
entropy_emax_kernel(const float* __restrict__ H, int rows, const int32_t* __restrict__ sel,
                    int n_sel, float* __restrict__ emax) {
  __shared__ float red[kThreads];
  __shared__ int rnan[kThreads];
  float m = kNegInf;
  int nan = 0;
  const int n = sel ? n_sel : rows;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int r = sel ? sel[i] : i;
    const float h = (r >= 0 && r < rows) ? H[r] : NAN;
    if (h != h) nan = 1;
    else m = fmaxf(m, h);
  }
  red[threadIdx.x] = m;
  rnan[threadIdx.x] = nan;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) {
      red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
      rnan[threadIdx.x] |= rnan[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *emax = rnan[0] ? NAN : red[0];
}

__global__ void fill_kernel(float* p, float v) { *p = v; }

// slice length: kU vectors per thread -> 8192 bf16 / 4096 f32 elements per workgroup
int slice_len(ec_dtype dt) { return kThreads * kU * (dt == EC_BF16 ? 8 : 4); }

}  // namespace

size_t entropy_ws_bytes(int rows, int vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  const int splits = (vocab + slice_len(EC_F32) - 1) / slice_len(EC_F32);  // the larger count
  return (size_t)rows * splits * sizeof(Part) + 256;
}

ec_status entropy(ec_dtype dt, const void* logits, int rows, int vocab, int64_t stride,
                  const int32_t* sel, int n_sel, float* H, int32_t* amax, float* c, float* emax,
                  void* ws, size_t ws_bytes, hipStream_t s) {
  if (rows == 0) {
    if (emax) {
      fill_kernel<<<1, 1, 0, s>>>(emax, kNegInf);
      EC_CHECK_LAUNCH("fill_kernel");
    }
    return EC_OK;
  }
  const int chunk = slice_len(dt);
  const int splits = (vocab + chunk - 1) / chunk;
  Part* parts = (Part*)ws;
  const size_t esz = dt == EC_BF16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * esz) % 16 == 0);
  dim3 grid(splits, rows);
  if (dt == EC_BF16) {
    if (vec)
      entropy_slice_kernel<bf16, true><<<grid, kThreads, 0, s>>>((const bf16*)logits, vocab, stride, chunk, parts);
    else
      entropy_slice_kernel<bf16, false><<<grid, kThreads, 0, s>>>((const bf16*)logits, vocab, stride, chunk, parts);
  } else {
    if (vec)
      entropy_slice_kernel<float, true><<<grid, kThreads, 0, s>>>((const float*)logits, vocab, stride, chunk, parts);
    else
      entropy_slice_kernel<float, false><<<grid, kThreads, 0, s>>>((const float*)logits, vocab, stride, chunk, parts);
  }
  EC_CHECK_LAUNCH("entropy_slice_kernel");
  entropy_merge_kernel<<<rows, 64, 0, s>>>(parts, splits, H, amax, c);
  EC_CHECK_LAUNCH("entropy_merge_kernel");
  if (emax) {
    entropy_emax_kernel<<<1, kThreads, 0, s>>>(H, rows, sel, n_sel, emax);
    EC_CHECK_LAUNCH("entropy_emax_kernel");
  }
  return EC_OK;
}

}  // namespace ec
