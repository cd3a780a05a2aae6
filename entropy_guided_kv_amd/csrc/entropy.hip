// Fused softmax entropy / argmax / confidence reduction over the vocabulary.
//
// The decision signal of EntropyCache is E_{t+1}, the largest softmax entropy
// (nats) among the newly decoded tokens' distributions; it costs O(V) per row
// and does not depend on sequence length or depth (EntropyCache explainer,
// Arabic technical summary, section 2, "Decode and evaluate entropy").
//
// Single pass over the logits with an online (running-max) form: with m the
// running max, Z = sum exp(x - m) and S = sum (x - m) exp(x - m), the entropy
// is ln Z - S/Z, the confidence max_j p_j = 1/Z and the argmax the first
// index holding m. Two states merge exactly:
//   m = max(ma, mb); Z = Za e^(ma-m) + Zb e^(mb-m);
//   S = (Sa + (ma-m) Za) e^(ma-m) + (Sb + (mb-m) Zb) e^(mb-m).
// One exponential per element; each 16-byte vector first updates the max once.
//
// Layout: grid (splits, rows); each workgroup streams one contiguous slice of
// one row with coalesced 16-byte loads (consecutive lanes, consecutive
// vectors), reduces (m, Z, S, idx) across the wavefront with shuffles and
// across waves through LDS, and writes one partial state. A second small
// kernel merges the splits of every row in split order (deterministic) and
// takes the max entropy over the selected rows.
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr float kNegInf = -INFINITY;

struct Part {
  float m, z, s;
  int idx;
  int nan;
};

__device__ __forceinline__ void merge(Part& a, const Part& b) {
  a.nan |= b.nan;
  float m = fmaxf(a.m, b.m);
  if (m == kNegInf) {  // both empty (all -inf so far); keep the lower index
    a.idx = min(a.idx, b.idx);
    return;
  }
  float za = 0.f, sa = 0.f, zb = 0.f, sb = 0.f;
  if (a.m != kNegInf) {
    float d = a.m - m, f = __expf(d);
    za = a.z * f;
    sa = (a.s + d * a.z) * f;
  }
  if (b.m != kNegInf) {
    float d = b.m - m, f = __expf(d);
    zb = b.z * f;
    sb = (b.s + d * b.z) * f;
  }
  int idx;
  if (a.m == b.m) idx = min(a.idx, b.idx);
  else idx = (a.m > b.m) ? a.idx : b.idx;
  a.m = m;
  a.z = za + zb;
  a.s = sa + sb;
  a.idx = idx;
}

// Add n values (n <= 8) at global indices j0..j0+n-1, in increasing order.
__device__ __forceinline__ void absorb(Part& p, const float* x, int n, int j0) {
  float cm = kNegInf;
  int ci = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < n) {
      float v = x[k];
      p.nan |= (v != v);
      if (v > cm) { cm = v; ci = j0 + k; }
    }
  }
  if (cm > p.m) {
    if (p.m != kNegInf) {
      float d = p.m - cm, f = __expf(d);
      p.s = (p.s + d * p.z) * f;
      p.z = p.z * f;
    }
    p.m = cm;
    p.idx = ci;
  } else if (cm == p.m && ci < p.idx) {
    p.idx = ci;
  }
  if (p.m == kNegInf) return;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < n) {
      float t = x[k] - p.m;
      float e = __expf(t);
      p.z += e;
      p.s += (e > 0.f) ? t * e : 0.f;
    }
  }
}

__device__ __forceinline__ void load8(const bf16* base, int64_t j, float* x) {
  uint4 u = *reinterpret_cast<const uint4*>(base + j);
  uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(w[k] << 16);
    x[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* base, int64_t j, float* x) {
  float4 a = *reinterpret_cast<const float4*>(base + j);
  float4 b = *reinterpret_cast<const float4*>(base + j + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ Part shfl_part(const Part& p, int mask) {
  Part o;
  o.m = __shfl_xor(p.m, mask);
  o.z = __shfl_xor(p.z, mask);
  o.s = __shfl_xor(p.s, mask);
  o.idx = __shfl_xor(p.idx, mask);
  o.nan = __shfl_xor(p.nan, mask);
  return o;
}

// grid: (splits, rows). Slice of row r: [split * chunk, min(V, (split+1) * chunk)).
template <typename T, bool VEC>
__global__ void __launch_bounds__(kThreads)
entropy_partial_kernel(const T* __restrict__ logits, int V, int64_t stride, int chunk,
                       Part* __restrict__ parts) {
  const int split = blockIdx.x, row = blockIdx.y, splits = gridDim.x;
  const T* base = logits + (int64_t)row * stride;
  const int lo = split * chunk;
  const int hi = min(V, lo + chunk);
  Part p{kNegInf, 0.f, 0.f, 0x7fffffff, 0};
  float x[8];
  if (VEC) {
    // chunk is a multiple of 8, so [lo, hi8) is made of whole 8-element vectors
    const int hi8 = lo + ((hi - lo) & ~7);
    int j = lo + threadIdx.x * 8;
    for (; j + 3 * kThreads * 8 < hi8; j += 4 * kThreads * 8) {
      float y[3][8];
      load8(base, j, x);
      load8(base, j + kThreads * 8, y[0]);
      load8(base, j + 2 * kThreads * 8, y[1]);
      load8(base, j + 3 * kThreads * 8, y[2]);
      absorb(p, x, 8, j);
      absorb(p, y[0], 8, j + kThreads * 8);
      absorb(p, y[1], 8, j + 2 * kThreads * 8);
      absorb(p, y[2], 8, j + 3 * kThreads * 8);
    }
    for (; j < hi8; j += kThreads * 8) {
      load8(base, j, x);
      absorb(p, x, 8, j);
    }
    // ragged tail (< 8 elements), only in the last slice of a row
    if (threadIdx.x == 0 && hi8 < hi) {
      int n = hi - hi8;
      for (int k = 0; k < n; ++k) x[k] = to_f(base[hi8 + k]);
      absorb(p, x, n, hi8);
    }
  } else {
    for (int j = lo + threadIdx.x; j < hi; j += kThreads) {
      x[0] = to_f(base[j]);
      absorb(p, x, 1, j);
    }
  }
  // wavefront reduction (64 lanes)
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) {
    Part o = shfl_part(p, mask);
    merge(p, o);
  }
  __shared__ Part wp[kThreads / 64];
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) wp[wave] = p;
  __syncthreads();
  if (threadIdx.x == 0) {
    Part a = wp[0];
    for (int w = 1; w < kThreads / 64; ++w) merge(a, wp[w]);
    parts[(int64_t)row * splits + split] = a;
  }
}

// One workgroup: merges the splits of every row (in split order), writes
// entropy / argmax / confidence, then the max entropy over the selected rows.
__global__ void __launch_bounds__(kThreads)
entropy_merge_kernel(const Part* __restrict__ parts, int rows, int splits,
                     const int32_t* __restrict__ sel, int n_sel, float* __restrict__ H,
                     int32_t* __restrict__ amax, float* __restrict__ conf,
                     float* __restrict__ emax) {
  for (int r = threadIdx.x; r < rows; r += kThreads) {
    Part a = parts[(int64_t)r * splits];
    for (int s = 1; s < splits; ++s) merge(a, parts[(int64_t)r * splits + s]);
    float h, c;
    if (a.nan || a.m == kNegInf) {
      h = NAN;
      c = NAN;
    } else {
      h = __logf(a.z) - a.s / a.z;
      c = 1.0f / a.z;
    }
    H[r] = h;
    conf[r] = c;
    amax[r] = a.idx == 0x7fffffff ? 0 : a.idx;
  }
  if (emax == nullptr) return;
  __syncthreads();
  __shared__ float red[kThreads];
  __shared__ int rnan[kThreads];
  float m = kNegInf;
  int nan = 0;
  const int n = sel ? n_sel : rows;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    int r = sel ? sel[i] : i;
    float h = (r >= 0 && r < rows) ? H[r] : NAN;
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

void choose_split(int rows, int V, int& splits, int& chunk) {
  splits = (V + 8191) / 8192;
  if (rows * splits < 1024) splits = (1024 + rows - 1) / rows;
  int max_splits = (V + 2047) / 2048;
  if (splits > max_splits) splits = max_splits;
  if (splits > 128) splits = 128;
  if (splits < 1) splits = 1;
  chunk = ((V + splits - 1) / splits + 7) & ~7;
  splits = (V + chunk - 1) / chunk;
}

}  // namespace

size_t entropy_ws_bytes(int rows, int vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  int splits, chunk;
  choose_split(rows, vocab, splits, chunk);
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
  int splits, chunk;
  choose_split(rows, vocab, splits, chunk);
  Part* parts = (Part*)ws;
  const size_t esz = dt == EC_BF16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * esz) % 16 == 0);
  dim3 grid(splits, rows);
  if (dt == EC_BF16) {
    if (vec)
      entropy_partial_kernel<bf16, true><<<grid, kThreads, 0, s>>>((const bf16*)logits, vocab, stride, chunk, parts);
    else
      entropy_partial_kernel<bf16, false><<<grid, kThreads, 0, s>>>((const bf16*)logits, vocab, stride, chunk, parts);
  } else {
    if (vec)
      entropy_partial_kernel<float, true><<<grid, kThreads, 0, s>>>((const float*)logits, vocab, stride, chunk, parts);
    else
      entropy_partial_kernel<float, false><<<grid, kThreads, 0, s>>>((const float*)logits, vocab, stride, chunk, parts);
  }
  EC_CHECK_LAUNCH("entropy_partial_kernel");
  entropy_merge_kernel<<<1, kThreads, 0, s>>>(parts, rows, splits, sel, n_sel, H, amax, c, emax);
  EC_CHECK_LAUNCH("entropy_merge_kernel");
  return EC_OK;
}

}  // namespace ec
