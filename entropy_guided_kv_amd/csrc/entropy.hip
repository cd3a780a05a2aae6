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
// ec_entropy_max runs as one launch (entropy_fused_kernel, described there): every
// logit is read once from HBM with 16-byte loads, exponentiated once (exp2 of
// x log2 e - m log2 e, one FMA) against its lane's running maximum, and the slice
// states of a row merge in a fixed order, so results are reproducible. A NaN logit
// is skipped by the maximum and carried as a flag, which makes its row's entropy and
// confidence NaN. The fused LM-head epilogue of the GEMM produces slice states of its
// own; entropy_merge_kernel (one wavefront per row) merges those.
#include "ec_internal.h"

#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

namespace ec {

namespace {

constexpr float kNegInf = -INFINITY;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef EntPart Part;  // s in natural units: sum (x - m) e^(x - m)

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

// a <- merge(a, b) of two partial states: m = max, z and s rescaled to it,
// argmax = larger value, lower index on ties
__device__ __forceinline__ void part_merge(Part& a, const Part& b) {
  const float mm = fmaxf(a.m, b.m);
  if (b.m > a.m || (b.m == a.m && b.idx < a.idx)) a.idx = b.idx;
  a.nan |= b.nan;
  if (mm == kNegInf) return;  // both empty: z = s = 0
  float z = 0.f, s = 0.f;
  if (a.m != kNegInf) {
    const float d = a.m - mm, f = __expf(d);
    z += a.z * f;
    s += (a.s + d * a.z) * f;
  }
  if (b.m != kNegInf) {
    const float d = b.m - mm, f = __expf(d);
    z += b.z * f;
    s += (b.s + d * b.z) * f;
  }
  a.m = mm;
  a.z = z;
  a.s = s;
}

// Kernel 2, one wavefront per row: one pass over the row's partial states. Lane l
// merges states l, l+64, ... in ascending order (loads batched four deep), then the
// 64 lane states combine along a fixed butterfly, so the result is reproducible.
constexpr int kMergeBatch = 4;
__global__ void __launch_bounds__(64)
entropy_merge_kernel(const Part* __restrict__ parts, int splits, float* __restrict__ H,
                     int32_t* __restrict__ amax, float* __restrict__ conf) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const Part* pr = parts + (int64_t)row * splits;
  Part acc{kNegInf, 0.f, 0.f, 0x7fffffff, 0, {0, 0, 0}};
  for (int s0 = 0; s0 < splits; s0 += 64 * kMergeBatch) {
    Part p[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const int q = s0 + lane + 64 * u;
      if (q < splits) p[u] = pr[q];
      else p[u] = Part{kNegInf, 0.f, 0.f, 0x7fffffff, 0, {0, 0, 0}};
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) part_merge(acc, p[u]);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    Part b;
    b.m = __shfl_xor(acc.m, o);
    b.z = __shfl_xor(acc.z, o);
    b.s = __shfl_xor(acc.s, o);
    b.idx = __shfl_xor(acc.idx, o);
    b.nan = __shfl_xor(acc.nan, o);
    if (lane & o) {  // the lower lanes' state first, on every lane alike
      Part lo = b;
      part_merge(lo, acc);
      acc = lo;
    } else {
      part_merge(acc, b);
    }
  }
  if (lane == 0) {
    const bool bad = acc.nan || acc.m == kNegInf;
    H[row] = bad ? NAN : __logf(acc.z) - acc.s / acc.z;
    conf[row] = bad ? NAN : 1.0f / acc.z;
    amax[row] = acc.idx == 0x7fffffff ? 0 : acc.idx;
  }
}

// ---------------------------------------------------------------- single-launch reduction
// ec_entropy_max in one launch. Workgroup b reduces slice split = b / rows of row
// row = b % rows (S slices per row, S = 1 when there are enough rows to cover the CUs):
// every element is read once, the loads of a pass are issued before their use, each
// element takes one exp2 against its lane's running maximum, and lanes and wavefronts
// merge along a fixed order.
//
// S > 1: every workgroup but the last publishes its state as four 64-bit words
// {call tag, value} (device-scope atomic stores). The last workgroup of the grid polls
// all of them with device-scope atomic loads until every word carries the call's tag,
// merges each row's states in slice order, writes the rows' entropy, argmax and
// confidence, and takes E over the selected rows: one cross-workgroup hop per call.
// S = 1: each workgroup writes its own row; with E requested it publishes the row's
// entropy as one tagged word and the last workgroup waits for all of them.
// No word can be read before it is written in this call (the tag is new for every
// call) and no fence is needed (each word carries its own tag). The last workgroup
// clears every tag it consumed, so a replay of the same launch with the same tag (a
// captured graph) cannot read last replay's words. It was dispatched after every
// workgroup it waits for, which never wait themselves; each wait is also bounded
// (after kSpinLimit polls the rows concerned read as NaN).
constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFU = 8;                 // 16-byte vectors per lane per pass
constexpr int kSpinLimit = 1 << 22;    // polls before a wait gives up (far beyond any normal wait)
constexpr int kMaxSplits = 256;
constexpr int kMaxStates = 512;        // rows x S when S > 1 (S > 1 only below 256 rows)

__device__ __forceinline__ void tag_store(uint64_t* p, uint32_t tag, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// waits until each of the N words at p carries `tag` (the N loads of a poll are issued
// together: one memory round trip per poll); false if the wait gave up
template <int N>
__device__ __forceinline__ bool tag_wait(uint64_t* p, uint32_t tag, uint32_t* v) {
  for (int it = 0; it < kSpinLimit; ++it) {
    uint64_t w[N];
#pragma unroll
    for (int i = 0; i < N; ++i) w[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool all = true;
#pragma unroll
    for (int i = 0; i < N; ++i) all = all && (uint32_t)(w[i] >> 32) == tag;
    if (all) {
#pragma unroll
      for (int i = 0; i < N; ++i) v[i] = (uint32_t)w[i];
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Wavefront reductions: a butterfly inside each row of 16 lanes (DPP quad permutes, then
// the half-row and row mirrors: every lane of a row ends with the row's total), then the
// four row totals read from lanes 0, 16, 32, 48 and combined in that order. Results are
// uniform over the wavefront and independent of timing.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  if constexpr (sizeof(T) == 4 && std::is_same<T, float>::value) {
    v = op(v, dpp_f<0xB1>(v));   // quad_perm [1, 0, 3, 2]
    v = op(v, dpp_f<0x4E>(v));   // quad_perm [2, 3, 0, 1]
    v = op(v, dpp_f<0x141>(v));  // row_half_mirror
    v = op(v, dpp_f<0x140>(v));  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return op(op(r0, r1), op(r2, r3));
  } else {
    v = op(v, dpp_i<0xB1>(v));
    v = op(v, dpp_i<0x4E>(v));
    v = op(v, dpp_i<0x141>(v));
    v = op(v, dpp_i<0x140>(v));
    const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    return op(op(r0, r1), op(r2, r3));
  }
}

// The wavefront's lane states (m, z, s2 in log2 units against the lane's own m, first
// index of m, NaN flag) -> one state: the largest m, z and s2 rescaled to it and summed,
// the smallest index among the lanes holding that m. Empty lanes have m = -inf.
__device__ __forceinline__ void wave_state(float m, float z, float s2, int idx, int nan, float& M, float& Z,
                                           float& S2, int& I, int& N) {
  M = wave_reduce(m, [](float a, float b) { return fmaxf(a, b); });
  float zz = 0.f, ss = 0.f;
  if (m != kNegInf) {  // then M is finite too
    const float d = (m - M) * kLog2e, f = __builtin_amdgcn_exp2f(d);
    zz = z * f;
    ss = (s2 + d * z) * f;
  }
  const auto add = [](float a, float b) { return a + b; };
  Z = wave_reduce(zz, add);
  S2 = wave_reduce(ss, add);
  I = wave_reduce(m == M ? idx : 0x7fffffff, [](int a, int b) { return a < b ? a : b; });
  N = wave_reduce(nan, [](int a, int b) { return a | b; });
}

// online update of a lane's state (m, z, s2, idx) by one pass of NV values: x[q] is
// element blk + ((q / E) kFThreads + tid) E + q % E (increasing in q); -inf entries are
// empty. A NaN value is skipped by the maximum and turns z into NaN through its
// exponential; only a pass with no finite value is scanned for NaN explicitly.
template <int NV, int E>
__device__ __forceinline__ void lane_update(const float* x, int blk, int tid, float& m, float& z, float& s2,
                                            int& idx, int& has_nan) {
  float cm = kNegInf;
#pragma unroll
  for (int q = 0; q < NV; ++q) cm = fmaxf(cm, x[q]);
  if (cm == kNegInf) {  // nothing finite here: a NaN would not reach z below, so look for one
#pragma unroll
    for (int q = 0; q < NV; ++q) has_nan |= x[q] != x[q];
  }
  if (cm > m) {  // a strictly larger maximum moves idx to its first occurrence in this pass
    int qi = 0;
#pragma unroll
    for (int q = NV - 1; q >= 0; --q) qi = x[q] == cm ? q : qi;
    idx = blk + ((qi / E) * kFThreads + tid) * E + qi % E;
    if (m != kNegInf) {  // rescale the sums to the new maximum
      const float dl = (m - cm) * kLog2e, f = __builtin_amdgcn_exp2f(dl);
      s2 = (s2 + dl * z) * f;
      z *= f;
    }
    m = cm;
  }
  if (m != kNegInf) {
    const float mb = m * kLog2e;
    float t[NV], e[NV];
#pragma unroll
    for (int q = 0; q < NV; ++q) t[q] = fmaf(x[q], kLog2e, -mb);
#pragma unroll
    for (int q = 0; q < NV; ++q) e[q] = __builtin_amdgcn_exp2f(t[q]);
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      z += e[q];
      s2 = fmaf(fmaxf(t[q], -1000.f), e[q], s2);  // -inf logit: -1000 * 0 = 0
    }
  }
}

// one pass of whole vectors at blk: FULL = every vector of the pass lies below hiv (no
// masking); otherwise vectors at or past hiv re-read the slice's first vector (so every
// load is issued unconditionally) and are masked to -inf
template <typename T, bool FULL>
__device__ __forceinline__ void vec_pass(const T* __restrict__ base, int blk, int lo, int hiv, int tid, float& m,
                                         float& z, float& s2, int& idx, int& has_nan) {
  constexpr int E = Vec<T>::E;
  v4u u[kFU];
#pragma unroll
  for (int k = 0; k < kFU; ++k) {
    const int j = blk + (k * kFThreads + tid) * E;
    u[k] = *reinterpret_cast<const v4u*>(base + (FULL || j < hiv ? j : lo));
  }
  float x[kFU * E];
#pragma unroll
  for (int k = 0; k < kFU; ++k) {
    Vec<T>::unpack(u[k], x + k * E);
    if (!FULL && blk + (k * kFThreads + tid) * E >= hiv) {
#pragma unroll
      for (int e = 0; e < E; ++e) x[k * E + e] = kNegInf;
    }
  }
  // two halves, so that the first half's arithmetic runs while the second half's loads
  // are still in flight
  constexpr int H = kFU / 2;
  lane_update<H * E, E>(x, blk, tid, m, z, s2, idx, has_nan);
  lane_update<H * E, E>(x + H * E, blk + H * kFThreads * E, tid, m, z, s2, idx, has_nan);
}

// partial state of elements [lo, hi) of one row over the workgroup (valid in thread 0).
// Whole vectors [lo, hiv) go through vec_pass; the < E elements of a ragged end [hiv, hi)
// (or every element, when the row is not 16-byte aligned) follow one per thread.
template <typename T, bool VEC>
__device__ Part slice_state(const T* __restrict__ base, int lo, int hi, Part* red) {
  constexpr int E = Vec<T>::E;
  constexpr int P = kFThreads * kFU * E;  // elements per pass
  const int tid = threadIdx.x;
  float m = kNegInf, z = 0.f, s2 = 0.f;  // s2 = sum (x - m) log2(e) e^(x - m), against this lane's m
  int idx = 0x7fffffff, has_nan = 0;
  int hiv = lo;
  if (VEC) {
    hiv = lo + ((hi - lo) / E) * E;
    for (int blk = lo; blk < hiv; blk += P) {
      if (blk + P <= hiv) vec_pass<T, true>(base, blk, lo, hiv, tid, m, z, s2, idx, has_nan);
      else vec_pass<T, false>(base, blk, lo, hiv, tid, m, z, s2, idx, has_nan);
    }
  }
  for (int j = hiv + tid; j < hi; j += kFThreads) {  // one element per thread
    const float xt[1] = {to_f(base[j])};
    lane_update<1, 1>(xt, j, 0, m, z, s2, idx, has_nan);
  }
  // lanes, then wavefronts (wavefront 0 reduces the kFWaves wavefront states the same way);
  // a NaN among finite values has reached z through its exponential
  float M, Z, S2;
  int I, N;
  wave_state(m, z, s2, idx, has_nan | (z != z), M, Z, S2, I, N);
  if ((tid & 63) == 0) red[tid >> 6] = Part{M, Z, S2, I, N, {0, 0, 0}};
  __syncthreads();
  Part p{kNegInf, 0.f, 0.f, 0x7fffffff, 0, {0, 0, 0}};
  if (tid < 64) {
    const Part w = tid < kFWaves ? red[tid] : Part{kNegInf, 0.f, 0.f, 0x7fffffff, 0, {0, 0, 0}};
    wave_state(w.m, w.z, w.s, w.idx, w.nan, M, Z, S2, I, N);
    p = Part{M, Z, S2 * kLn2, I, N, {0, 0, 0}};
  }
  return p;
}

__device__ __forceinline__ float row_entropy(const Part& a) {
  return a.nan || a.m == kNegInf ? NAN : __logf(a.z) - a.s / a.z;
}

__device__ __forceinline__ float write_row(const Part& a, int row, float* H, int32_t* amax, float* conf) {
  const float h = row_entropy(a);
  H[row] = h;
  conf[row] = a.nan || a.m == kNegInf ? NAN : 1.0f / a.z;
  amax[row] = a.idx == 0x7fffffff ? 0 : a.idx;
  return h;
}

// E = max over the selected rows of h_of(row) (NaN if any is NaN, a selection is out of
// range, or `fail`); every thread of the workgroup calls it, thread 0 writes *emax.
// sel_pre is the row thread tid selects (loaded at the kernel's start, so that no global
// load sits on the path after the states arrive); threads past the first kFThreads
// selections read theirs here.
template <typename HOf>
__device__ void emax_over(const int32_t* __restrict__ sel, int n_sel, int sel_pre, int rows, int fail, HOf h_of,
                          float* emax_sh, int* enan_sh, float* __restrict__ emax) {
  const int tid = threadIdx.x;
  float mx = kNegInf;
  int nan = fail;
  const int n = sel ? n_sel : rows;
  for (int i = tid; i < n; i += kFThreads) {
    const int r = i == tid ? sel_pre : (sel ? sel[i] : i);
    if (r < 0 || r >= rows) {
      nan = 1;
      continue;
    }
    const float h = h_of(r);
    if (h != h) nan = 1;
    else mx = fmaxf(mx, h);
  }
  mx = wave_reduce(mx, [](float a, float b) { return fmaxf(a, b); });
  nan = wave_reduce(nan, [](int a, int b) { return a | b; });
  if ((tid & 63) == 0) {
    emax_sh[tid >> 6] = mx;
    enan_sh[tid >> 6] = nan;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kFWaves; ++w) {
      mx = fmaxf(mx, emax_sh[w]);
      nan |= enan_sh[w];
    }
    *emax = nan ? NAN : mx;
  }
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(kFThreads)
entropy_fused_kernel(const T* __restrict__ logits, int rows, int V, int64_t stride, int S, int chunk,
                     const int32_t* __restrict__ sel, int n_sel, float* __restrict__ H,
                     int32_t* __restrict__ amax, float* __restrict__ conf, float* __restrict__ emax,
                     uint64_t* __restrict__ parts, uint64_t* __restrict__ hpub, uint32_t tag) {
  __shared__ Part red[kFWaves];
  __shared__ Part got[kMaxStates];
  __shared__ float h_sh[kMaxStates];
  __shared__ int fail_sh;
  __shared__ float emax_sh[kFWaves];
  __shared__ int enan_sh[kFWaves];
  const int b = blockIdx.x, split = b / rows, row = b % rows, tid = threadIdx.x;
  const bool last = b == (int)gridDim.x - 1;
  int sel_pre = -1;
  if (last && emax && tid < (sel ? n_sel : rows)) sel_pre = sel ? sel[tid] : tid;
  const int lo = min(V, split * chunk), hi = min(V, lo + chunk);
  Part p = slice_state<T, VEC>(logits + (int64_t)row * stride, lo, hi, red);

  if (S == 1) {  // the workgroup holds its whole row
    if (tid == 0) {
      const float h = write_row(p, row, H, amax, conf);
      if (emax && !last) tag_store(hpub + row, tag, __float_as_uint(h));
      if (last) h_sh[0] = h;
    }
    if (!emax || !last) return;
    // the last workgroup: E once every other row has published its entropy
    if (tid == 0) fail_sh = 0;
    __syncthreads();
    for (int r = tid; r < rows - 1; r += kFThreads) {
      uint32_t w = 0;
      if (!tag_wait<1>(hpub + r, tag, &w)) atomicOr(&fail_sh, 1);
    }
    __syncthreads();
    const float h_last = h_sh[0];
    emax_over(sel, n_sel, sel_pre, rows, fail_sh, [&](int r) {
      return r == rows - 1 ? h_last
                           : __uint_as_float((uint32_t)__hip_atomic_load(hpub + r, __ATOMIC_RELAXED,
                                                                        __HIP_MEMORY_SCOPE_AGENT));
    }, emax_sh, enan_sh, emax);
    __syncthreads();
    for (int r = tid; r < rows - 1; r += kFThreads) tag_store(hpub + r, 0u, 0u);  // consumed
    return;
  }

  // S > 1: state b of the grid is published at parts[4 b .. 4 b + 3]
  if (!last) {
    if (tid == 0) {
      uint64_t* q = parts + (int64_t)b * 4;
      tag_store(q + 0, tag, __float_as_uint(p.m));
      tag_store(q + 1, tag, __float_as_uint(p.z));
      tag_store(q + 2, tag, __float_as_uint(p.s));
      tag_store(q + 3, tag, (uint32_t)p.idx | (p.nan ? 0x80000000u : 0u));
    }
    return;
  }
  // ---- the last workgroup: collect every other state, merge each row in slice order.
  // Its global stores (the rows' results, E, the cleared tags) are issued only after its
  // last barrier, so no barrier waits for them.
  const int ns = rows * S;
  if (tid == 0) {
    fail_sh = 0;
    got[ns - 1] = p;
  }
  __syncthreads();
  for (int j = tid; j < ns - 1; j += kFThreads) {
    uint32_t w[4] = {0x7fc00000u, 0u, 0u, 0x80000000u};  // read as a NaN state if the wait gives up
    if (!tag_wait<4>(parts + (int64_t)j * 4, tag, w)) atomicOr(&fail_sh, 1);
    got[j] = Part{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), (int)(w[3] & 0x7fffffffu),
                  (int)(w[3] >> 31), {0, 0, 0}};
  }
  __syncthreads();
  Part a{kNegInf, 0.f, 0.f, 0x7fffffff, 0, {0, 0, 0}};
  float h = NAN;
  if (tid < rows) {  // rows < kFThreads whenever S > 1
    a = got[tid];
    for (int k = 1; k < S; ++k) part_merge(a, got[k * rows + tid]);
    if (fail_sh) a.nan = 1;
    h = row_entropy(a);
  }
  const int n = sel ? n_sel : rows;
  if (rows <= 64 && n <= 64) {
    // wavefront 0 holds every row's entropy: E from its registers, no further barrier
    if (emax && tid < 64) {
      const int r = sel_pre;
      const float hr = __shfl(h, r & 63);
      float mx = kNegInf;
      int nan = fail_sh;
      if (tid < n) {
        if (r < 0 || r >= rows || hr != hr) nan = 1;
        else mx = hr;
      }
      mx = wave_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
      nan = wave_reduce(nan, [](int x, int y) { return x | y; });
      if (tid == 0) *emax = nan ? NAN : mx;
    }
  } else if (emax) {
    if (tid < rows) h_sh[tid] = h;
    __syncthreads();
    emax_over(sel, n_sel, sel_pre, rows, fail_sh, [&](int r) { return h_sh[r]; }, emax_sh, enan_sh, emax);
  }
  if (tid < rows) write_row(a, tid, H, amax, conf);
  for (int j = tid; j < ns - 1; j += kFThreads) {
#pragma unroll
    for (int i = 0; i < 4; ++i) tag_store(parts + (int64_t)j * 4 + i, 0u, 0u);  // consumed
  }
}

__global__ void fill_kernel(float* p, float v) { *p = v; }

// slices per row: enough workgroups to cover the CUs, slices of at least 2048 elements
int splits_for(int rows, int vocab) {
  const int by_cus = (256 + rows - 1) / rows;
  const int by_len = (vocab + 2047) / 2048;
  return std::max(1, std::min({by_cus, by_len, kMaxSplits}));
}

}  // namespace

namespace {
// A fresh tag per call: a counter passed through a 32-bit mixing bijection, so that tags
// do not look like the small integers a reused workspace may hold; never 0 (the tag of
// a cleared word).
uint32_t next_tag() {
  static std::atomic<uint32_t> counter{0};
  for (;;) {
    uint32_t t = counter.fetch_add(1, std::memory_order_relaxed) + 0x632BE5ABu;
    t ^= t >> 16;
    t *= 0x85EBCA6Bu;
    t ^= t >> 13;
    t *= 0xC2B2AE35u;
    t ^= t >> 16;
    if (t != 0) return t;
  }
}
}  // namespace

size_t entropy_ws_bytes(int rows, int vocab) {
  if (rows <= 0 || vocab <= 0) return 0;
  // tagged slice states [S][rows][4] and published row entropies [rows], 64-bit words
  return ((size_t)rows * splits_for(rows, vocab) * 4 + (size_t)rows) * sizeof(uint64_t) + 256;
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
  const int E = dt == EC_BF16 ? 8 : 4;
  const int P = kFThreads * kFU * E;  // elements per pass of a workgroup
  int S = splits_for(rows, vocab);
  // slice starts stay 16-byte aligned; where rounding the slice length up to whole passes
  // keeps the number of slices, it is rounded, so that only the last slice of a row has a
  // partial (masked) pass
  int chunk = ((vocab + S - 1) / S + E - 1) / E * E;
  const int whole = (chunk + P - 1) / P * P;
  if (S > 1 && (vocab + whole - 1) / whole == S) chunk = whole;
  EC_REQUIRE(S == 1 || (int64_t)rows * S <= kMaxStates, EC_ERR_UNSUPPORTED,
             "ec_entropy_max: %d rows x %d slices exceed %d slice states", rows, S, kMaxStates);
  uint64_t* parts = (uint64_t*)ws;
  uint64_t* hpub = parts + (size_t)rows * S * 4;
  const uint32_t tag = next_tag();
  const size_t esz = dt == EC_BF16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((stride * esz) % 16 == 0);
  const dim3 grid((unsigned)((int64_t)rows * S));
#define EC_LAUNCH(T, V)                                                                                  \
  entropy_fused_kernel<T, V><<<grid, kFThreads, 0, s>>>((const T*)logits, rows, vocab, stride, S, chunk, \
                                                        sel, n_sel, H, amax, c, emax, parts, hpub, tag)
  if (dt == EC_BF16) {
    if (vec) EC_LAUNCH(bf16, true);
    else EC_LAUNCH(bf16, false);
  } else {
    if (vec) EC_LAUNCH(float, true);
    else EC_LAUNCH(float, false);
  }
#undef EC_LAUNCH
  EC_CHECK_LAUNCH("entropy_fused_kernel");
  return EC_OK;
}

// ---------------------------------------------------------------- allocation-free variant
// Scratch of ec_entropy_max_noalloc: the tagged slice states and row entropies of the
// single-launch reduction, in a device array of the library instead of a caller's
// workspace. It is zero when the code object loads, and every word a call tags is set
// back to zero by the workgroup that consumes it, so each call finds it cleared. One
// array per GPU (each device has its own copy at its own address), shared by every call
// on that GPU: calls that overlap in time on one GPU race.
static __device__ __align__(256) uint64_t scratch[kEntropyScratchBytes / sizeof(uint64_t)];

namespace {
std::atomic<void*> g_scratch_ptr[64];  // device address of `scratch` per device ordinal

// `scratch` is only a host-side stand-in for the array: kernels get its device address,
// looked up once per device with that device current
ec_status scratch_ptr(void** out) {
  int dev = 0;
  EC_CHECK_HIP(hipGetDevice(&dev));
  EC_REQUIRE(dev >= 0 && dev < 64, EC_ERR_UNSUPPORTED, "ec_entropy_max_noalloc: device ordinal %d >= 64", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    EC_CHECK_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    EC_REQUIRE(p != nullptr, EC_ERR_HIP, "ec_entropy_max_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return EC_OK;
}
}  // namespace

ec_status entropy_noalloc(ec_dtype dt, const void* logits, int rows, int vocab, int64_t stride, const int32_t* sel,
                          int n_sel, float* H, int32_t* amax, float* c, float* emax, hipStream_t s) {
  const size_t need = entropy_ws_bytes(rows, vocab);
  EC_REQUIRE(need <= kEntropyScratchBytes, EC_ERR_UNSUPPORTED,
             "ec_entropy_max_noalloc: %d rows of %d need %zu bytes of scratch, above the %zu-byte array", rows,
             vocab, need, (size_t)kEntropyScratchBytes);
  void* p = nullptr;
  const ec_status st = scratch_ptr(&p);
  if (st != EC_OK) return st;
  return entropy(dt, logits, rows, vocab, stride, sel, n_sel, H, amax, c, emax, p, kEntropyScratchBytes, s);
}

ec_status entropy_merge(const EntPart* parts, int rows, int splits, float* H, int32_t* amax, float* c,
                        hipStream_t s) {
  entropy_merge_kernel<<<rows, 64, 0, s>>>(parts, splits, H, amax, c);
  EC_CHECK_LAUNCH("entropy_merge_kernel");
  return EC_OK;
}

}  // namespace ec
