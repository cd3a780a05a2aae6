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
// ec_entropy_max in one launch. Workgroup b handles slice split = b / rows of row
// row = b % rows (S slices per row), so the slices of every row are dispatched in
// split order and the last slice of each row comes after every other workgroup but
// the last slices of other rows. A workgroup reduces its slice (every element read
// once, loads of a pass issued before their use, one exp2 per element against the
// running maximum of its lane, lanes and wavefronts merged along a fixed order).
// Slices 0 .. S-2 publish their partial state as four 64-bit words {call tag, value}
// written with device-scope atomic stores; the last slice of the row (the merger)
// polls them with device-scope atomic loads until every word carries the call's tag,
// merges the S states in slice order and writes the row's entropy, argmax and
// confidence. No word can be read before it is written in this call (the tag is new
// for every call) and no fence is needed (each word carries its own tag). The merger
// clears the tags it consumed, so a replay of the same launch with the same tag (a
// captured graph) cannot read last replay's words. When E is requested every merger
// publishes its row's entropy the same way and the last workgroup of the grid (the
// merger of the last row) waits for all of them, takes the maximum over the selected
// rows and clears those tags. Every workgroup a wait depends on was dispatched
// before the waiting one and never waits itself; each wait is also bounded (after
// kSpinLimit polls the row reads as NaN).
constexpr int kFThreads = 512;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFU = 8;                 // 16-byte vectors per lane per pass
constexpr int kSpinLimit = 1 << 22;    // polls before a wait gives up (far beyond any normal wait)
constexpr int kMaxSplits = 256;

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

__device__ __forceinline__ Part shfl_part(const Part& a, int o) {
  Part b;
  b.m = __shfl_xor(a.m, o);
  b.z = __shfl_xor(a.z, o);
  b.s = __shfl_xor(a.s, o);
  b.idx = __shfl_xor(a.idx, o);
  b.nan = __shfl_xor(a.nan, o);
  return b;
}

// online update of a lane's state (m, z, s2, idx) by the values x[0..NV) at indices
// j0[k] + e (increasing in k then e); -inf entries are empty. A NaN value is skipped by
// the maximum and turns z into NaN through its exponential; only a pass with no finite
// value is scanned for NaN explicitly.
template <int NV, int E>
__device__ __forceinline__ void lane_update(const float* x, const int* j0, float& m, float& z, float& s2, int& idx,
                                            int& has_nan) {
  float cm = kNegInf;
#pragma unroll
  for (int q = 0; q < NV; ++q) cm = fmaxf(cm, x[q]);
  if (cm == kNegInf) {  // nothing finite here: a NaN would not reach z below, so look for one
#pragma unroll
    for (int q = 0; q < NV; ++q) has_nan |= x[q] != x[q];
  }
  if (cm > m) {  // a strictly larger maximum moves idx to its first occurrence in this pass
#pragma unroll
    for (int q = NV - 1; q >= 0; --q)
      if (x[q] == cm) idx = j0[q / E] + q % E;
    if (m != kNegInf) {  // rescale the sums to the new maximum
      const float dl = (m - cm) * kLog2e, f = __builtin_amdgcn_exp2f(dl);
      s2 = (s2 + dl * z) * f;
      z *= f;
    }
    m = cm;
  }
  if (m != kNegInf) {
    const float mb = m * kLog2e;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const float t = fmaf(x[q], kLog2e, -mb);
      const float e = __builtin_amdgcn_exp2f(t);
      z += e;
      s2 = fmaf(fmaxf(t, -1000.f), e, s2);  // -inf logit: -1000 * 0 = 0
    }
  }
}

// partial state of elements [lo, hi) of one row over the workgroup (valid in thread 0).
// Whole vectors [lo, hiv): every load of a pass is issued unconditionally (vectors past
// hiv re-read the slice's first vector and are masked to -inf), so the loads of a pass
// are in flight together; the < E elements of a ragged end [hiv, hi) follow one per
// thread.
template <typename T, bool VEC>
__device__ Part slice_state(const T* __restrict__ base, int lo, int hi, Part* red) {
  constexpr int E = Vec<T>::E;
  constexpr int NV = kFU * E;
  const int tid = threadIdx.x;
  float m = kNegInf, z = 0.f, s2 = 0.f;  // s2 = sum (x - m) log2(e) e^(x - m), against this lane's m
  int idx = 0x7fffffff, has_nan = 0;
  const int hiv = VEC ? lo + ((hi - lo) / E) * E : hi;
  for (int blk = lo; blk < hiv; blk += kFThreads * NV) {
    float x[NV];
    int j0[kFU];
#pragma unroll
    for (int k = 0; k < kFU; ++k) j0[k] = blk + (k * kFThreads + tid) * E;
    if (VEC) {
      v4u u[kFU];
#pragma unroll
      for (int k = 0; k < kFU; ++k) u[k] = *reinterpret_cast<const v4u*>(base + (j0[k] < hiv ? j0[k] : lo));
#pragma unroll
      for (int k = 0; k < kFU; ++k) {
        Vec<T>::unpack(u[k], x + k * E);
        if (j0[k] >= hiv) {
#pragma unroll
          for (int e = 0; e < E; ++e) x[k * E + e] = kNegInf;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < kFU; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int j = j0[k] + e;
          const float v = to_f(base[j < hiv ? j : lo]);
          x[k * E + e] = j < hiv ? v : kNegInf;
        }
    }
    // two halves, so that the first half's arithmetic runs while the second half's loads
    // are still in flight
    lane_update<NV / 2, E>(x, j0, m, z, s2, idx, has_nan);
    lane_update<NV / 2, E>(x + NV / 2, j0 + kFU / 2, m, z, s2, idx, has_nan);
  }
  if (VEC && hiv < hi && tid < hi - hiv) {  // ragged end: one element per thread
    const int j0t[1] = {hiv + tid};
    const float xt[1] = {to_f(base[hiv + tid])};
    lane_update<1, 1>(xt, j0t, m, z, s2, idx, has_nan);
  }
  // a NaN among finite values has reached z through its exponential
  Part p{m, z, s2 * kLn2, idx, has_nan | (z != z), {0, 0, 0}};
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {  // symmetric merge: every lane ends with the same state
    const Part q = shfl_part(p, o);
    part_merge(p, q);
  }
  if ((tid & 63) == 0) red[tid >> 6] = p;
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kFWaves; ++w) part_merge(p, red[w]);
  }
  return p;
}

__device__ __forceinline__ void write_row(const Part& a, int row, float* H, int32_t* amax, float* conf, float* h_out) {
  const bool bad = a.nan || a.m == kNegInf;
  const float h = bad ? NAN : __logf(a.z) - a.s / a.z;
  H[row] = h;
  conf[row] = bad ? NAN : 1.0f / a.z;
  amax[row] = a.idx == 0x7fffffff ? 0 : a.idx;
  *h_out = h;
}

template <typename T, bool VEC>
__global__ void __launch_bounds__(kFThreads)
entropy_fused_kernel(const T* __restrict__ logits, int rows, int V, int64_t stride, int S, int chunk,
                     const int32_t* __restrict__ sel, int n_sel, float* __restrict__ H,
                     int32_t* __restrict__ amax, float* __restrict__ conf, float* __restrict__ emax,
                     uint64_t* __restrict__ parts, uint64_t* __restrict__ hpub, uint32_t tag) {
  __shared__ Part red[kFWaves];
  __shared__ Part got[kMaxSplits];
  __shared__ int fail_sh;
  __shared__ float emax_sh[kFWaves];
  __shared__ int enan_sh[kFWaves];
  const int split = blockIdx.x / rows, row = blockIdx.x % rows, tid = threadIdx.x;
  const int lo = min(V, split * chunk), hi = min(V, lo + chunk);
  Part p = slice_state<T, VEC>(logits + (int64_t)row * stride, lo, hi, red);
  uint64_t* pr = parts + (int64_t)row * S * 4;
  if (split < S - 1) {  // publish this slice's state for the row's merger
    if (tid == 0) {
      uint64_t* q = pr + split * 4;
      tag_store(q + 0, tag, __float_as_uint(p.m));
      tag_store(q + 1, tag, __float_as_uint(p.z));
      tag_store(q + 2, tag, __float_as_uint(p.s));
      tag_store(q + 3, tag, (uint32_t)p.idx | (p.nan ? 0x80000000u : 0u));
    }
    return;
  }
  // ---- merger of this row: thread j < S - 1 collects slice j
  if (tid == 0) fail_sh = 0;
  __syncthreads();
  if (tid < S - 1) {
    uint64_t* q = pr + tid * 4;
    uint32_t w[4] = {0x7fc00000u, 0u, 0u, 0x80000000u};  // read as a NaN row if the wait gives up
    if (!tag_wait<4>(q, tag, w)) atomicOr(&fail_sh, 1);
    got[tid] = Part{__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), (int)(w[3] & 0x7fffffffu),
                    (int)(w[3] >> 31), {0, 0, 0}};
#pragma unroll
    for (int i = 0; i < 4; ++i) tag_store(q + i, 0u, 0u);  // consumed
  }
  __syncthreads();
  float h_row = NAN;
  if (tid == 0) {
    Part a = S > 1 ? got[0] : p;
    for (int j = 1; j < S - 1; ++j) part_merge(a, got[j]);
    if (S > 1) part_merge(a, p);
    if (fail_sh) a.nan = 1;
    write_row(a, row, H, amax, conf, &h_row);
    if (emax) tag_store(hpub + row, tag, __float_as_uint(h_row));
  }
  if (!emax || blockIdx.x != gridDim.x - 1) return;
  // ---- the last workgroup: E over the selected rows once every row has published
  // (all rows' words are awaited and cleared, also rows outside the selection)
  if (tid == 0) fail_sh = 0;
  __syncthreads();
  for (int r = tid; r < rows; r += kFThreads) {
    uint32_t w = 0;
    if (!tag_wait<1>(hpub + r, tag, &w)) atomicOr(&fail_sh, 1);
  }
  __syncthreads();
  float mx = kNegInf;
  int nan = fail_sh;
  const int n = sel ? n_sel : rows;
  for (int i = tid; i < n; i += kFThreads) {
    const int r = sel ? sel[i] : i;
    if (r < 0 || r >= rows) {
      nan = 1;
      continue;
    }
    const float h = __uint_as_float((uint32_t)__hip_atomic_load(hpub + r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (h != h) nan = 1;
    else mx = fmaxf(mx, h);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o));
    nan |= __shfl_xor(nan, o);
  }
  if ((tid & 63) == 0) {
    emax_sh[tid >> 6] = mx;
    enan_sh[tid >> 6] = nan;
  }
  __syncthreads();
  for (int r = tid; r < rows; r += kFThreads) tag_store(hpub + r, 0u, 0u);  // consumed
  if (tid == 0) {
    for (int w = 1; w < kFWaves; ++w) {
      mx = fmaxf(mx, emax_sh[w]);
      nan |= enan_sh[w];
    }
    *emax = nan ? NAN : mx;
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
  // tagged slice states [rows][S][4] and published row entropies [rows], 64-bit words
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
  const int S = splits_for(rows, vocab);
  const int E = dt == EC_BF16 ? 8 : 4;
  const int chunk = ((vocab + S - 1) / S + E - 1) / E * E;  // slice starts stay 16-byte aligned
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
