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
// Kernel 1: each wavefront owns one slice of one row and reads it exactly once
// from HBM with 16-byte loads, all issued up front (U vectors per lane held in
// registers; consecutive lanes read consecutive vectors). The slice max and its
// first index come from DPP wavefront reductions (no LDS, no barrier); then
// every element is exponentiated once against the slice max (exp2 of
// x log2 e - max log2 e, one FMA) and Z, S are summed the same way. No
// per-element rescaling and no data reread. A NaN logit is skipped by the max
// but turns Z into NaN, so the row's entropy and confidence come out NaN.
// Kernel 2 (grid: rows, one wavefront each): merges the slices of a row in a
// fixed order (deterministic) and writes entropy / argmax / confidence.
// Kernel 3 (one workgroup, only when E is requested): max over selected rows.
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int kU = 2;  // 16-byte vectors per lane per slice (measured best of 1, 2, 4)
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

// ---- wavefront reductions with DPP (no LDS round trip). After the six steps
// lane 63 holds the result over all 64 lanes; readlane broadcasts it.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROW_MASK, 0xF, false);
}
#define EC_WAVE_REDUCE(NAME, TYPE, OP, TO, FROM)                                 \
  __device__ __forceinline__ TYPE NAME(TYPE v) {                                 \
    int x = TO(v);                                                               \
    x = TO(OP(FROM(x), FROM(dpp<0xB1>(x, x))));        /* quad_perm 1,0,3,2 */   \
    x = TO(OP(FROM(x), FROM(dpp<0x4E>(x, x))));        /* quad_perm 2,3,0,1 */   \
    x = TO(OP(FROM(x), FROM(dpp<0x141>(x, x))));       /* row_half_mirror */     \
    x = TO(OP(FROM(x), FROM(dpp<0x140>(x, x))));       /* row_mirror */          \
    x = TO(OP(FROM(x), FROM(dpp<0x142, 0xA>(x, x))));  /* row_bcast15 */         \
    x = TO(OP(FROM(x), FROM(dpp<0x143, 0xC>(x, x))));  /* row_bcast31 */         \
    return FROM(__builtin_amdgcn_readlane(x, 63));                               \
  }
__device__ __forceinline__ int f2i(float v) { return __float_as_int(v); }
__device__ __forceinline__ float i2f(int v) { return __int_as_float(v); }
__device__ __forceinline__ int iid(int v) { return v; }
__device__ __forceinline__ float fadd(float a, float b) { return a + b; }
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }
EC_WAVE_REDUCE(wave_max_f, float, fmaxf, f2i, i2f)
EC_WAVE_REDUCE(wave_sum_f, float, fadd, f2i, i2f)
EC_WAVE_REDUCE(wave_min_i, int, imin, iid, iid)
#undef EC_WAVE_REDUCE

// One wavefront per slice of one row (grid: ceil(slices / 4) x rows, 256 threads).
// Lane l reads vectors l, l+64, ... of the slice (coalesced 1 KB per step), all
// loads issued before any use. Two register passes: the max (and its first
// index), then one exp2 per element against that max for Z and S.
template <typename T, bool VEC, int U>
__global__ void __launch_bounds__(256)
entropy_slice_kernel(const T* __restrict__ logits, int V, int64_t stride, int chunk,
                     int slices, Part* __restrict__ parts) {
  constexpr int E = Vec<T>::E;
  constexpr int NV = U * E;  // values per lane
  const int lane = threadIdx.x % 64;
  const int slice = blockIdx.x * 4 + threadIdx.x / 64, row = blockIdx.y;
  if (slice >= slices) return;
  const T* base = logits + (int64_t)row * stride;
  const int lo = slice * chunk;
  const int hi = min(V, lo + chunk);

  float x[NV];
  int j0[U];
#pragma unroll
  for (int k = 0; k < U; ++k) j0[k] = lo + (lane + 64 * k) * E;
  if (VEC) {
    const int hiv = lo + ((hi - lo) / E) * E;  // end of the whole vectors
    v4u u[U];
#pragma unroll
    for (int k = 0; k < U; ++k)
      if (j0[k] < hiv) u[k] = *reinterpret_cast<const v4u*>(base + j0[k]);
#pragma unroll
    for (int k = 0; k < U; ++k) {
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
    for (int k = 0; k < U; ++k)
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = j0[k] + e;
        x[k * E + e] = j < hi ? to_f(base[j]) : kNegInf;
      }
  }

  // ---- pass 1: max (NaN is skipped here; it reaches Z below and makes H NaN)
  float lm = kNegInf;
#pragma unroll
  for (int q = 0; q < NV; ++q) lm = fmaxf(lm, x[q]);
  const float mv = wave_max_f(lm);
  // first index of the max: only lanes holding it search their values
  int mi = 0x7fffffff;
  if (lm == mv) {
#pragma unroll
    for (int k = U - 1; k >= 0; --k)
#pragma unroll
      for (int e = E - 1; e >= 0; --e)
        if (x[k * E + e] == mv) mi = j0[k] + e;  // ends at this lane's first hit
  }
  mi = wave_min_i(mi);

  // ---- pass 2: Z and S against the max, log2 domain, one exp2 per element:
  // t = x log2e - m log2e, e = 2^t, Z += e, S2 += max(t, -1000) e. The clamp
  // makes a -inf logit (e = 0) add -1000 * 0 = 0 instead of -inf * 0 = NaN;
  // a NaN logit gives e = NaN, which still reaches Z and S.
  float z = 0.f, s2 = 0.f;
  if (mv != kNegInf) {
    const float mb = mv * kLog2e;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
      const float t = fmaf(x[q], kLog2e, -mb);
      const float e = __builtin_amdgcn_exp2f(t);  // v_exp_f32; results below 2^-126 flush to 0
      z += e;
      s2 = fmaf(fmaxf(t, -1000.f), e, s2);
    }
  }
  z = wave_sum_f(z);
  s2 = wave_sum_f(s2);
  if (lane == 0) {
    Part p;
    p.m = mv;
    p.z = z;
    p.s = s2 * kLn2;
    p.idx = mi;
    p.nan = 0;
    parts[(int64_t)row * slices + slice] = p;
  }
}

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

// slice length: kU vectors per lane of one wavefront -> 1024 bf16 / 512 f32 elements
int slice_len(ec_dtype dt) { return 64 * kU * (dt == EC_BF16 ? 8 : 4); }

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
  dim3 grid((splits + 3) / 4, rows);
  if (dt == EC_BF16) {
    if (vec)
      entropy_slice_kernel<bf16, true, kU><<<grid, 256, 0, s>>>((const bf16*)logits, vocab, stride, chunk, splits, parts);
    else
      entropy_slice_kernel<bf16, false, kU><<<grid, 256, 0, s>>>((const bf16*)logits, vocab, stride, chunk, splits, parts);
  } else {
    if (vec)
      entropy_slice_kernel<float, true, kU><<<grid, 256, 0, s>>>((const float*)logits, vocab, stride, chunk, splits, parts);
    else
      entropy_slice_kernel<float, false, kU><<<grid, 256, 0, s>>>((const float*)logits, vocab, stride, chunk, splits, parts);
  }
  EC_CHECK_LAUNCH("entropy_slice_kernel");
  return entropy_merge(parts, rows, splits, H, amax, c, sel, n_sel, emax, s);
}

ec_status entropy_merge(const EntPart* parts, int rows, int splits, float* H, int32_t* amax, float* c,
                        const int32_t* sel, int n_sel, float* emax, hipStream_t s) {
  entropy_merge_kernel<<<rows, 64, 0, s>>>(parts, splits, H, amax, c);
  EC_CHECK_LAUNCH("entropy_merge_kernel");
  if (emax) {
    entropy_emax_kernel<<<1, kThreads, 0, s>>>(H, rows, sel, n_sel, emax);
    EC_CHECK_LAUNCH("entropy_emax_kernel");
  }
  return EC_OK;
}

}  // namespace ec
