// Row-wise kernels of the forward: embedding gather, RMSNorm, K/V cache
// scatter and the rotary-angle tables.
//
// All are bandwidth-bound and move whole rows with 16-byte vector accesses,
// one workgroup per row (rows are d_model = 2048..4096 elements wide).
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;

// h[i, :] = embed[tokens[rows[i]], :]  (fp32 residual stream)
template <typename T>
__global__ void __launch_bounds__(kThreads)
embed_kernel(const T* __restrict__ table, int vocab, const int32_t* __restrict__ tokens, int L,
             const int32_t* __restrict__ rows, int d, float* __restrict__ h,
             const SeqPtrs tok_of, const int32_t* __restrict__ row_seq) {
  const int i = blockIdx.x;
  const int p = rows[i];
  const int32_t* tk = row_seq ? (const int32_t*)tok_of.p[row_seq[i]] : tokens;
  const int tok = (p >= 0 && p < L) ? tk[p] : -1;
  float* dst = h + (int64_t)i * d;
  if (tok < 0 || tok >= vocab) {  // invalid position or id: zero row
    for (int j = threadIdx.x; j < d; j += kThreads) dst[j] = 0.f;
    return;
  }
  const T* src = table + (int64_t)tok * d;
  for (int j = threadIdx.x; j < d; j += kThreads) dst[j] = to_f(src[j]);
}

// out[i, :] = T(h[src, :] / sqrt(mean(h[src]^2) + eps) * gain), src = idx ? idx[i] : i

__device__ __forceinline__ void store4(bf16* y, float a, float b, float c, float e) {
  bf16x4 o;
  o[0] = (bf16)a;
  o[1] = (bf16)b;
  o[2] = (bf16)c;
  o[3] = (bf16)e;
  *reinterpret_cast<bf16x4*>(y) = o;
}
__device__ __forceinline__ void store4(float* y, float a, float b, float c, float e) {
  *reinterpret_cast<float4*>(y) = make_float4(a, b, c, e);
}
__device__ __forceinline__ float4 load_gain4(const bf16* g) {
  const bf16x4 v = *reinterpret_cast<const bf16x4*>(g);
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
__device__ __forceinline__ float4 load_gain4(const float* g) { return *reinterpret_cast<const float4*>(g); }

// With partials (the split-K residual fusion, idx unused): the row is first updated in
// place, h[i] += sum_s part[s][i] with the partials added in ascending s to a zero
// start (the split-K epilogue's order), and the norm then reads the updated values.
// SP > 0 is the partial count known at compile time: every load of the row and of its
// partials is issued before the first addition, so the partials cost one memory round
// trip rather than one per partial and register slot. SP < 0 takes the count S at run
// time (one partial at a time); SP = 0 has no partials.
__device__ __forceinline__ float4 add_parts(float4 v, const float* __restrict__ part, int S, int M, int i,
                                            int d, int j) {
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(part + ((int64_t)s * M + i) * d + j);
    a.x += p.x;
    a.y += p.y;
    a.z += p.z;
    a.w += p.w;
  }
  return make_float4(v.x + a.x, v.y + a.y, v.z + a.z, v.w + a.w);
}

// NREG float4 per thread hold the row when d <= 4 * kThreads * NREG; each thread sums its
// own float4s in ascending order, and wider rows (read a second time for the scaling
// pass) round alike.
template <typename T, int SP, int NREG>
__global__ void __launch_bounds__(kThreads)
rmsnorm_kernel(float* __restrict__ h, int n_src, const int32_t* __restrict__ idx, int d,
               const T* __restrict__ gain, float eps, T* __restrict__ out, const float* __restrict__ part,
               int S) {
  constexpr bool PARTS = SP != 0;
  const int i = blockIdx.x;
  int src = (!PARTS && idx) ? idx[i] : i;
  if (src < 0 || src >= n_src) src = 0;  // invalid index: normalise row 0 (no out-of-range read)
  float* x = h + (int64_t)src * d;
  const bool in_regs = d <= 4 * kThreads * NREG;
  float4 v[NREG], gv[NREG];
  float ss = 0.f;
  if (in_regs) {
    // slots past the row end load its last float4 (kept in bounds, never used); the gain
    // is loaded with the row, so the scaling pass does not wait for memory again
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const int j = min((threadIdx.x + k * kThreads) * 4, d - 4);
      v[k] = *reinterpret_cast<const float4*>(x + j);
      gv[k] = load_gain4(gain + j);
    }
    if constexpr (SP > 0) {
      float4 a[NREG];
#pragma unroll
      for (int k = 0; k < NREG; ++k) a[k] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int s = 0; s < SP; ++s)
#pragma unroll
        for (int k = 0; k < NREG; ++k) {
          const int j = min((threadIdx.x + k * kThreads) * 4, d - 4);
          const float4 p = *reinterpret_cast<const float4*>(part + ((int64_t)s * n_src + i) * d + j);
          a[k].x += p.x;
          a[k].y += p.y;
          a[k].z += p.z;
          a[k].w += p.w;
        }
#pragma unroll
      for (int k = 0; k < NREG; ++k)
        v[k] = make_float4(v[k].x + a[k].x, v[k].y + a[k].y, v[k].z + a[k].z, v[k].w + a[k].w);
    }
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const int j = (threadIdx.x + k * kThreads) * 4;
      if (j < d) {
        if constexpr (SP < 0) v[k] = add_parts(v[k], part, S, n_src, i, d, j);
        if constexpr (PARTS) *reinterpret_cast<float4*>(x + j) = v[k];
        ss += v[k].x * v[k].x + v[k].y * v[k].y + v[k].z * v[k].z + v[k].w * v[k].w;
      }
    }
  } else {
    for (int j = threadIdx.x * 4; j < d; j += kThreads * 4) {
      float4 w = *reinterpret_cast<const float4*>(x + j);
      if (PARTS) {
        w = add_parts(w, part, SP > 0 ? SP : S, n_src, i, d, j);
        *reinterpret_cast<float4*>(x + j) = w;
      }
      ss += w.x * w.x + w.y * w.y + w.z * w.z + w.w * w.w;
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
  __shared__ float red[kThreads / 64];
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) tot += red[w];
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  T* y = out + (int64_t)i * d;
  if (in_regs) {
#pragma unroll
    for (int k = 0; k < NREG; ++k) {
      const int j = (threadIdx.x + k * kThreads) * 4;
      if (j < d) {
        const float4 g = gv[k];
        store4(y + j, v[k].x * rs * g.x, v[k].y * rs * g.y, v[k].z * rs * g.z, v[k].w * rs * g.w);
      }
    }
  } else {
    for (int j = threadIdx.x * 4; j < d; j += kThreads * 4) {
      const float4 w = *reinterpret_cast<const float4*>(x + j);
      const float4 g = load_gain4(gain + j);
      store4(y + j, w.x * rs * g.x, w.y * rs * g.y, w.z * rs * g.z, w.w * rs * g.w);
    }
  }
}

// cache[idx[i], :] = rows[i, :] for K and V; 16-byte copies.
__global__ void __launch_bounds__(kThreads)
scatter_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc, int64_t L, int vecs_per_row,
               const uint4* __restrict__ kr, const uint4* __restrict__ vr,
               const int32_t* __restrict__ idx) {
  const int i = blockIdx.x;
  const int p = idx[i];
  if (p < 0 || p >= L) return;
  const int64_t so = (int64_t)i * vecs_per_row, dof = (int64_t)p * vecs_per_row;
  for (int j = threadIdx.x; j < vecs_per_row; j += kThreads) {
    kc[dof + j] = kr[so + j];
    vc[dof + j] = vr[so + j];
  }
}

template <typename T>
__global__ void __launch_bounds__(kThreads)
scatter_scalar_kernel(T* __restrict__ kc, T* __restrict__ vc, int64_t L, int width,
                      const T* __restrict__ kr, const T* __restrict__ vr,
                      const int32_t* __restrict__ idx) {
  const int i = blockIdx.x;
  const int p = idx[i];
  if (p < 0 || p >= L) return;
  for (int j = threadIdx.x; j < width; j += kThreads) {
    kc[(int64_t)p * width + j] = kr[(int64_t)i * width + j];
    vc[(int64_t)p * width + j] = vr[(int64_t)i * width + j];
  }
}

// Row gather of two row-major buffers in one launch: blockIdx.y = 0 copies row idx[i]
// of a (a_vecs 16-byte vectors per row) to row i of ao, blockIdx.y = 1 the same for b.
__global__ void __launch_bounds__(kThreads)
gather2_kernel(const int32_t* __restrict__ idx, const uint4* __restrict__ a, uint4* __restrict__ ao, int a_vecs,
               const uint4* __restrict__ b, uint4* __restrict__ bo, int b_vecs) {
  const int i = blockIdx.x;
  const int src = idx[i];
  const uint4* x = blockIdx.y == 0 ? a : b;
  uint4* y = blockIdx.y == 0 ? ao : bo;
  const int nv = blockIdx.y == 0 ? a_vecs : b_vecs;
  for (int j = threadIdx.x; j < nv; j += kThreads) y[(int64_t)i * nv + j] = x[(int64_t)src * nv + j];
}

// cos/sin(pos * base^(-2i/D)) in fp64, stored fp32; one thread per (pos, i).
__global__ void rope_table_kernel(float* c, float* sn, int max_pos, int half, int D, double base) {
  const int64_t n = (int64_t)max_pos * half;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < n;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(t / half), i = (int)(t % half);
    const double theta = (double)p * pow(base, -2.0 * (double)i / (double)D);
    c[t] = (float)cos(theta);
    sn[t] = (float)sin(theta);
  }
}

// register slots per thread: 4 float4 cover rows up to 4096 wide, 8 up to 8192
template <typename T, int SP>
ec_status launch_norm(float* h, int n_src, const int32_t* idx, int n, int d, const T* gain, float eps, T* out,
                      const float* part, int S, hipStream_t s) {
  if (d <= 4 * kThreads * 4)
    rmsnorm_kernel<T, SP, 4><<<n, kThreads, 0, s>>>(h, n_src, idx, d, gain, eps, out, part, S);
  else
    rmsnorm_kernel<T, SP, 8><<<n, kThreads, 0, s>>>(h, n_src, idx, d, gain, eps, out, part, S);
  EC_CHECK_LAUNCH("rmsnorm_kernel");
  return EC_OK;
}
template <typename T>
ec_status resid_norm_t(const float* part, int S, int M, int d, float* h, const T* gain, float eps, T* out,
                       hipStream_t s) {
  switch (S) {
    case 2: return launch_norm<T, 2>(h, M, nullptr, M, d, gain, eps, out, part, S, s);
    case 4: return launch_norm<T, 4>(h, M, nullptr, M, d, gain, eps, out, part, S, s);
    case 8: return launch_norm<T, 8>(h, M, nullptr, M, d, gain, eps, out, part, S, s);
    default: return launch_norm<T, -1>(h, M, nullptr, M, d, gain, eps, out, part, S, s);
  }
}

}  // namespace

ec_status embed(ec_dtype dt, const void* table, int vocab, const int32_t* tokens, int L,
                const int32_t* rows, int n, int d, float* h, hipStream_t s,
                const SeqPtrs* tok, const int32_t* row_seq) {
  const SeqPtrs tp = tok ? *tok : SeqPtrs{};
  if (n == 0) return EC_OK;
  if (dt == EC_BF16)
    embed_kernel<bf16><<<n, kThreads, 0, s>>>((const bf16*)table, vocab, tokens, L, rows, d, h, tp, row_seq);
  else
    embed_kernel<float><<<n, kThreads, 0, s>>>((const float*)table, vocab, tokens, L, rows, d, h, tp, row_seq);
  EC_CHECK_LAUNCH("embed_kernel");
  return EC_OK;
}

ec_status rmsnorm(ec_dtype dt, const float* h, int n_src, const int32_t* idx, int n, int d,
                  const void* gain, float eps, void* out, hipStream_t s) {
  if (n == 0) return EC_OK;
  EC_REQUIRE(d % 4 == 0, EC_ERR_UNSUPPORTED, "rmsnorm: d_model %d not a multiple of 4", d);
  float* hm = const_cast<float*>(h);  // read only without parts
  if (dt == EC_BF16)
    return launch_norm<bf16, 0>(hm, n_src, idx, n, d, (const bf16*)gain, eps, (bf16*)out, nullptr, 0, s);
  return launch_norm<float, 0>(hm, n_src, idx, n, d, (const float*)gain, eps, (float*)out, nullptr, 0, s);
}

ec_status resid_norm(ec_dtype dt, const float* part, int S, int M, int d, float* h, const void* gain,
                     float eps, void* out, hipStream_t s) {
  if (M == 0) return EC_OK;
  EC_REQUIRE(d % 4 == 0, EC_ERR_UNSUPPORTED, "resid_norm: d_model %d not a multiple of 4", d);
  EC_REQUIRE(S >= 1, EC_ERR_ARG, "resid_norm: %d partials", S);
  if (dt == EC_BF16) return resid_norm_t<bf16>(part, S, M, d, h, (const bf16*)gain, eps, (bf16*)out, s);
  return resid_norm_t<float>(part, S, M, d, h, (const float*)gain, eps, (float*)out, s);
}

ec_status scatter(ec_dtype dt, void* kc, void* vc, int64_t L, int width, const void* kr,
                  const void* vr, const int32_t* idx, int n, hipStream_t s) {
  if (n == 0) return EC_OK;
  const size_t esz = dt == EC_BF16 ? 2 : 4;
  const size_t row_bytes = (size_t)width * esz;
  const bool vec = row_bytes % 16 == 0 && (uintptr_t)kc % 16 == 0 && (uintptr_t)vc % 16 == 0 &&
                   (uintptr_t)kr % 16 == 0 && (uintptr_t)vr % 16 == 0;
  if (vec) {
    scatter_kernel<<<n, kThreads, 0, s>>>((uint4*)kc, (uint4*)vc, L, (int)(row_bytes / 16),
                                          (const uint4*)kr, (const uint4*)vr, idx);
  } else if (dt == EC_BF16) {
    scatter_scalar_kernel<bf16><<<n, kThreads, 0, s>>>((bf16*)kc, (bf16*)vc, L, width,
                                                       (const bf16*)kr, (const bf16*)vr, idx);
  } else {
    scatter_scalar_kernel<float><<<n, kThreads, 0, s>>>((float*)kc, (float*)vc, L, width,
                                                        (const float*)kr, (const float*)vr, idx);
  }
  EC_CHECK_LAUNCH("scatter_kernel");
  return EC_OK;
}

ec_status gather_rows2(const int32_t* idx, int n, const void* a, void* ao, size_t a_row_bytes, const void* b,
                       void* bo, size_t b_row_bytes, hipStream_t s) {
  if (n == 0) return EC_OK;
  EC_REQUIRE(a_row_bytes % 16 == 0 && b_row_bytes % 16 == 0 &&
                 (((uintptr_t)a | (uintptr_t)ao | (uintptr_t)b | (uintptr_t)bo) & 15) == 0,
             EC_ERR_UNSUPPORTED, "gather_rows2: rows of %zu and %zu bytes need 16-byte alignment", a_row_bytes,
             b_row_bytes);
  gather2_kernel<<<dim3(n, 2), kThreads, 0, s>>>(idx, (const uint4*)a, (uint4*)ao, (int)(a_row_bytes / 16),
                                                 (const uint4*)b, (uint4*)bo, (int)(b_row_bytes / 16));
  EC_CHECK_LAUNCH("gather2_kernel");
  return EC_OK;
}

ec_status rope_table(float* c, float* sn, int max_pos, int head_dim, double base, hipStream_t s) {
  const int half = head_dim / 2;
  const int64_t n = (int64_t)max_pos * half;
  if (n == 0) return EC_OK;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  rope_table_kernel<<<blocks, 256, 0, s>>>(c, sn, max_pos, half, head_dim, base);
  EC_CHECK_LAUNCH("rope_table_kernel");
  return EC_OK;
}

}  // namespace ec
