// Row-block GEMMs of the forward, C[M,N] = A[M,K] . B[N,K]^T, with the
// element-wise work of the transformer block fused into the epilogue:
//   EPI_QKV    -- rotary embedding of q and k at the rows' absolute positions,
//                 q to a compact buffer, k and v straight into the layer's
//                 K/V cache at positions rows[m] (the recomputed rows' cache
//                 update of a skip step; every row on a refresh);
//   EPI_RESID  -- residual add into the fp32 hidden state (O-proj, down-proj);
//   EPI_SWIGLU -- two weight matrices (gate, up) share the A tile; the
//                 epilogue writes silu(gate) * up;
//   EPI_STORE  -- plain store (LM head logits).
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 (gfx950). Both operands are
// K-contiguous, so every fragment is one 16-byte LDS read. 256 threads = 4
// wavefronts; a wavefront owns a WM x WN block made of 32x32 MFMA tiles.
// With WN = 128 a wavefront's four column tiles are one attention head
// (columns c and c + 64 sit in tiles j and j + 2 of the same lane and
// register), so the rotary pairs and the gate/up pairs are register-local.
// Tiles are staged global -> registers -> LDS (row stride padded by 16 bytes
// against bank conflicts), double-buffered over BK = 64, with the next tile's
// global loads in flight during the current tile's MFMAs.
//
// Block order is XCD-aware: MI355X dispatches consecutive workgroups round-
// robin over its 8 XCDs (each with its own L2), so block ids are remapped to
// give each XCD a contiguous range in which the M tiles of one weight tile
// are adjacent; a weight tile is then fetched from HBM once and re-read from
// that XCD's L2.
//
// When M x N tiles cannot fill the 256 CUs (skinny M on skip steps, N = d on
// the projections), K is split across workgroups; partial sums go to an fp32
// workspace and a second kernel adds them in a fixed order (deterministic)
// and applies the epilogue.
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;
// native 16-byte vector (a plain vector load/store, unlike the uint4 struct)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr int LDS_STRIDE = BK + 8;  // bf16 elements per LDS row (144 bytes)

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// -------------------------------------------------------------------- epilogue helpers
template <typename T>
__device__ __forceinline__ void epi_qkv_pair(const EpiArgs& e, int m, int col, float x1, float x2) {
  // col: column of the first element of the pair within [0, 3d); partner is col + D/2
  const int d = e.d_model, D = e.head_dim, half = D / 2;
  const int sec = col / d;
  const int hc = col % d;            // column within the q / k / v section
  const int c = hc % D;              // column within the head (< half)
  const int pos = e.rows[m];
  if (sec > 0 && (pos < 0 || pos >= e.seq_len)) return;  // invalid position: no cache write
  float y1 = x1, y2 = x2;
  if (sec < 2 && pos >= 0 && pos < e.seq_len) {
    const float cs = e.rope_cos[(int64_t)pos * half + c];
    const float sn = e.rope_sin[(int64_t)pos * half + c];
    y1 = x1 * cs - x2 * sn;
    y2 = x1 * sn + x2 * cs;
  }
  T* dst;
  if (sec == 0) dst = (T*)e.out + (int64_t)m * d;
  else if (sec == 1) dst = (T*)e.k_cache + (int64_t)pos * d;
  else dst = (T*)e.v_cache + (int64_t)pos * d;
  dst[hc] = from_f<T>(y1);
  dst[hc + half] = from_f<T>(y2);
}

template <typename T>
__device__ __forceinline__ void epi_single(const EpiArgs& e, int m, int col, float x) {
  if (e.kind == EPI_RESID) {
    e.resid[(int64_t)m * e.ldo + col] += x;
  } else {
    ((T*)e.out)[(int64_t)m * e.ldo + col] = from_f<T>(x);
  }
}

template <typename T>
__device__ __forceinline__ void epi_swiglu(const EpiArgs& e, int m, int col, float g, float u) {
  ((T*)e.out)[(int64_t)m * e.ldo + col] = from_f<T>(silu(g) * u);
}

// -------------------------------------------------------------------- block mapping
__device__ __forceinline__ int xcd_remap(int pid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int x = pid % 8, local = pid / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}

// -------------------------------------------------------------------- bf16 MFMA GEMM
// BM x BN workgroup tile, WM x WN per wavefront, (BM/WM)*(BN/WN) wavefronts,
// K staged BKT at a time through two LDS buffers; STAGES register sets hold
// the next K-steps' tiles in flight (prefetch depth).
// DUAL: B rows [0, BN/2) come from B (gate), rows [BN/2, BN) from B2 (up);
//       the workgroup writes BN/2 output columns.
// SPLIT: write raw fp32 partials to `part` ([S][M][ncols]) instead of the epilogue.
template <int BM, int BN, int WM, int WN, int BKT, int STAGES, int EPI, bool DUAL, bool SPLIT>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B,
                 const bf16* __restrict__ B2, int M, int N, int K, int k_chunk, int splits,
                 EpiArgs epi, float* __restrict__ part) {
  constexpr int WAVES_N = BN / WN;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LS = BKT + 8;                    // LDS row stride (bf16), 16-byte pad
  constexpr int CPR = BKT / 8;                   // 16-byte chunks per row
  constexpr int A_VECS = BM * CPR / NT;          // 16-byte vectors per thread
  constexpr int B_VECS = BN * CPR / NT;
  // paired epilogues: a wavefront's first TN/2 column tiles pair with its last TN/2
  // (rotary halves c / c+64 of one head, or gate / up of the same output columns)
  constexpr bool PAIRED = DUAL || EPI == EPI_QKV;
  static_assert(EPI != EPI_QKV || BN == 128, "QKV tiles are one head (128 columns) wide");
  static_assert(!PAIRED || TN % 2 == 0, "paired epilogue needs an even number of column tiles");
  static_assert(A_VECS >= 1 && B_VECS >= 1 && A_VECS * NT == BM * CPR && B_VECS * NT == BN * CPR,
                "tile / thread mismatch");

  extern __shared__ __align__(16) unsigned char smem[];
  bf16* sA = (bf16*)smem;                        // [2][BM][LS]
  bf16* sB = sA + 2 * BM * LS;                   // [2][BN][LS]

  const int MT = (M + BM - 1) / BM;
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = bid % MT;
  const int rest = bid / MT;
  const int kz = rest % splits;
  const int nt = rest / splits;
  const int m0 = mt * BM;
  const int NOUT = DUAL ? BN / 2 : BN;           // output columns per workgroup
  const int n0 = nt * NOUT;                      // first output column (B row for non-dual)
  const int kbeg = kz * k_chunk;
  const int nk = k_chunk / BKT;

  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  const bf16* a_src[A_VECS];
  int a_lds[A_VECS];
#pragma unroll
  for (int i = 0; i < A_VECS; ++i) {
    const int v = tid + i * NT;
    const int r = v / CPR, kv = v % CPR;
    a_src[i] = A + (int64_t)min(m0 + r, M - 1) * K + kbeg + kv * 8;
    a_lds[i] = r * LS + kv * 8;
  }
  const bf16* b_src[B_VECS];
  int b_lds[B_VECS];
#pragma unroll
  for (int i = 0; i < B_VECS; ++i) {
    const int v = tid + i * NT;
    const int r = v / CPR, kv = v % CPR;
    int grow;
    const bf16* mat = B;
    if (DUAL) {
      const bool up = r >= BN / 2;
      mat = up ? B2 : B;
      grow = n0 + (up ? r - BN / 2 : r);
    } else {
      grow = n0 + r;
    }
    b_src[i] = mat + (int64_t)min(grow, N - 1) * K + kbeg + kv * 8;
    b_lds[i] = r * LS + kv * 8;
  }

  // D register sets of prefetched tiles: the global loads of K-step k+D are in
  // flight while step k computes, so D steps of MFMA work cover the load latency
  constexpr int D = STAGES;
  v4u ra[D][A_VECS], rb[D][B_VECS];
#define EC_GLOAD(KT, XA, XB)                                                          \
  do {                                                                                \
    _Pragma("unroll") for (int i_ = 0; i_ < A_VECS; ++i_)                             \
      XA[i_] = *reinterpret_cast<const v4u*>(a_src[i_] + (KT) * BKT);               \
    _Pragma("unroll") for (int i_ = 0; i_ < B_VECS; ++i_)                             \
      XB[i_] = *reinterpret_cast<const v4u*>(b_src[i_] + (KT) * BKT);               \
  } while (0)
#define EC_SSTORE(BUF, XA, XB)                                                        \
  do {                                                                                \
    bf16* a_ = sA + (BUF) * BM * LS;                                                  \
    bf16* b_ = sB + (BUF) * BN * LS;                                                  \
    _Pragma("unroll") for (int i_ = 0; i_ < A_VECS; ++i_)                             \
      *reinterpret_cast<v4u*>(a_ + a_lds[i_]) = XA[i_];                             \
    _Pragma("unroll") for (int i_ = 0; i_ < B_VECS; ++i_)                             \
      *reinterpret_cast<v4u*>(b_ + b_lds[i_]) = XB[i_];                             \
  } while (0)

  int brow[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (PAIRED) {
      const int jj = j % (TN / 2);
      brow[j] = (j < TN / 2 ? 0 : BN / 2) + wn * (WN / 2) + 32 * jj;
    } else {
      brow[j] = wn * WN + 32 * j;
    }
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int lrow = lane % 32, lk = 8 * (lane / 32);
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const bf16* a = sA + buf * BM * LS;
    const bf16* b = sB + buf * BN * LS;
#pragma unroll
    for (int kk = 0; kk < BKT / 16; ++kk) {
      bf16x8 fa[TM], fb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(a + (wm * WM + 32 * i + lrow) * LS + kk * 16 + lk);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(b + (brow[j] + lrow) * LS + kk * 16 + lk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < nk) EC_GLOAD(j, ra[j], rb[j]);
  EC_SSTORE(0, ra[0], rb[0]);
  if (D < nk) EC_GLOAD(D, ra[0], rb[0]);
  __syncthreads();
  for (int kt = 0; kt < nk; kt += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int k = kt + j;
      if (k < nk) {
        compute(k & 1);
        if (k + 1 < nk) {
          EC_SSTORE((k + 1) & 1, ra[(j + 1) % D], rb[(j + 1) % D]);
          if (k + 1 + D < nk) EC_GLOAD(k + 1 + D, ra[(j + 1) % D], rb[(j + 1) % D]);
        }
        __syncthreads();
      }
    }
  }
#undef EC_GLOAD
#undef EC_SSTORE

  // ---------------------------------------------------------------- epilogue
  // acc[i][j][v]: row = m0 + wm*WM + 32i + 8(v/4) + 4(lane/32) + v%4, column lane%32 of tile j
  const int rbase = m0 + wm * WM + 4 * (lane / 32);
  if (SPLIT) {
    const int ncols = DUAL ? 2 * N : N;
    float* dst = part + (int64_t)kz * M * ncols;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int col;
        if (DUAL) {
          const int jj = j % (TN / 2);
          col = (j < TN / 2 ? 0 : N) + n0 + wn * (WN / 2) + 32 * jj + lrow;
        } else {
          col = n0 + brow[j] + lrow;
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = rbase + 32 * i + 8 * (v / 4) + (v % 4);
          if (m < M) dst[(int64_t)m * ncols + col] = acc[i][j][v];
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = rbase + 32 * i + 8 * (v / 4) + (v % 4);
      if (m >= M) continue;
      if (PAIRED) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const float x1 = acc[i][j][v], x2 = acc[i][j + TN / 2][v];
          const int col = n0 + wn * (WN / 2) + 32 * j + lrow;
          if (EPI == EPI_QKV) {
            epi_qkv_pair<bf16>(epi, m, col, x1, x2);
          } else {
            epi_swiglu<bf16>(epi, m, col, x1, x2);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int col = n0 + wn * WN + 32 * j + lrow;
          if (col < N) epi_single<bf16>(epi, m, col, acc[i][j][v]);
        }
      }
    }
  }
}

// -------------------------------------------------------------------- split-K reduction
// One thread per output unit; sums the S partials in order, then the epilogue.
template <typename T>
__global__ void __launch_bounds__(kThreads)
splitk_epilogue_kernel(const float* __restrict__ part, int S, int M, int N, int kind,
                       EpiArgs epi) {
  const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (kind == EPI_QKV) {
    // units: (m, pair) with pair over [0, 3d/2): head-major, c < D/2
    const int half = epi.head_dim / 2;
    const int64_t units_per_row = N / 2;
    if (t >= (int64_t)M * units_per_row) return;
    const int m = (int)(t / units_per_row);
    const int u = (int)(t % units_per_row);
    const int head = u / half, c = u % half;
    const int col = head * epi.head_dim + c;
    float x1 = 0.f, x2 = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = part + ((int64_t)s * M + m) * N;
      x1 += p[col];
      x2 += p[col + half];
    }
    epi_qkv_pair<T>(epi, m, col, x1, x2);
  } else if (kind == EPI_SWIGLU) {
    if (t >= (int64_t)M * N) return;
    const int m = (int)(t / N), col = (int)(t % N);
    float g = 0.f, u = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* p = part + ((int64_t)s * M + m) * (2 * N);
      g += p[col];
      u += p[N + col];
    }
    epi_swiglu<T>(epi, m, col, g, u);
  } else {
    if (t >= (int64_t)M * N) return;
    const int m = (int)(t / N), col = (int)(t % N);
    float x = 0.f;
    for (int s = 0; s < S; ++s) x += part[((int64_t)s * M + m) * N + col];
    epi_single<T>(epi, m, col, x);
  }
}

// -------------------------------------------------------------------- fp32 SIMT GEMM
// Plain fp32 path (fp32 models): one thread per output unit (an element, or
// the pair the rotary / SwiGLU epilogue needs), dot products over K.
__global__ void __launch_bounds__(kThreads)
gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                const float* __restrict__ B2, int M, int N, int K, EpiArgs epi) {
  const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (epi.kind == EPI_QKV) {
    const int half = epi.head_dim / 2;
    const int64_t upr = N / 2;
    if (t >= (int64_t)M * upr) return;
    const int m = (int)(t / upr), u = (int)(t % upr);
    const int col = (u / half) * epi.head_dim + (u % half);
    const float* a = A + (int64_t)m * K;
    const float* b1 = B + (int64_t)col * K;
    const float* b2 = B + (int64_t)(col + half) * K;
    float x1 = 0.f, x2 = 0.f;
    for (int k = 0; k < K; ++k) {
      x1 = fmaf(a[k], b1[k], x1);
      x2 = fmaf(a[k], b2[k], x2);
    }
    epi_qkv_pair<float>(epi, m, col, x1, x2);
  } else if (epi.kind == EPI_SWIGLU) {
    if (t >= (int64_t)M * N) return;
    const int m = (int)(t / N), col = (int)(t % N);
    const float* a = A + (int64_t)m * K;
    const float* bg = B + (int64_t)col * K;
    const float* bu = B2 + (int64_t)col * K;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < K; ++k) {
      g = fmaf(a[k], bg[k], g);
      u = fmaf(a[k], bu[k], u);
    }
    epi_swiglu<float>(epi, m, col, g, u);
  } else {
    if (t >= (int64_t)M * N) return;
    const int m = (int)(t / N), col = (int)(t % N);
    const float* a = A + (int64_t)m * K;
    const float* b = B + (int64_t)col * K;
    float x = 0.f;
    for (int k = 0; k < K; ++k) x = fmaf(a[k], b[k], x);
    epi_single<float>(epi, m, col, x);
  }
}

// -------------------------------------------------------------------- host-side planning
struct Plan {
  int BM, BN, S, k_chunk, MT, NT;
  bool skinny;  // M <= 64: 64-row tiles
};

constexpr int kCUs = 256;

// Tile choice, measured on MI355X for the projection shapes of the 2k / 4k models:
// 128x128 workgroup tiles with 8 or 16 wavefronts (two or four per SIMD hide the LDS
// and global latency); 64x128 tiles when M <= 64 (LM head over the candidates, skinny
// skip steps). K is split only when the tiles cannot give every CU one workgroup.
Plan plan_bf16(int M, int N, int K, int kind) {
  Plan p{};
  const bool dual = kind == EPI_SWIGLU;
  p.skinny = M <= 64 && kind != EPI_QKV && kind != EPI_SWIGLU;
  p.BM = p.skinny ? 64 : 128;
  p.BN = 128;
  const int nout = dual ? p.BN / 2 : p.BN;
  p.MT = (M + p.BM - 1) / p.BM;
  p.NT = (N + nout - 1) / nout;
  const int tiles = p.MT * p.NT;
  int S = 1;
  const int nk = K / BK;
  while (tiles * S < kCUs && S < 8 && nk % (2 * S) == 0 && nk / (2 * S) >= 8) S *= 2;
  p.S = S;
  p.k_chunk = K / S;
  return p;
}

template <int BM, int BN, int WM, int WN, int BKT, int STAGES, int EPI, bool DUAL>
ec_status launch_bf16(const Plan& p, const bf16* A, const bf16* B, const bf16* B2, int M, int N,
                      int K, const EpiArgs& epi, float* part, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const size_t lds = (size_t)2 * (BM + BN) * (BKT + 8) * sizeof(bf16);
  const int grid = p.MT * p.NT * p.S;
  if (p.S > 1) {
    auto kern = gemm_bf16_kernel<BM, BN, WM, WN, BKT, STAGES, EPI, DUAL, true>;
    static bool attr = false;
    if (!attr) {
      EC_CHECK_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      attr = true;
    }
    kern<<<grid, NT, lds, s>>>(A, B, B2, M, N, K, p.k_chunk, p.S, epi, part);
  } else {
    auto kern = gemm_bf16_kernel<BM, BN, WM, WN, BKT, STAGES, EPI, DUAL, false>;
    static bool attr = false;
    if (!attr) {
      EC_CHECK_HIP(hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      attr = true;
    }
    kern<<<grid, NT, lds, s>>>(A, B, B2, M, N, K, p.k_chunk, p.S, epi, part);
  }
  EC_CHECK_LAUNCH("gemm_bf16_kernel");
  return EC_OK;
}

}  // namespace

size_t gemm_splitk_ws_bytes(int M, int N, int K, int kind, bool is_bf16) {
  if (!is_bf16 || M <= 0) return 0;
  Plan p = plan_bf16(M, N, K, kind);
  if (p.S <= 1) return 0;
  const size_t ncols = kind == EPI_SWIGLU ? 2 * (size_t)N : (size_t)N;
  return (size_t)p.S * M * ncols * sizeof(float);
}

ec_status gemm(ec_dtype dt, const void* A, const void* B, const void* B2, int M, int N, int K,
               const EpiArgs& epi, float* splitk_ws, size_t splitk_ws_bytes, hipStream_t s) {
  if (M == 0) return EC_OK;
  const int kind = epi.kind;
  if (dt == EC_F32) {
    const int64_t units = (kind == EPI_QKV) ? (int64_t)M * (N / 2) : (int64_t)M * N;
    const int blocks = (int)((units + kThreads - 1) / kThreads);
    gemm_f32_kernel<<<blocks, kThreads, 0, s>>>((const float*)A, (const float*)B,
                                                (const float*)B2, M, N, K, epi);
    EC_CHECK_LAUNCH("gemm_f32_kernel");
    return EC_OK;
  }
  EC_REQUIRE(K % BK == 0, EC_ERR_UNSUPPORTED, "gemm: K=%d not a multiple of %d", K, BK);
  Plan p = plan_bf16(M, N, K, kind);
  if (kind == EPI_QKV)
    EC_REQUIRE(epi.head_dim == 128 && N % 128 == 0, EC_ERR_UNSUPPORTED,
               "gemm: bf16 QKV needs head_dim 128");
  if (kind == EPI_SWIGLU)
    EC_REQUIRE(N % 128 == 0, EC_ERR_UNSUPPORTED, "gemm: bf16 SwiGLU needs F %% 128 == 0");
  float* part = nullptr;
  if (p.S > 1) {
    const size_t need = gemm_splitk_ws_bytes(M, N, K, kind, true);
    EC_REQUIRE(splitk_ws && splitk_ws_bytes >= need, EC_ERR_WORKSPACE,
               "gemm: split-K workspace %zu < %zu bytes", splitk_ws_bytes, need);
    part = splitk_ws;
  }
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  const bf16* b2 = (const bf16*)B2;
  ec_status st;
  switch (kind) {
    case EPI_QKV:
      st = launch_bf16<128, 128, 32, 64, 64, 3, EPI_QKV, false>(p, a, b, b2, M, N, K, epi, part, s);
      break;
    case EPI_SWIGLU:
      st = launch_bf16<128, 128, 32, 64, 64, 2, EPI_SWIGLU, true>(p, a, b, b2, M, N, K, epi, part, s);
      break;
    case EPI_RESID:
      st = p.skinny
               ? launch_bf16<64, 128, 32, 32, 64, 3, EPI_RESID, false>(p, a, b, b2, M, N, K, epi, part, s)
               : launch_bf16<128, 128, 32, 32, 64, 2, EPI_RESID, false>(p, a, b, b2, M, N, K, epi, part, s);
      break;
    default:
      st = p.skinny
               ? launch_bf16<64, 128, 32, 32, 64, 3, EPI_STORE, false>(p, a, b, b2, M, N, K, epi, part, s)
               : launch_bf16<128, 128, 32, 64, 64, 3, EPI_STORE, false>(p, a, b, b2, M, N, K, epi, part, s);
      break;
  }
  if (st != EC_OK) return st;
  if (p.S > 1) {
    const int64_t units = (kind == EPI_QKV) ? (int64_t)M * (N / 2) : (int64_t)M * N;
    const int blocks = (int)((units + kThreads - 1) / kThreads);
    splitk_epilogue_kernel<bf16><<<blocks, kThreads, 0, s>>>(part, p.S, M, N, kind, epi);
    EC_CHECK_LAUNCH("splitk_epilogue_kernel");
  }
  return EC_OK;
}

}  // namespace ec
