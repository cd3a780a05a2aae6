// Row-block GEMMs of the forward, C[M,N] = A[M,K] . B[N,K]^T, with the
// element-wise work of the transformer block fused into the epilogue:
//   EPI_QKV    -- rotary embedding of q and k at the rows' absolute positions,
//                 q to a compact buffer, k and v straight into the layer's
//                 K/V cache at positions rows[m] (the recomputed rows' cache
//                 update of a skip step; every row on a refresh);
//   EPI_RESID  -- residual add into the fp32 hidden state (O-proj, down-proj);
//   EPI_SWIGLU -- gate and up rows interleaved in one packed weight matrix;
//                 the epilogue writes silu(gate) * up;
//   EPI_STORE  -- plain store (LM head logits).
//
// bf16 path: MFMA v_mfma_f32_32x32x16_bf16 (gfx950), both operands K-contiguous.
// Global tiles are loaded straight into LDS (buffer_load_dwordx4 ... lds) in a
// swizzled, unpadded layout; several K-steps are in flight while the MFMAs of
// the current one run. The rotary and SwiGLU pairs come from packed weights
// (ec_pack_weights) that place the two members of a pair 16 columns apart in
// one 32-column MFMA tile, so the pair is exchanged with one lane swizzle and
// any tile width that is a multiple of 32 works for every epilogue.
//
// Block order is XCD-aware: MI355X dispatches consecutive workgroups round-
// robin over its 8 XCDs (each with its own L2), so block ids are remapped to
// give each XCD a contiguous range of the tile order, in which the row tiles of
// one weight tile are adjacent (a weight tile is fetched from HBM once and
// re-read from that XCD's L2) and row tiles come in groups of four (at large M
// a wave of tiles on one XCD then reads 4 A tiles, not 32).
//
// When M x N tiles cannot fill the 256 CUs (skinny M on skip steps, N = d on
// the projections), K is split across workgroups; partial sums go to an fp32
// workspace and a second kernel adds them in a fixed order (deterministic)
// and applies the epilogue.
#include "ec_internal.h"

#include <math.h>

#include <algorithm>

namespace ec {

namespace {

constexpr int kThreads = 256;
constexpr int BK = 64;
// native 16-byte vector (a plain vector load/store, unlike the uint4 struct)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// -------------------------------------------------------------------- epilogue helpers
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// a <- merge(a, b) of partial softmax states, a covering the lower columns:
// m = max, z and s rescaled to it; argmax = larger value, lower index on ties
__device__ __forceinline__ void part_merge(EntPart& a, const EntPart& b) {
  const float mm = fmaxf(a.m, b.m);
  if (b.m > a.m || (b.m == a.m && b.idx < a.idx)) a.idx = b.idx;
  a.nan |= b.nan;
  if (mm == -INFINITY) return;  // both empty: z = s = 0
  float z = 0.f, s = 0.f;
  if (a.m != -INFINITY) {
    const float dd = a.m - mm, f = __expf(dd);
    z += a.z * f;
    s += (a.s + dd * a.z) * f;
  }
  if (b.m != -INFINITY) {
    const float dd = b.m - mm, f = __expf(dd);
    z += b.z * f;
    s += (b.s + dd * b.z) * f;
  }
  a.m = mm;
  a.z = z;
  a.s = s;
}

// Rotary pair (x1, x2) at columns (col, col + D/2) of the [3d] q|k|v output, col in
// the first half of its head. WHICH bit 0 writes the rotated first element, bit 1
// the second (q to the compact buffer, k and v to the cache row of position rows[m]).
template <typename T>
__device__ __forceinline__ void epi_qkv_pair(const EpiArgs& e, int m, int col, float x1, float x2,
                                             int which = 3) {
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
  else dst = kv_dst<T>(e, m, sec == 2) + (int64_t)pos * d;
  if (which & 1) dst[hc] = from_f<T>(y1);
  if (which & 2) dst[hc + half] = from_f<T>(y2);
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
constexpr int kGroupM = 4;  // row tiles per group of the tile order

// -------------------------------------------------------------------- bf16 MFMA GEMM
// Packed weight layouts (built once by ec_pack_weights) put the two operands of
// every paired epilogue 16 columns apart inside one 32-column MFMA tile, so a
// lane finds its partner in lane ^ 16 of the same accumulator register:
//   rotary (QKV):  inside each head of D columns, 32-column group g holds the
//                  first-half columns 16g .. 16g+15 followed by their partners
//                  D/2 + 16g .. D/2 + 16g + 15;
//   SwiGLU:        [2F, d] with 32-row group g = gate rows 16g .. 16g+15, then up
//                  rows 16g .. 16g+15.
// Any column tile that is a multiple of 32 then keeps every pair in one wavefront.
typedef __attribute__((address_space(1))) void glb_void_t;
typedef __attribute__((address_space(1))) bf16x4 gbf16x4;

// workgroup barrier for LDS produced by direct-to-LDS loads: the waits are explicit
// (the loads are tracked by vmcnt only), the fences keep the compiler from moving
// LDS accesses across it
__device__ __forceinline__ void lds_stage_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// C tile BM x BN from A[M, K] (row stride K) and B[N, K] (row stride K), bf16 in,
// fp32 accumulate on v_mfma_f32_32x32x16_bf16. Wavefront tile WM x WN.
//
// Staging: K advances 64 at a time; each stage of LDS holds BM + BN rows of 128
// bytes, unpadded, with the 16-byte chunk c of row r stored at chunk c ^ ((r/2) % 8)
// so that the 32 rows a fragment read touches fall in distinct banks. Global tiles
// go straight to LDS with buffer_load_dwordx4 ... lds (no staging registers; the
// buffer form, unlike the flat one, is tracked by vmcnt alone): lane l
// of a load instruction fills bytes 16 l of the wavefront's 1 KB slice, and is
// given the global address of the chunk that belongs there. NSTG stages rotate;
// AHEAD of them are in flight. With LATE the stage refilled after the barrier of
// K-step t is the one read during step t-1 (no LDS wait before the barrier);
// otherwise it is the one just read (deeper prefetch, an LDS wait first). With NSB > 0
// the B tiles have a ring of their own, NSB stages after the A stages: the weights,
// streamed from HBM, are requested NSB - NSTG K-steps ahead of the activations, which
// come from L2 (the 256x192 refresh tile: 2 A + 4 B stages, all 160 KB of LDS).
//
// Fragment reads of the next 16-wide K slice are issued in the middle of the
// current slice's MFMAs; the first slice of K-step t+1 is read right after the
// barrier that publishes it.
template <int BM, int BN, int WM, int WN, int NSTG, bool LATE, int EPI, bool SPLIT, int BKS = 64, int NSB = 0>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B, int M, int N, int K,
                 int k_chunk, int splits, EpiArgs epi, float* __restrict__ part) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NT = NW * 64;
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int CPR = BKS / 8;                     // 16-byte chunks per tile row
  constexpr int ROWB = BKS * 2;                    // LDS bytes per tile row
  constexpr int NS = BKS / 16;                     // 16-wide K slices per K-step
  constexpr int SWS = CPR == 8 ? 1 : 2;            // chunk c of row r sits at c ^ ((r >> SWS) % CPR)
  constexpr int STAGE = (BM + BN) * ROWB;
  constexpr int LPA = BM * CPR / NT, LPB = BN * CPR / NT, LPT = LPA + LPB;
  static_assert(BKS == 32 || BKS == 64, "K-step of 32 or 64");
  constexpr int AHEAD = LATE ? NSTG - 1 : NSTG;   // stages in flight
  constexpr int RD_AT = (TM * TN) / 2;             // fragment reads after this many MFMAs
  static_assert(WM % 32 == 0 && WN % 32 == 0 && BM % WM == 0 && BN % WN == 0, "tile shape");
  static_assert(LPA >= 1 && LPB >= 1 && LPA * NT == BM * CPR && LPB * NT == BN * CPR, "load split");
  static_assert(AHEAD >= 2 && (AHEAD - 1) * LPT < 64, "pipeline depth");
  // NSB > 0: the B (weight) tiles get a ring of their own, NSB stages deep, after the NSTG
  // stages of A tiles; both rings refill the stage read during the K-step that just ended
  constexpr bool ASYM = NSB > 0;
  constexpr int SA = BM * ROWB, SB = BN * ROWB;
  constexpr int B_RING = ASYM ? NSTG * SA : 0;
  constexpr int LDS_BYTES = ASYM ? NSTG * SA + NSB * SB : NSTG * STAGE;
  // (the waits of the separate ring below are written for 2 A stages and at least 3 B stages)
  static_assert(!ASYM || (!LATE && NSTG == 2 && NSB >= 3 && NSTG * LPA + NSB * LPB < 64), "separate B ring");
  extern __shared__ __align__(16) unsigned char smem[];

  const int MT = (M + BM - 1) / BM;
  // tile order: groups of kGroupM row tiles; inside a group the row tile varies
  // fastest, then the (weight tile, K split) pair, so any 32 consecutive tiles (one
  // XCD's share of a wave) cover at most kGroupM row tiles and re-read few A tiles
  const int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int ntk = ((int)gridDim.x / MT);  // weight tiles x splits
  const int per_group = kGroupM * ntk;
  const int first_m = (bid / per_group) * kGroupM;
  const int gm = min(MT - first_m, kGroupM);
  const int in_group = bid % per_group;
  const int mt = first_m + in_group % gm;
  const int rest = in_group / gm;
  const int kz = rest % splits;
  const int nt = rest / splits;
  const int m0 = mt * BM, n0 = nt * BN;
  const int kbeg = kz * k_chunk;
  const int nk = k_chunk / BKS;
  // With one row tile (skinny M: the projections of skip steps) and at least 64 weight
  // tiles, the K loop of weight tile nt starts at step rot and wraps: tiles running at the
  // same time then read different K columns, which spreads their weight rows (K x 2 bytes
  // apart) over the L2 channels instead of one (up to 18 % faster at 17 .. 256 rows).
  // With several row tiles the tiles of a group walk K together to share A in L2, and
  // with few weight tiles the K splits already spread the reads, so there is no rotation;
  // nor for the LM head with the entropy epilogue (988 weight tiles), which it made 10 %
  // slower. The order depends only on the weight tile and the plan.
  const int rot = (EPI != EPI_ENTROPY && EPI != EPI_STORE && MT == 1 && ntk / splits >= 64)
                      ? (int)(((unsigned)nt * 5u) % (unsigned)nk) : 0;

  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;

  // Direct-to-LDS loads through buffer resources (buffer_load_dwordx4 ... lds): the
  // per-lane byte offset of each load is fixed, the K-step advances the scalar
  // offset. A rows past M get the offset M*K*2, the end of A's resource: out of range,
  // so the load returns zeros without a memory access (a skinny product's row tile
  // then moves only its M real rows). B rows past N clamp to the last row. Products
  // of such rows land in rows / columns the epilogue skips.
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(A, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(B, (int64_t)N * K * 2);
  int oa[LPA], ob[LPB];
#pragma unroll
  for (int i = 0; i < LPA; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    const int r = q / CPR, c = (q % CPR) ^ ((r >> SWS) & (CPR - 1));
    oa[i] = m0 + r < M ? (int)(((int64_t)(m0 + r) * K + kbeg + c * 8) * 2) : (int)((int64_t)M * K * 2);
  }
#pragma unroll
  for (int i = 0; i < LPB; ++i) {
    const int q = (i * NW + wave) * 64 + lane;
    const int r = q / CPR, c = (q % CPR) ^ ((r >> SWS) & (CPR - 1));
    ob[i] = (int)(((int64_t)min(n0 + r, N - 1) * K + kbeg + c * 8) * 2);
  }
  auto issue_a = [&](int kt, int stage) __attribute__((always_inline)) {
    unsigned char* base = smem + stage * (ASYM ? SA : STAGE);
    const int ks = (kt + rot < nk ? kt + rot : kt + rot - nk) * BKS * 2;
#pragma unroll
    for (int i = 0; i < LPA; ++i) buffer_load_lds16(rA, base + (i * NW + wave) * 1024, oa[i], ks);
  };
  auto issue_b = [&](int kt, int stage) __attribute__((always_inline)) {
    unsigned char* base = ASYM ? smem + B_RING + stage * SB : smem + stage * STAGE + BM * ROWB;
    const int ks = (kt + rot < nk ? kt + rot : kt + rot - nk) * BKS * 2;
#pragma unroll
    for (int i = 0; i < LPB; ++i) buffer_load_lds16(rB, base + (i * NW + wave) * 1024, ob[i], ks);
  };
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    issue_a(kt, stage);
    issue_b(kt, stage);
  };

  // fragment addresses: A/B operand of lane = row lane%32 of the tile, K chunk
  // 2*kk + lane/32; the swizzle term depends only on the row bits below 32
  const int lrow = lane % 32, hi = lane / 32;
  const int swr = (lrow >> SWS) & (CPR - 1);
  const int a_row = (wm * WM + lrow) * ROWB;
  const int b_row = (ASYM ? 0 : BM * ROWB) + (wn * WN + lrow) * ROWB;
  int koff[NS];
#pragma unroll
  for (int kk = 0; kk < NS; ++kk) koff[kk] = ((2 * kk + hi) ^ swr) * 16;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  bf16x8 fa[2][TM], fb[2][TN];
  // fragment reads of K slice kk from the A stage at base_a and the B stage at base_b
  auto rdfrag = [&](const unsigned char* base_a, const unsigned char* base_b, int kk, int slot)
                    __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(base_a + a_row + i * 32 * ROWB + koff[kk]);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(base_b + b_row + j * 32 * ROWB + koff[kk]);
  };
  auto a_stage = [&](int st) __attribute__((always_inline)) { return smem + st * (ASYM ? SA : STAGE); };
  auto b_stage = [&](int st) __attribute__((always_inline)) {
    return ASYM ? smem + B_RING + st * SB : smem + st * STAGE;
  };
  // MFMAs on fragment slot ms; the reads of (stage, kk) into slot rs go after RD_AT of them
  auto slice = [&](int ms, const unsigned char* base_a, const unsigned char* base_b, int kk, int rs)
                   __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < TM * TN; ++q) {
      if (q == RD_AT) {
        __builtin_amdgcn_sched_barrier(0);
        rdfrag(base_a, base_b, kk, rs);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int i = q / TN, j = q % TN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ms][i], fb[ms][j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // QKV: each lane keeps the position and the K / V cache base of slab row lane % 32
  // (one per 32-row MFMA slab), loaded before the main loop so that the epilogue's
  // rotary-table loads do not wait behind them
  int pre_pos[TM];
  uintptr_t pre_k[TM], pre_v[TM];
  if constexpr (EPI == EPI_QKV && !SPLIT) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int m = min(m0 + wm * WM + 32 * i + (lane & 31), M - 1);
      pre_pos[i] = epi.rows[m];
      if (epi.row_seq) {
        const int q = epi.row_seq[m];
        pre_k[i] = (uintptr_t)epi.k_seq.p[q];
        pre_v[i] = (uintptr_t)epi.v_seq.p[q];
      } else {
        pre_k[i] = (uintptr_t)epi.k_cache;
        pre_v[i] = (uintptr_t)epi.v_cache;
      }
    }
  }

  if constexpr (ASYM) {
    // loads in issue order: A0 B0 A1 B1 B2 .. B(NSB-1) (prologue), then A(t+2) B(t+NSB)
    // after the barrier of step t: when step t+1 is due, B(t+1) is older than A(t+1), and
    // the only loads issued after A(t+1) are those of B(t+NSB-1) (in the prologue also
    // B2 .. B(NSB-2), which the wait then covers too)
#pragma unroll
    for (int st = 0; st < NSB; ++st) {
      if (st < NSTG && st < nk) issue_a(st, st);
      if (st < nk) issue_b(st, st);
    }
    if (nk >= NSB) wait_vmcnt<(NSTG - 1) * LPA + (NSB - 1) * LPB>(); else wait_vmcnt<0>();
    lds_stage_barrier();
    rdfrag(a_stage(0), b_stage(0), 0, 0);
    for (int t = 0; t < nk; ++t) {
      const int sa = t % NSTG, sb = t % NSB;
#pragma unroll
      for (int kk = 0; kk + 1 < NS; ++kk) slice(kk & 1, a_stage(sa), b_stage(sb), kk + 1, (kk + 1) & 1);
      if (t + 1 < nk) {
        wait_lgkmcnt0();
        if (t + NSB - 1 < nk) wait_vmcnt<LPB>(); else wait_vmcnt<0>();
        lds_stage_barrier();
        if (t + NSTG < nk) issue_a(t + NSTG, sa);
        if (t + NSB < nk) issue_b(t + NSB, sb);
      }
      slice((NS - 1) & 1, a_stage((t + 1) % NSTG), b_stage((t + 1) % NSB), 0, 0);
    }
  } else {
#pragma unroll
    for (int st = 0; st < AHEAD; ++st)
      if (st < nk) issue(st, st);
    if (nk >= AHEAD) wait_vmcnt<(AHEAD - 1) * LPT>(); else wait_vmcnt<0>();
    lds_stage_barrier();
    rdfrag(a_stage(0), b_stage(0), 0, 0);

    for (int t = 0; t < nk; ++t) {
      const int stage = t % NSTG;
#pragma unroll
      for (int kk = 0; kk + 1 < NS; ++kk) slice(kk & 1, a_stage(stage), b_stage(stage), kk + 1, (kk + 1) & 1);
      if (t + 1 < nk) {
        if (!LATE) wait_lgkmcnt0();
        // this lane's loads of step t+1 have landed once at most the later steps'
        // (t+2 .. min(t+AHEAD-1, nk-1)) are outstanding
        if (t + AHEAD - 1 < nk) wait_vmcnt<(AHEAD - 2) * LPT>(); else wait_vmcnt<0>();
        lds_stage_barrier();
        if (t + AHEAD < nk) issue(t + AHEAD, (t + AHEAD) % NSTG);
      }
      // on the last step the read of stage (t+1) % NSTG stays inside LDS and is unused
      slice((NS - 1) & 1, a_stage((t + 1) % NSTG), b_stage((t + 1) % NSTG), 0, 0);
    }
  }

  // ---------------------------------------------------------------- epilogue
  // The accumulators go through LDS (each wavefront stages its own 32 x WN fp32
  // slab, one 32-row MFMA slab at a time) so that every output is written as a
  // row-contiguous 4-column vector: bf16 x4 stores for q / K / V / logits /
  // SwiGLU, fp32 x4 read-modify-write for the residual, x4 partials for split K.
  // A paired column's partner (packed column ^ 16) is read from the same slab.
  wait_lgkmcnt0();
  lds_stage_barrier();  // every wavefront is done with the staging buffers
  constexpr int ES = WN + 4;                 // slab row stride (floats)
  constexpr int C4 = WN / 4;                 // 4-column units per slab row
  constexpr int PL_BYTES = EPI == EPI_ENTROPY ? BM * WAVES_N * (int)sizeof(EntPart) : 0;
  static_assert(NW * 32 * ES * 4 + PL_BYTES <= LDS_BYTES, "epilogue staging exceeds the LDS tile buffers");
  static_assert(EPI != EPI_ENTROPY || !SPLIT, "the entropy epilogue needs whole K");
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * ES;
  const int d = epi.d_model, D = epi.head_dim, half = D / 2;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) slab[(8 * (v / 4) + 4 * hi + (v % 4)) * ES + 32 * j + lrow] = acc[i][j][v];
    const int mrow = m0 + wm * WM + 32 * i;  // first output row of this slab
    if (EPI == EPI_ENTROPY) {
      // partial softmax state of each slab row over this wavefront's WN columns, on
      // the logits rounded to bf16 (the values a stored logits tensor would hold):
      // lanes l and l + 32 take the lower / upper WN/2 columns of row l % 32
      constexpr int CW = WN / 2;
      const int r = lane & 31, cb = (lane >> 5) * CW;
      const int colb = n0 + wn * WN + cb;
      float mx = -INFINITY, z = 0.f, s2 = 0.f;
      int ix = 0x7fffffff, has_nan = 0;
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        const float x = colb + c < N ? (float)(bf16)slab[r * ES + cb + c] : -INFINITY;
        has_nan |= x != x;  // carried as a flag: a share of NaN / -inf alone keeps z = 0
        if (x > mx) {  // NaN never wins; the first index of the max stays
          mx = x;
          ix = colb + c;
        }
      }
      if (mx != -INFINITY) {
        const float mb = mx * kLog2e;
#pragma unroll
        for (int c = 0; c < CW; ++c) {
          const float x = colb + c < N ? (float)(bf16)slab[r * ES + cb + c] : -INFINITY;
          const float t = fmaf(x, kLog2e, -mb);
          const float e = __builtin_amdgcn_exp2f(t);  // a NaN logit makes z NaN
          z += e;
          s2 = fmaf(fmaxf(t, -1000.f), e, s2);     // -inf logit: -1000 * 0 = 0
        }
      }
      EntPart a{mx, z, s2 * kLn2, ix, has_nan, {0, 0, 0}};
      EntPart b{__shfl_xor(a.m, 32), __shfl_xor(a.z, 32), __shfl_xor(a.s, 32), __shfl_xor(a.idx, 32),
                __shfl_xor(a.nan, 32), {0, 0, 0}};
      if (lane < 32) {
        part_merge(a, b);
        reinterpret_cast<EntPart*>(smem + NW * 32 * ES * 4)[(wm * WM + 32 * i + r) * WAVES_N + wn] = a;
      }
      continue;
    }
    if (EPI == EPI_SWIGLU && !SPLIT) {
      // units: (row, 4 gate columns); the up partner is 16 columns on. The unit loops
      // have a constant trip count (32 * WN / 8 and 32 * WN / 4 units, multiples of
      // 64) so that they unroll and their global loads issue together.
      constexpr int UG = C4 / 2;
      static_assert((32 * UG) % 64 == 0, "unit count");
#pragma unroll
      for (int it = 0; it < 32 * UG / 64; ++it) {
        const int u = lane + 64 * it;
        const int r = u / UG, k = u % UG;
        const int c = (k / 4) * 32 + (k % 4) * 4;
        const int m = mrow + r, pc = n0 + wn * WN + c;
        if (m >= M || pc >= N) continue;
        const f32x4 g = *reinterpret_cast<const f32x4*>(slab + r * ES + c);
        const f32x4 up = *reinterpret_cast<const f32x4*>(slab + r * ES + c + 16);
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)(silu(g[e]) * up[e]);
        const int f = (pc >> 5) * 16 + (pc & 15);
        *reinterpret_cast<bf16x4*>((bf16*)epi.out + (int64_t)m * epi.ldo + f) = o;
      }
      continue;
    }
    static_assert((32 * C4) % 64 == 0, "unit count");
    if constexpr (EPI == EPI_QKV && !SPLIT) {
      // units: (row, 4 first-half packed columns c) with their rotary partners at c + 16;
      // a lane computes both halves of a pair, so one cos / sin load serves both. All
      // table loads of the slab are issued before its first store (on this target stores
      // and loads share one counter, so a store would otherwise make the next unit's
      // loads wait for it).
      constexpr int UP = C4 / 2;  // pairs per slab row
      constexpr int NPI = 32 * UP / 64;
      static_assert((32 * UP) % 64 == 0, "pair count");
      f32x4 tcs[NPI], tsn[NPI];
#pragma unroll
      for (int it = 0; it < NPI; ++it) {
        const int u = lane + 64 * it;
        const int r = u / UP, k = u % UP;
        const int pc = n0 + wn * WN + (k / 4) * 32 + (k % 4) * 4;
        const int p = pc & (D - 1);  // D is a power of two
        const int rc = (p >> 5) * 16 + (p & 15);
        const int pos = __shfl(pre_pos[i], r);
        const bool pos_ok = pos >= 0 && pos < epi.seq_len;
        const int64_t tp = (int64_t)(pos_ok ? pos : 0) * half + rc;
        tcs[it] = *reinterpret_cast<const f32x4*>(epi.rope_cos + tp);
        tsn[it] = *reinterpret_cast<const f32x4*>(epi.rope_sin + tp);
      }
      const bool per_row_kv = epi.row_seq != nullptr;
#pragma unroll
      for (int it = 0; it < NPI; ++it) {
        const int u = lane + 64 * it;
        const int r = u / UP, k = u % UP;
        const int c = (k / 4) * 32 + (k % 4) * 4;
        const int m = mrow + r, pc = n0 + wn * WN + c;
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(slab + r * ES + c);
        const f32x4 x2 = *reinterpret_cast<const f32x4*>(slab + r * ES + c + 16);
        const int p = pc & (D - 1), hb = pc - p;
        const int rc = (p >> 5) * 16 + (p & 15);
        const int sec = (hb >= d) + (hb >= 2 * d);  // 0: q, 1: k, 2: v
        const int hcol = hb - sec * d + rc;         // first-half column; its partner is + D/2
        const int pos = __shfl(pre_pos[i], r);
        const bool pos_ok = pos >= 0 && pos < epi.seq_len;
        const bool rot = sec < 2 && pos_ok;
        // first half: x1 cos - x2 sin; second half: x1 sin + x2 cos
        bf16x4 o1, o2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = fmaf(x1[e], tcs[it][e], -x2[e] * tsn[it][e]);
          const float b = fmaf(x1[e], tsn[it][e], x2[e] * tcs[it][e]);
          o1[e] = (bf16)(rot ? a : x1[e]);
          o2[e] = (bf16)(rot ? b : x2[e]);
        }
        uintptr_t kb = (uintptr_t)epi.k_cache, vb = (uintptr_t)epi.v_cache;
        if (per_row_kv) {
          kb = ((uintptr_t)(uint32_t)__shfl((int)(uint32_t)pre_k[i], r)) |
               ((uintptr_t)(uint32_t)__shfl((int)(uint32_t)(pre_k[i] >> 32), r) << 32);
          vb = ((uintptr_t)(uint32_t)__shfl((int)(uint32_t)pre_v[i], r)) |
               ((uintptr_t)(uint32_t)__shfl((int)(uint32_t)(pre_v[i] >> 32), r) << 32);
        }
        if (m >= M || pc >= N) continue;
        uintptr_t dst;
        if (sec == 0) dst = (uintptr_t)((bf16*)epi.out + (int64_t)m * d + hcol);
        else if (pos_ok) dst = (uintptr_t)((bf16*)(sec == 2 ? vb : kb) + (int64_t)pos * d + hcol);
        else continue;
        // the destination is device memory: global (not flat) stores, which neither wait
        // on nor alias the LDS slab reads
        gbf16x4* g = (gbf16x4*)dst;
        g[0] = o1;
        *(gbf16x4*)(dst + half * sizeof(bf16)) = o2;
      }
      continue;
    }
#pragma unroll
    for (int it = 0; it < 32 * C4 / 64; ++it) {
      const int u = lane + 64 * it;
      const int r = u / C4, c = (u % C4) * 4;
      const int m = mrow + r, pc = n0 + wn * WN + c;
      const f32x4 x = *reinterpret_cast<const f32x4*>(slab + r * ES + c);
      if (EPI == EPI_RESID && !SPLIT) {
        // the residual load is unconditional (clamped) so that the loads of the unrolled
        // loop issue together; the store is predicated
        f32x4* hp = reinterpret_cast<f32x4*>(epi.resid + (int64_t)min(m, M - 1) * epi.ldo + min(pc, N - 4));
        const f32x4 h0 = *hp;
        if (m < M && pc < N) *hp = h0 + x;
        continue;
      }
      if (m >= M || pc >= N) continue;
      if (SPLIT) {
        *reinterpret_cast<f32x4*>(part + ((int64_t)kz * M + m) * N + pc) = x;
      } else if (EPI == EPI_STORE) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16)x[e];
        *reinterpret_cast<bf16x4*>((bf16*)epi.out + (int64_t)m * epi.ldo + pc) = o;
      }
    }
  }
  if (EPI == EPI_ENTROPY) {
    // one state per (row, column tile): the wavefronts' states merged in column order
    lds_stage_barrier();
    const EntPart* pl = reinterpret_cast<const EntPart*>(smem + NW * 32 * ES * 4);
    for (int r = tid; r < BM; r += NT) {
      if (m0 + r >= M) continue;
      EntPart a = pl[r * WAVES_N];
#pragma unroll
      for (int w = 1; w < WAVES_N; ++w) part_merge(a, pl[r * WAVES_N + w]);
      epi.parts[(int64_t)(m0 + r) * epi.ntiles + nt] = a;
    }
  }
}

// -------------------------------------------------------------------- split-K reduction
// Partials part[S][M][N] over the packed columns of the bf16 kernel. One thread per
// output unit sums the S partials in order (deterministic), then the epilogue:
// QKV and SwiGLU units are the (pc, pc + 16) pairs of each 32-column group. With the
// split count SP known at compile time every partial load is issued before the first
// addition (one memory round trip, not S); SP < 0 takes S at run time.
template <int SP>
__device__ __forceinline__ void sum_parts(const float* __restrict__ part, int S, int64_t stride, int64_t o1,
                                          int64_t o2, bool two, float& x1, float& x2) {
  if constexpr (SP > 0) {
    float p1[SP], p2[SP];
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      p1[s] = part[s * stride + o1];
      p2[s] = two ? part[s * stride + o2] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      x1 += p1[s];
      x2 += p2[s];
    }
  } else {
    for (int s = 0; s < S; ++s) {
      x1 += part[s * stride + o1];
      if (two) x2 += part[s * stride + o2];
    }
  }
}

template <int SP>
__global__ void __launch_bounds__(kThreads)
splitk_epilogue_kernel(const float* __restrict__ part, int S, int M, int N, int kind, EpiArgs epi) {
  const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  const int64_t stride = (int64_t)M * N;
  if (kind == EPI_QKV || kind == EPI_SWIGLU) {
    const int64_t upr = N / 2;
    if (t >= (int64_t)M * upr) return;
    const int m = (int)(t / upr), u = (int)(t % upr);
    const int pc = (u >> 4) * 32 + (u & 15);
    float x1 = 0.f, x2 = 0.f;
    sum_parts<SP>(part, S, stride, (int64_t)m * N + pc, (int64_t)m * N + pc + 16, true, x1, x2);
    if (kind == EPI_SWIGLU) {
      epi_swiglu<bf16>(epi, m, u, x1, x2);
    } else {
      const int hb = pc - pc % epi.head_dim, pp = pc - hb;
      epi_qkv_pair<bf16>(epi, m, hb + (pp >> 5) * 16 + (pp & 15), x1, x2);
    }
  } else {
    if (t >= (int64_t)M * N) return;
    const int m = (int)(t / N), col = (int)(t % N);
    float x = 0.f, unused = 0.f;
    sum_parts<SP>(part, S, stride, (int64_t)m * N + col, 0, false, x, unused);
    epi_single<bf16>(epi, m, col, x);
  }
}

// -------------------------------------------------------------------- fp32 SIMT GEMM
// fp32 path for what the matrix-unit kernel below does not take (K not a multiple of 4,
// operands not 16-byte aligned, or rotary halves narrower than 32 columns): one thread per
// output unit (an element, or the pair the rotary / SwiGLU epilogue needs), dot products
// over K.
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

// fp32 models on the matrix unit (v_mfma_f32_32x32x2_f32): one wavefront per 32 output
// rows and two 32-column blocks that its epilogue pairs: the rotary partners half a head
// away (q/k/v), the up rows of the same columns (SwiGLU, from B2), or the next 32
// columns. Lane l loads four consecutive K elements at offset 4 (l / 32) of each 8-wide K
// step from row l % 32 of A and of each B block, so MFMA j of the step takes K positions
// k + j (lanes 0-31) and k + 4 + j (lanes 32-63). Every output sums its K positions in the
// same order whatever M and whichever rows share its launch.
constexpr int kF32Waves = 4;
__global__ void __launch_bounds__(kF32Waves * 64)
gemm_f32_mfma_kernel(const float* __restrict__ A, const float* __restrict__ B, const float* __restrict__ B2,
                     int M, int N, int K, int units, EpiArgs epi) {
  const int lane = threadIdx.x % 64;
  const int64_t w = (int64_t)blockIdx.x * kF32Waves + threadIdx.x / 64;
  const int mb = (M + 31) / 32;
  if (w >= (int64_t)mb * units) return;  // a whole wavefront
  const int mt = (int)(w % mb), u = (int)(w / mb);
  const int kind = epi.kind;
  int c1, c2;
  const float* Bs = B;
  if (kind == EPI_QKV) {
    const int half = epi.head_dim / 2, per_head = half / 32;
    c1 = (u / per_head) * epi.head_dim + (u % per_head) * 32;
    c2 = c1 + half;
  } else if (kind == EPI_SWIGLU) {
    c1 = c2 = u * 32;
    Bs = B2;
  } else {
    c1 = u * 64;
    c2 = c1 + 32;
  }
  const int r = lane % 32, kq = 4 * (lane / 32), m0 = mt * 32;
  const float* a = A + (int64_t)min(m0 + r, M - 1) * K + kq;
  const float* b1 = B + (int64_t)min(c1 + r, N - 1) * K + kq;
  const float* b2 = Bs + (int64_t)min(c2 + r, N - 1) * K + kq;
  f32x16 acc1, acc2;
#pragma unroll
  for (int v = 0; v < 16; ++v) acc1[v] = acc2[v] = 0.f;
  auto step = [&](const float4& x, const float4& y1, const float4& y2) __attribute__((always_inline)) {
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y1.x, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.x, y2.x, acc2, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y1.y, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.y, y2.y, acc2, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y1.z, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.z, y2.z, acc2, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y1.w, acc1, 0, 0, 0);
    acc2 = __builtin_amdgcn_mfma_f32_32x32x2f32(x.w, y2.w, acc2, 0, 0, 0);
  };
  int k = 0;
  for (; k + 8 <= K; k += 8)
    step(*reinterpret_cast<const float4*>(a + k), *reinterpret_cast<const float4*>(b1 + k),
         *reinterpret_cast<const float4*>(b2 + k));
  if (k < K) {  // K % 8 == 4: the upper half-wavefront's elements lie past K and count as zero
    const bool in = k + kq < K;
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    step(in ? *reinterpret_cast<const float4*>(a + k) : z, in ? *reinterpret_cast<const float4*>(b1 + k) : z,
         in ? *reinterpret_cast<const float4*>(b2 + k) : z);
  }
  // accumulator element v of lane l: row 8 (v / 4) + 4 (l / 32) + v % 4, column l % 32
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int m = m0 + 8 * (v / 4) + 4 * (lane / 32) + (v % 4);
    if (m >= M) continue;
    if (kind == EPI_QKV) {
      epi_qkv_pair<float>(epi, m, c1 + r, acc1[v], acc2[v]);
    } else if (kind == EPI_SWIGLU) {
      if (c1 + r < N) epi_swiglu<float>(epi, m, c1 + r, acc1[v], acc2[v]);
    } else {
      if (c1 + r < N) epi_single<float>(epi, m, c1 + r, acc1[v]);
      if (c2 + r < N) epi_single<float>(epi, m, c2 + r, acc2[v]);
    }
  }
}

// -------------------------------------------------------------------- weight packing
// dst row pr <- src row of the packed layouts described above (one workgroup per row)
__global__ void __launch_bounds__(kThreads)
pack_rows_kernel(const unsigned char* __restrict__ a, const unsigned char* __restrict__ b,
                 unsigned char* __restrict__ dst, int rows, int row_bytes, int mode, int head_dim) {
  const int pr = blockIdx.x;
  if (pr >= rows) return;
  const unsigned char* src;
  const int g = (pr & 31) >> 4, l = pr & 15, grp = pr >> 5;
  if (mode == 0) {  // rotary: within each head
    const int hb = pr - pr % head_dim, p = pr - hb;
    const int c = (p >> 5) * 16 + l + (g ? head_dim / 2 : 0);
    src = a + (int64_t)(hb + c) * row_bytes;
  } else {          // gate / up interleave
    src = (g ? b : a) + (int64_t)(grp * 16 + l) * row_bytes;
  }
  unsigned char* out = dst + (int64_t)pr * row_bytes;
  if (row_bytes % 16 == 0) {
    for (int i = threadIdx.x; i < row_bytes / 16; i += kThreads)
      reinterpret_cast<v4u*>(out)[i] = reinterpret_cast<const v4u*>(src)[i];
  } else {
    for (int i = threadIdx.x; i < row_bytes; i += kThreads) out[i] = src[i];
  }
}

// -------------------------------------------------------------------- host-side planning
constexpr int kCUs = 256;

enum TileCfg {
  T256x192, T256x128, T128x128, T64x128, T256x96, T128x96, T256x64, T128x64, T256x32, T64x96, T64x64, kNumTileCfg
};
struct TileInfo {
  int BM, BN;
  double eff;  // sustained MFMA rate relative to 4 TFLOP/s per CU, measured on MI355X
};
constexpr TileInfo kTile[kNumTileCfg] = {
    {256, 192, 1.10}, {256, 128, 1.10}, {128, 128, 0.80}, {64, 128, 0.45},
    {256, 96, 0.90}, {128, 96, 0.786}, {256, 64, 0.80}, {128, 64, 0.55}, {256, 32, 0.50},
    {64, 96, 0.377}, {64, 64, 0.311}};
// Sustained global-to-LDS rate of one CU (bytes per microsecond) with the weights streamed
// from HBM: a tile's staging time is (BM + BN) x K x 2 bytes at this rate.
constexpr double kCuLoadBytesPerUs = 60e3;

struct Plan {
  TileCfg cfg;
  int S, k_chunk, MT, NT;
};

// Tile choice by a cost model fitted to MI355X measurements of every candidate on the
// projection shapes (N x K = 12288 x 4096, 24576 x 4096, 4096 x 4096, 4096 x 12288; rows
// 17 .. 4096, weights streamed from HBM): time = waves x per-tile time, waves =
// ceil(tiles * S / 256), per-tile time = the larger of the MFMA time
// 2 BM BN (K / S) / (eff x 4 TFLOP/s) and the staging time (Mr + BN) (K / S) 2 bytes
// at kCuLoadBytesPerUs (Mr = the tile's rows that exist, min(BM, M rounded up to 32):
// rows past M are not loaded), plus, for split K, the partials' round trip (S M N x 8 bytes at
// 3 TB/s) and 6 us for the reduction launch (measured with the K rotation of skinny
// tiles). Larger tiles carry more MFMA work per staged byte; smaller ones and split K
// fill the 256 CUs at skinny M (skip steps, the LM head over the candidates). The
// all-rows tiles (four wavefronts stacked along M over one weight slice of 96, 64 or 32
// columns) are priced only at M <= 256, and the 64-row tiles with 96 or 64 columns, which
// cut the projections into about 256 workgroups, also at M <= 64; their efficiencies were
// fitted, with the four older tiles' figures held fixed, to sweeps of every tile and split
// at M = 17 .. 256 on the four projection shapes. Over those sweeps the choices cost 1.2 %
// more than the fastest measured candidate in total, at most 11 % on one shape (17 rows of
// the 4096 x 4096 product). Every tile shape and split S in {1, 2, 4, 8} (K chunks of at
// least 8 steps) is priced and the cheapest taken.
Plan plan_bf16(int M, int N, int K, int kind) {
  Plan best{};
  double best_us = 1e300;
  const int nk = K / BK;
  // the fused entropy epilogue needs whole K and stages one state per row and
  // wavefront column next to the slabs: 128x128 and 64x128 tiles only. The stored-logits
  // LM head (EPI_STORE) takes the same plan and K order, so the logits it writes are
  // exactly the values the fused epilogue reduces.
  const bool ent = kind == EPI_ENTROPY || kind == EPI_STORE;
  for (int c = 0; c < kNumTileCfg; ++c) {
    const TileInfo& t = kTile[c];
    if (ent && c != T128x128 && c != T64x128) continue;  // the only tiles launch_cfg has for them
    if (c >= T256x96 && M > 256) continue;  // all-rows tiles: measured at skinny M only
    if (M <= 64 && c != T64x128 && c != T64x96 && c != T64x64) continue;
    if (M <= 128 && (c == T256x192 || c == T256x128)) continue;
    const int MT = (M + t.BM - 1) / t.BM, NT = (N + t.BN - 1) / t.BN;
    const int64_t tiles = (int64_t)MT * NT;
    for (int S = 1; S <= (ent ? 1 : 8); S *= 2) {
      if (S > 1 && (nk % S != 0 || nk / S < 8)) break;
      const int64_t waves = (tiles * S + kCUs - 1) / kCUs;
      const double kc = (double)K / S;
      const double mfma_us = 2.0 * t.BM * t.BN * kc / (t.eff * 4e6);
      const int rows = std::min(t.BM, (M + 31) / 32 * 32);
      const double load_us = (double)(rows + t.BN) * kc * 2.0 / kCuLoadBytesPerUs;
      double us = (double)waves * (mfma_us > load_us ? mfma_us : load_us);
      if (S > 1) us += (double)S * M * N * 8.0 / 3e6 + 6.0;
      if (us < best_us) {
        best_us = us;
        best.cfg = (TileCfg)c;
        best.MT = MT;
        best.NT = NT;
        best.S = S;
        best.k_chunk = K / S;
      }
    }
  }
  return best;
}

template <int BM, int BN, int WM, int WN, int NSTG, bool LATE, int EPI, int BKS = 64, int NSB = 0>
ec_status launch_bf16(const Plan& p, const bf16* A, const bf16* B, int M, int N, int K,
                      const EpiArgs& epi, float* part, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  constexpr size_t lds = NSB > 0 ? ((size_t)NSTG * BM + (size_t)NSB * BN) * BKS * 2
                                 : (size_t)NSTG * (BM + BN) * BKS * 2;
  static_assert(lds <= 160 * 1024, "LDS budget");
  const int grid = p.MT * p.NT * p.S;
  // one limit record per kernel: the split and whole-K kernels share a function type,
  // so a static inside the generic lambda would be shared by both
  static LdsLimit whole, split;
  auto run = [&](auto kern, LdsLimit& limit) -> ec_status {
    const ec_status st = limit.ensure((const void*)kern, (int)lds);
    if (st != EC_OK) return st;
    kern<<<grid, NT, lds, s>>>(A, B, M, N, K, p.k_chunk, p.S, epi, part);
    EC_CHECK_LAUNCH("gemm_bf16_kernel");
    return EC_OK;
  };
  if constexpr (EPI != EPI_ENTROPY) {
    if (p.S > 1) return run(gemm_bf16_kernel<BM, BN, WM, WN, NSTG, LATE, EPI, true, BKS, NSB>, split);
  }
  return run(gemm_bf16_kernel<BM, BN, WM, WN, NSTG, LATE, EPI, false, BKS, NSB>, whole);
}

template <int EPI>
ec_status launch_cfg(const Plan& p, const bf16* A, const bf16* B, int M, int N, int K,
                     const EpiArgs& epi, float* part, hipStream_t s) {
  if constexpr (EPI == EPI_ENTROPY || EPI == EPI_STORE) {
    if (p.cfg == T128x128) return launch_bf16<128, 128, 32, 64, 4, true, EPI>(p, A, B, M, N, K, epi, part, s);
    return launch_bf16<64, 128, 32, 32, 6, true, EPI>(p, A, B, M, N, K, epi, part, s);
  } else {
    switch (p.cfg) {
      case T256x192: return launch_bf16<256, 192, 64, 96, 2, false, EPI, 64, 4>(p, A, B, M, N, K, epi, part, s);
      case T256x128: return launch_bf16<256, 128, 64, 64, 3, false, EPI>(p, A, B, M, N, K, epi, part, s);
      case T128x128: return launch_bf16<128, 128, 32, 64, 4, true, EPI>(p, A, B, M, N, K, epi, part, s);
      // all-rows tiles of skinny products: four wavefronts stacked along M share one weight slice
      case T256x96: return launch_bf16<256, 96, 64, 96, 3, false, EPI>(p, A, B, M, N, K, epi, part, s);
      case T128x96: return launch_bf16<128, 96, 32, 96, 4, true, EPI>(p, A, B, M, N, K, epi, part, s);
      case T256x64: return launch_bf16<256, 64, 64, 64, 3, false, EPI>(p, A, B, M, N, K, epi, part, s);
      case T128x64: return launch_bf16<128, 64, 32, 64, 4, true, EPI>(p, A, B, M, N, K, epi, part, s);
      case T256x32: return launch_bf16<256, 32, 64, 32, 3, false, EPI>(p, A, B, M, N, K, epi, part, s);
      // skinny tiles that cut the projections into 256 workgroups at small M
      case T64x96: return launch_bf16<64, 96, 32, 96, 6, true, EPI>(p, A, B, M, N, K, epi, part, s);
      case T64x64: return launch_bf16<64, 64, 32, 32, 6, true, EPI>(p, A, B, M, N, K, epi, part, s);
      default: return launch_bf16<64, 128, 32, 32, 6, true, EPI>(p, A, B, M, N, K, epi, part, s);
    }
  }
}

// B rows of the bf16 kernel: the packed gate/up matrix has 2F rows for F outputs
int b_rows(int N, int kind) { return kind == EPI_SWIGLU ? 2 * N : N; }

}  // namespace

int gemm_col_tiles(int M, int N, int K, int kind) {
  if (M <= 0) return 0;
  return plan_bf16(M, b_rows(N, kind), K, kind).NT;
}

size_t gemm_splitk_ws_bytes(int M, int N, int K, int kind, bool is_bf16) {
  if (!is_bf16 || M <= 0) return 0;
  const int NB = b_rows(N, kind);
  // the kernel addresses A and B through buffer resources with 32-bit byte offsets
  EC_REQUIRE((int64_t)M * K * 2 <= 0x7fffffff && (int64_t)NB * K * 2 <= 0x7fffffff, EC_ERR_UNSUPPORTED,
             "gemm: operands of %d x %d and %d x %d bf16 exceed the 2 GiB buffer range", M, K, NB, K);
  Plan p = plan_bf16(M, NB, K, kind);
  if (p.S <= 1) return 0;
  return (size_t)p.S * M * NB * sizeof(float);
}

ec_status gemm(ec_dtype dt, const void* A, const void* B, const void* B2, int M, int N, int K,
               const EpiArgs& epi, float* splitk_ws, size_t splitk_ws_bytes, hipStream_t s,
               bool* normed) {
  if (normed) *normed = false;
  if (M == 0) return EC_OK;
  const int kind = epi.kind;
  if (dt == EC_F32) {
    EC_REQUIRE(kind != EPI_ENTROPY, EC_ERR_UNSUPPORTED, "gemm: the fused entropy epilogue is bf16 only");
    const bool a16 = (((uintptr_t)A | (uintptr_t)B | (uintptr_t)(B2 ? B2 : B)) & 15) == 0;
    if (K % 4 == 0 && a16 && (kind != EPI_QKV || epi.head_dim % 64 == 0)) {
      // matrix-unit path: 16-byte row loads, rotary halves of whole 32-column blocks
      const int units = kind == EPI_QKV ? N / 64 : kind == EPI_SWIGLU ? (N + 31) / 32 : (N + 63) / 64;
      const int64_t waves = (int64_t)((M + 31) / 32) * units;
      const int blocks = (int)((waves + kF32Waves - 1) / kF32Waves);
      gemm_f32_mfma_kernel<<<blocks, kF32Waves * 64, 0, s>>>((const float*)A, (const float*)B, (const float*)B2, M,
                                                             N, K, units, epi);
      EC_CHECK_LAUNCH("gemm_f32_mfma_kernel");
      return EC_OK;
    }
    const int64_t units = (kind == EPI_QKV) ? (int64_t)M * (N / 2) : (int64_t)M * N;
    const int blocks = (int)((units + kThreads - 1) / kThreads);
    gemm_f32_kernel<<<blocks, kThreads, 0, s>>>((const float*)A, (const float*)B,
                                                (const float*)B2, M, N, K, epi);
    EC_CHECK_LAUNCH("gemm_f32_kernel");
    return EC_OK;
  }
  EC_REQUIRE(K % BK == 0, EC_ERR_UNSUPPORTED, "gemm: K=%d not a multiple of %d", K, BK);
  EC_REQUIRE(N % 4 == 0, EC_ERR_UNSUPPORTED, "gemm: N=%d not a multiple of 4 (4-column output vectors)", N);
  if (kind == EPI_QKV)
    EC_REQUIRE(epi.head_dim >= 32 && (epi.head_dim & (epi.head_dim - 1)) == 0 && N % epi.head_dim == 0,
               EC_ERR_UNSUPPORTED, "gemm: packed QKV needs a power-of-two head_dim >= 32");
  if (kind == EPI_SWIGLU)
    EC_REQUIRE(N % 16 == 0, EC_ERR_UNSUPPORTED, "gemm: packed SwiGLU needs F %% 16 == 0");
  const int NB = b_rows(N, kind);
  // the kernel addresses A and B through buffer resources with 32-bit byte offsets
  EC_REQUIRE((int64_t)M * K * 2 <= 0x7fffffff && (int64_t)NB * K * 2 <= 0x7fffffff, EC_ERR_UNSUPPORTED,
             "gemm: operands of %d x %d and %d x %d bf16 exceed the 2 GiB buffer range", M, K, NB, K);
  Plan p = plan_bf16(M, NB, K, kind);
  EpiArgs e = epi;
  if (kind == EPI_ENTROPY) {
    EC_REQUIRE(epi.parts != nullptr, EC_ERR_ARG, "gemm: entropy epilogue without a parts buffer");
    e.ntiles = p.NT;
  }
  float* part = nullptr;
  if (p.S > 1) {
    const size_t need = gemm_splitk_ws_bytes(M, N, K, kind, true);
    EC_REQUIRE(splitk_ws && splitk_ws_bytes >= need, EC_ERR_WORKSPACE,
               "gemm: split-K workspace %zu < %zu bytes", splitk_ws_bytes, need);
    part = splitk_ws;
  }
  const bf16* a = (const bf16*)A;
  const bf16* b = (const bf16*)B;
  ec_status st;
  switch (kind) {
    case EPI_QKV: st = launch_cfg<EPI_QKV>(p, a, b, M, NB, K, e, part, s); break;
    case EPI_SWIGLU: st = launch_cfg<EPI_SWIGLU>(p, a, b, M, NB, K, e, part, s); break;
    case EPI_RESID: st = launch_cfg<EPI_RESID>(p, a, b, M, NB, K, e, part, s); break;
    case EPI_ENTROPY: st = launch_cfg<EPI_ENTROPY>(p, a, b, M, NB, K, e, part, s); break;
    default: st = launch_cfg<EPI_STORE>(p, a, b, M, NB, K, e, part, s); break;
  }
  if (st != EC_OK) return st;
  if (p.S > 1) {
    if (kind == EPI_RESID && epi.norm_out && normed && epi.ldo == NB) {
      // residual update fused with the next RMSNorm: one pass over the rows
      const ec_status sn = resid_norm(dt, part, p.S, M, NB, epi.resid, epi.norm_gain, epi.norm_eps, epi.norm_out, s);
      if (sn != EC_OK) return sn;
      *normed = true;
      return EC_OK;
    }
    const int64_t units = (kind == EPI_QKV || kind == EPI_SWIGLU) ? (int64_t)M * (NB / 2) : (int64_t)M * NB;
    const int blocks = (int)((units + kThreads - 1) / kThreads);
    switch (p.S) {
      case 2: splitk_epilogue_kernel<2><<<blocks, kThreads, 0, s>>>(part, p.S, M, NB, kind, epi); break;
      case 4: splitk_epilogue_kernel<4><<<blocks, kThreads, 0, s>>>(part, p.S, M, NB, kind, epi); break;
      case 8: splitk_epilogue_kernel<8><<<blocks, kThreads, 0, s>>>(part, p.S, M, NB, kind, epi); break;
      default: splitk_epilogue_kernel<-1><<<blocks, kThreads, 0, s>>>(part, p.S, M, NB, kind, epi); break;
    }
    EC_CHECK_LAUNCH("splitk_epilogue_kernel");
  }
  return EC_OK;
}

ec_status pack_weights(int elem_bytes, int d, int head_dim, int F, const void* wqkv,
                       const void* w_gate, const void* w_up, void* wqkv_packed,
                       void* gateup_packed, hipStream_t s) {
  const int row_bytes = d * elem_bytes;
  if (wqkv_packed) {
    pack_rows_kernel<<<3 * d, kThreads, 0, s>>>((const unsigned char*)wqkv, nullptr,
                                                 (unsigned char*)wqkv_packed, 3 * d, row_bytes, 0, head_dim);
    EC_CHECK_LAUNCH("pack_rows_kernel");
  }
  if (gateup_packed) {
    pack_rows_kernel<<<2 * F, kThreads, 0, s>>>((const unsigned char*)w_gate, (const unsigned char*)w_up,
                                                 (unsigned char*)gateup_packed, 2 * F, row_bytes, 1, head_dim);
    EC_CHECK_LAUNCH("pack_rows_kernel");
  }
  return EC_OK;
}

}  // namespace ec
