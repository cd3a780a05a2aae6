// Bidirectional attention of the recomputed rows over every cached row.
//
// In a diffusion LM every position attends to every other (EntropyCache
// explainer, Italian summary section 1), so the r recomputed query rows of a
// skip step attend over all L rows of the layer's K/V cache: the fresh rows
// just written and the stale cached rows of every other position. There is
// no mask.
//
// bf16 kernel (head_dim 128), flash-style with an online softmax, computed
// transposed so that no register shuffles are needed between the two
// products: a wavefront owns 32 query rows and, per 32-row K/V sub-tile,
//   S^T = K Q^T        8 x v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q rows)
//   O^T += V^T P^T     8 x v_mfma_f32_32x32x16_bf16 (A = V^T, B = P^T)
// In the 32x32 accumulator layout a lane holds one query column and 16 key
// rows; those 16 values, converted to bf16 in order, are exactly the lane's
// B operand of the second product for the two 16-key halves, provided V^T's
// A operand supplies keys in the same slot order. V stays in its natural
// [key][dim] layout in LDS and the V^T operand comes from gfx950's
// transposing LDS read (ds_read_tr16_b64: within 16 lanes, lane j receives
// element j of each of four source lanes' 8-byte rows), two per fragment.
// Softmax statistics are per lane (one query), completed with one
// cross-half exchange; the reference max is only moved (and O, l rescaled)
// when a row max exceeds it by 2^8, so most tiles skip the rescale. The
// reference is an integer in base-2 units, so the probabilities that enter the
// P.V product in bf16 are the weights 2^(t - M), t = score * log2(e) / sqrt(D),
// rounded to bf16 for an integer M: the same rounded values for any tiling (the
// row sum l takes the unrounded weights). All global
// loads go straight into LDS (buffer_load_dwordx4 ... lds, no staging registers):
// the workgroup's Q tile once, issued with the first K/V tiles and then read into
// registers for the whole loop, and the K and V tiles through a ring of LDS
// stages, so that the loads of the next tiles are in flight during the current
// tile's MFMAs (a split of no more tiles than stages issues all of its loads at
// once). The tiles are shared by the 8 wavefronts of a workgroup (two per SIMD:
// one's softmax and LDS reads overlap the other's MFMAs), in one of two shapes:
//   wide:   4 groups of 32 queries (128 queries), 64-key tiles, 4 stages; the two
//           wavefronts of a group take the lower and the upper 32 keys of a tile;
//   narrow: 2 groups of 32 queries (64 queries), 128-key tiles, 2 stages; the four
//           wavefronts of a group take one 32-key quarter of a tile each.
// The wavefronts of a query group combine their (m, l, o) through LDS at the end.
// A skip step's few hundred rows fill the 256 CUs with narrow workgroups and
// whole key ranges; when heads x query tiles still under-fill them, the key range
// is split over workgroups and a merge kernel combines (m, l, o) exactly.
#include "ec_internal.h"

#include <math.h>

namespace ec {

namespace {

constexpr int kThreads = 256;      // merge and fp32 kernels
constexpr int D = 128;       // head_dim of the MFMA kernel
constexpr int KS = D;        // LDS row stride (bf16): unpadded 256-byte rows, swizzled (below)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaxFloor = -1e30f;  // below every reachable score in log2 units
constexpr float kRescale = 8.f;  // lazy rescale: keep the reference max until a row max exceeds it by 2^8

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16 lds_bf16;

// Workgroup shape of the MFMA kernel: QG groups of 32 queries x KG wavefronts per group, each
// wavefront taking 32 keys of every K/V tile (BKV = 32 KG keys), over a ring of NSTG tiles.
//   wide   (4 x 2, 4 stages): 128 queries, 64-key tiles; refresh-sized and long query sets
//   narrow (2 x 4, 2 stages): 64 queries, 128-key tiles; the few hundred rows of a skip step,
//          where 128-query tiles leave most CUs idle unless the keys are split (and merged)
template <int QG_, int KG_, int NSTG_>
struct AttnShape {
  static constexpr int QG = QG_, KG = KG_, NSTG = NSTG_;
  static constexpr int NW = QG * KG, NT = NW * 64;
  static constexpr int BQ = 32 * QG;                        // queries per workgroup
  static constexpr int BKV = 32 * KG;                       // keys per LDS stage
  static constexpr int kTileBytes = BKV * KS * 2;           // K (or V) of one tile
  static constexpr int kVOff = NSTG * kTileBytes;           // V stages after the K stages
  static constexpr int kQOff = 2 * NSTG * kTileBytes;       // Q tile (BQ rows of 256 bytes) after the ring
  static constexpr int kHandBytes = (KG - 1) * QG * 64 * (D / 2 + 2) * 4;  // (m, l, o) hand-over, over the ring
  static constexpr int kLds = kQOff + BQ * D * 2;
  static constexpr int SL = BKV / 4 / NW;                   // 1 KB slices of K (and of V) per wavefront per tile
  static constexpr int kLoadsPerTile = 2 * SL;              // per wavefront
  static constexpr int kQLoads = BQ * D * 2 / 1024 / NW;    // per wavefront
  static_assert(kHandBytes <= kQOff, "hand-over fits in the ring");
  static_assert(kLds <= 160 * 1024, "LDS budget");
  static_assert(SL >= 1 && SL * NW * 4 == BKV && kQLoads >= 1 && kQLoads * NW * 4 == BQ, "load split");
  static_assert(kQLoads <= kLoadsPerTile && NSTG * kLoadsPerTile < 64, "the waits cover the Q loads and the ring");
  static_assert((NSTG - 1) * kTileBytes < 65536, "stage offsets are 16-bit immediates");
};
using AttnWide = AttnShape<4, 2, 4>;
using AttnNarrow = AttnShape<2, 4, 2>;
// planning figures fitted to MI355X measurements: time per K/V tile of one wave of
// workgroups, and the cost of a key split beyond its tiles (the merge launch, plus the
// partials' round trip per split and query at 32 heads). Fitted jointly to every forced
// shape x split (1, 2, 3, 4, 8) inside the partial forwards of a 32-layer 8B-shaped model
// (the layer's K/V no longer cached when its attention runs, as in a step): L = 1024 with
// r = 17 .. 384 and L = 4096 with r = 96 .. 2048; the choices are the fastest measured
// candidate at 12 of the 14 points and within 1 % at the other two.
constexpr double kWideTileUs = 1.308;
constexpr double kNarrowTileUs = 1.873;
constexpr double kMergeUs = 2.501;
constexpr double kPartialUs = 0.01127;

// s_waitcnt vmcnt(min(n, K) * PER) for a wave-uniform run-time n >= 0
template <int PER, int K>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (n >= K) wait_vmcnt<K * PER>();
    else wait_tiles<PER, K - 1>(n);
  }
}

// {x[l % 32], x[l % 32 + 32]} on every lane l: a lane's value and its partner's in the
// other half of the wavefront, lower half first (v_permlane32_swap_b32, no LDS round trip)
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// grid: query tiles x heads x splits; dynamic LDS of SH::kLds bytes
template <typename SH, bool SPLIT>
__global__ void __launch_bounds__(SH::NT)
attn_bf16_kernel(const bf16* __restrict__ q_all, const AttnSeqs seqs, int L, int H, float scale_log2,
                 int kv_chunk, int nsplit, int r_all, bf16* __restrict__ out_all, float* __restrict__ po,
                 float* __restrict__ pml) {
  // K and V tiles in natural [key][dim] layout, one stage per tile of the ring: the K
  // stages first, then the V stages, so that with the tile loop unrolled over the stages
  // every fragment read is a per-lane base register (computed once) plus an immediate
  // offset below 64 KB. After the loop the LDS holds the (m, l, o) hand-over.
  constexpr int QG = SH::QG, KG = SH::KG, NW = SH::NW, BQ = SH::BQ, BKV = SH::BKV, SL = SH::SL;
  constexpr int kStages = SH::NSTG, kTileBytes = SH::kTileBytes, kVOff = SH::kVOff, kQOff = SH::kQOff;
  constexpr int kLoadsPerTile = SH::kLoadsPerTile, kQLoads = SH::kQLoads;
  // LDS layout (64 banks of 4 bytes): a K row keeps its 16-byte chunk c at c ^ (row % 16), so the
  // 16 rows one b128 fragment read serves per cycle hit 16 distinct bank groups; a V row keeps
  // its 64-byte quarter q (dims 32q .. 32q+31) at q ^ (row % 4), so the four consecutive keys of
  // a transposing read fall in distinct quarters.
  extern __shared__ __align__(16) unsigned char lds_raw[];

  // Logical block order: sequence by sequence, inside one split-major, then head, with the
  // query tiles of a head consecutive; the XCD-aware remap gives each XCD a contiguous
  // run of it, so the query tiles that read one head's K / V share one L2.
  int bid = xcd_remap(blockIdx.x, gridDim.x), si = 0, qtiles = 1;
  for (;;) {
    qtiles = (seqs.s[si].nr + BQ - 1) / BQ;
    const int nb = qtiles * H * nsplit;
    if (bid < nb || si + 1 >= seqs.n) break;
    bid -= nb;
    ++si;
  }
  if (seqs.s[si].nr <= 0) return;  // (the grid counts only sequences with rows; uniform per workgroup)
  const int qt = bid % qtiles, h = (bid / qtiles) % H, split = bid / (qtiles * H);
  const int row0 = seqs.s[si].row0, r = seqs.s[si].nr;
  const bf16* __restrict__ q = q_all + (int64_t)row0 * H * D;
  const bf16* __restrict__ kc = (const bf16*)seqs.s[si].k;
  const bf16* __restrict__ vc = (const bf16*)seqs.s[si].v;
  bf16* __restrict__ out = SPLIT ? nullptr : out_all + (int64_t)row0 * H * D;
  const int tid = threadIdx.x, lane = tid % 64;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int qw = wave % QG, kh = wave / QG;  // query group, 32-key part of every tile
  const int lq = lane % 32, g = lane / 32;
  const int64_t HD = (int64_t)H * D;
  const int qrow = qt * BQ + qw * 32 + lq;  // this lane's query (column of S^T)
  const bool qok = qrow < r;

  // Q tile through LDS like K (chunk c of row i at c ^ (i % 16)); rows past r re-read row r - 1
  {
    const __amdgpu_buffer_rsrc_t rQ = buffer_rsrc(q, (int64_t)r * HD * 2);
#pragma unroll
    for (int i = 0; i < kQLoads; ++i) {
      const int sl = i * NW + wave, row = 4 * sl + lane / 16, pos = lane % 16;
      const int qr = min(qt * BQ + row, r - 1);
      buffer_load_lds16(rQ, lds_raw + kQOff + sl * 1024,
                        (int)(((int64_t)qr * HD + h * D) * 2) + (pos ^ (row & 15)) * 16, 0);
    }
  }

  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  // reference max (log2 units) and row sum. The max starts at a finite floor, not -inf:
  // a wavefront whose keys are all masked (its half of a split holding at most 32 keys,
  // or a cache of at most 32 rows) then gets p = 2^(-inf - floor) = 0 instead of
  // 2^(-inf + inf) = NaN, and hands over o = 0, l = 0 with a weight of 0.
  float m_ref = kMaxFloor, l_run = 0.f;

  const int kv_lo = split * kv_chunk;
  const int kv_hi = min(L, kv_lo + kv_chunk);
  const int ntiles = (kv_hi - kv_lo + BKV - 1) / BKV;

  // a tile is BKV / 4 slices of 1 KB (4 rows of 256 bytes) of K and as many of V;
  // wavefront w loads slices w, NW + w, ... of both. Lane l of a slice load fills bytes
  // 16 l of the slice, i.e. tile row 4 s + l / 16 at position l % 16, and fetches the
  // 16-byte chunk that the swizzle puts there. Keys past the cache end re-read row L - 1
  // (masked below).
  const __amdgpu_buffer_rsrc_t rK = buffer_rsrc(kc, (int64_t)L * HD * 2);
  const __amdgpu_buffer_rsrc_t rV = buffer_rsrc(vc, (int64_t)L * HD * 2);
  int lrow[SL], ok_[SL], ov_[SL];
#pragma unroll
  for (int i = 0; i < SL; ++i) {
    const int sl = i * NW + wave, row = 4 * sl + lane / 16, pos = lane % 16;
    lrow[i] = row;
    const int ck = (pos ^ (row & 15)) * 16;  // bytes within the row
    const int cv = ((((pos >> 2) ^ (row & 3)) << 2) | (pos & 3)) * 16;
    const int rb = (int)(((int64_t)row * HD + h * D) * 2);
    ok_[i] = rb + ck;
    ov_[i] = rb + cv;
  }
  // a whole tile takes its key offset in the scalar offset of the load; the last tile of a
  // range that ends past the cache (keys >= L) clamps each lane's row instead
  auto issue = [&](int t, int stage) __attribute__((always_inline)) {
    const int kv0 = kv_lo + t * BKV;
    unsigned char* sk = lds_raw + stage * kTileBytes;
    unsigned char* sv = lds_raw + kVOff + stage * kTileBytes;
    if (kv0 + BKV <= L) {
      const int so = (int)((int64_t)kv0 * HD * 2);
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        buffer_load_lds16(rK, sk + (i * NW + wave) * 1024, ok_[i], so);
        buffer_load_lds16(rV, sv + (i * NW + wave) * 1024, ov_[i], so);
      }
    } else {
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int key = min(kv0 + lrow[i], L - 1);
        const int d0 = (int)(((int64_t)(key - lrow[i]) * HD) * 2);
        buffer_load_lds16(rK, sk + (i * NW + wave) * 1024, ok_[i] + d0, 0);
        buffer_load_lds16(rV, sv + (i * NW + wave) * 1024, ov_[i] + d0, 0);
      }
    }
  };

  // transpose-read coordinates for the V^T operand: within each 16-lane group, source lane
  // s points at (key base + s/4, dim base + 4 (s%4)); ds_read_tr16_b64 then hands lane j the
  // four keys of dim base + j
  const int tr_key = (lane % 16) / 4, tr_dim = 16 * ((lane / 16) % 2) + 4 * (lane % 4);

  int issued = min(kStages, ntiles);
#pragma unroll
  for (int t = 0; t < kStages; ++t)
    if (t < issued) issue(t, t);
  // Q fragments (B operand of S^T): Q[qrow][16kk + 8g .. +7], read once the Q loads (older
  // than every tile's) have landed in every wavefront
  wait_tiles<kLoadsPerTile, kStages>(issued);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  bf16x8 fq[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    fq[kk] = *reinterpret_cast<const bf16x8*>(lds_raw + kQOff + (qw * 32 + lq) * (D * 2) +
                                               (((2 * kk + g) ^ (lq & 15)) * 16));
  // per-lane LDS offsets of the fragment reads (the stage adds an immediate): the V ones
  // carry the V region's offset (64 KB in both shapes) themselves, passed through an empty
  // asm so that the compiler keeps it in the register and the stage offset stays a 16-bit
  // immediate
  int koff[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) koff[kk] = ((kh * 32 + lq) * KS + (((2 * kk + g) ^ (lq & 15)) * 8)) * 2;
  int voff[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    voff[i] = kVOff + ((kh * 32 + 4 * g + tr_key) * KS + 32 * (i ^ tr_key) + tr_dim) * 2;
    __asm__ volatile("" : "+v"(voff[i]));
  }
  for (int t0 = 0; t0 < ntiles; t0 += kStages)
#pragma unroll
  for (int u = 0; u < kStages; ++u) {
    const int t = t0 + u;
    if (t >= ntiles) break;
    // this wavefront's loads of tile t (and of Q) have landed once at most the loads of
    // the tiles issued after t are outstanding; the barrier then publishes every
    // wavefront's share, and tells that all have finished tile t - 1, whose stage is
    // refilled with tile t - 1 + kStages
    wait_tiles<kLoadsPerTile, kStages - 1>(issued - t - 1);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (t >= 1 && t - 1 + kStages < ntiles) {
      issue(t - 1 + kStages, (u + kStages - 1) % kStages);
      ++issued;
    }
    const int kv0 = kv_lo + t * BKV;
    const unsigned char* kst = lds_raw + u * kTileBytes;   // + koff[kk]
    const unsigned char* vst = lds_raw + u * kTileBytes;   // + voff[i] (which holds kVOff)
    {
      const int sub = kh;  // this wavefront's 32 keys of the tile
      // ---- S^T[32 keys, 32 queries] (raw dot products)
      f32x16 st;
#pragma unroll
      for (int v = 0; v < 16; ++v) st[v] = 0.f;
      // all K fragments first, so that the MFMA chain waits for LDS once; the fence keeps
      // the scheduler from folding the eight reads into one register set read just in time
      // (one LDS round trip per MFMA)
      bf16x8 fk[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) fk[kk] = *reinterpret_cast<const bf16x8*>(kst + koff[kk]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[kk], fq[kk], st, 0, 0, 0);
      // key of st[v]: kv0 + sub*32 + 8(v/4) + 4g + v%4; mask keys past the end of the range
      if (kv0 + sub * 32 + 32 > kv_hi) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (kv0 + sub * 32 + 8 * (v / 4) + 4 * g + (v % 4) >= kv_hi) st[v] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) tmax = fmaxf(tmax, st[v]);
      {
        float a, b;
        half_pair(tmax, a, b);
        tmax = fmaxf(a, b) * scale_log2;
      }
      // lazy rescale: only when some row's max moved past the reference by 2^kRescale.
      // The reference is kept an integer (base-2 units), so every probability rounded to
      // bf16 below is 2^(t - M) for an integer M: bf16 rounding commutes with scaling by
      // powers of two, so the rounded weights equal those taken against the row's final
      // (integer) maximum, whatever the tiling, the split or the order of rescales.
      if (__any(tmax > m_ref + kRescale)) {
        const float m_new = ceilf(fmaxf(m_ref, tmax));
        const float alpha = __builtin_amdgcn_exp2f(m_ref - m_new);  // 0 on the first tile
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
        m_ref = m_new;
      }
      float psum = 0.f;
      bf16x8 fp[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[v], scale_log2, -m_ref));
        psum += p;
        fp[v / 8][v % 8] = (bf16)p;
      }
      {
        float a, b;
        half_pair(psum, a, b);
        l_run += a + b;
      }
      // ---- O^T[d, q] += V^T[d, keys] P^T[keys, q]; A operand by transpose reads, all
      // eight fragments read before the MFMAs
      bf16x8 fv[2][D / 32];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          // key sub*32 + 16c + 4g + tr_key (= tr_key mod 4), dims 32 (i ^ tr_key) + tr_dim
          const lds_bf16* p0 = (const lds_bf16*)(vst + voff[i] + 16 * c * KS * 2);
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * KS));
          const bf16x4 l4 = __builtin_bit_cast(bf16x4, lo), h4 = __builtin_bit_cast(bf16x4, hi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            fv[c][i][e] = l4[e];
            fv[c][i][4 + e] = h4[e];
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[c][i], fp[c], o[i], 0, 0, 0);
    }
  }
  __syncthreads();  // every wavefront is done with the last tile; no loads are outstanding

  // the wavefronts of each query group that took keys 32 .. BKV - 1 of the tiles hand their
  // (m, l, o) to the one that took keys 0 .. 31 through LDS, which merges them in key order
  if constexpr (KG > 1) {
    constexpr int XS = D / 2 + 2;  // floats per lane: 64 of o, m, l
    float* xb = reinterpret_cast<float*>(lds_raw);
    if (kh > 0) {
      float* x = xb + (((kh - 1) * QG + qw) * 64 + lane) * XS;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) x[16 * i + v] = o[i][v];
      x[D / 2] = m_ref;
      x[D / 2 + 1] = l_run;
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int k = 1; k < KG; ++k) {
      const float* x = xb + (((k - 1) * QG + qw) * 64 + lane) * XS;
      const float m2 = x[D / 2], l2 = x[D / 2 + 1];
      const float mm = fmaxf(m_ref, m2);
      const float a1 = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - mm);
      const float a2 = m2 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - mm);
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[i][v] = o[i][v] * a1 + x[16 * i + v] * a2;
      l_run = l_run * a1 + l2 * a2;
      m_ref = mm;
    }
  }
  if (!qok) return;
  // o[i][v]: dim = 32i + 8(v/4) + 4g + v%4 of query qrow
  if (!SPLIT) {
    const float inv = 1.0f / l_run;
    bf16* dst = out + (int64_t)qrow * HD + h * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[32 * i + 8 * (v / 4) + 4 * g + (v % 4)] = (bf16)(o[i][v] * inv);
  } else {
    float* dst = po + (((int64_t)split * r_all + row0 + qrow) * H + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) dst[32 * i + 8 * (v / 4) + 4 * g + (v % 4)] = o[i][v];
    if (g == 0) {
      float* ml = pml + (((int64_t)split * r_all + row0 + qrow) * H + h) * 2;
      ml[0] = m_ref;
      ml[1] = l_run;
    }
  }
}

// combine split partials: one thread per (query, head, dim). With the split count SP
// known at compile time every partial is loaded before the first use (one memory round
// trip instead of two per split); SP < 0 takes S at run time. The arithmetic and its
// order are the same either way.
template <typename T, int SP>
__global__ void __launch_bounds__(kThreads)
attn_merge_kernel(const float* __restrict__ po, const float* __restrict__ pml, int S, int r,
                  int H, int Dh, T* __restrict__ out) {
  const int64_t t = blockIdx.x * (int64_t)kThreads + threadIdx.x;
  if (t >= (int64_t)r * H * Dh) return;
  const int64_t qh = t / Dh;
  const int d = (int)(t % Dh);
  const int64_t rh = (int64_t)r * H;
  float m = -INFINITY, l = 0.f, acc = 0.f;
  if constexpr (SP > 0) {
    float mv[SP], lv[SP], ov[SP];
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      mv[s] = pml[(s * rh + qh) * 2];
      lv[s] = pml[(s * rh + qh) * 2 + 1];
      ov[s] = po[(s * rh + qh) * Dh + d];
    }
#pragma unroll
    for (int s = 0; s < SP; ++s) m = fmaxf(m, mv[s]);
    // a split with no finite score is skipped by selects, not a branch (which would let the
    // compiler sink its loads behind the first wait)
#pragma unroll
    for (int s = 0; s < SP; ++s) {
      const bool live = mv[s] != -INFINITY;
      const float w = exp2f(mv[s] - m);
      const float l2 = l + lv[s] * w, a2 = acc + ov[s] * w;
      l = live ? l2 : l;
      acc = live ? a2 : acc;
    }
  } else {
    for (int s = 0; s < S; ++s) m = fmaxf(m, pml[(s * rh + qh) * 2]);
    for (int s = 0; s < S; ++s) {
      const float ms = pml[(s * rh + qh) * 2];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - m);
      l += pml[(s * rh + qh) * 2 + 1] * w;
      acc += po[(s * rh + qh) * Dh + d] * w;
    }
  }
  out[qh * Dh + d] = from_f<T>(acc / l);
}

template <int SP>
ec_status launch_merge(const float* po, const float* pml, int S, int r, int H, int Dh, bf16* out, hipStream_t s) {
  const int64_t n = (int64_t)r * H * Dh;
  attn_merge_kernel<bf16, SP><<<(int)((n + kThreads - 1) / kThreads), kThreads, 0, s>>>(po, pml, S, r, H, Dh, out);
  EC_CHECK_LAUNCH("attn_merge_kernel");
  return EC_OK;
}

// fp32 path for other head sizes: one workgroup per (query, head); scores in LDS, exact softmax.
__global__ void __launch_bounds__(kThreads)
attn_f32_kernel(const float* __restrict__ q, const AttnSeqs seqs, int L, int H, int Dh, float scale,
                float* __restrict__ out) {
  extern __shared__ float sc[];  // [L] scores, then [Dh] query
  float* sq = sc + L;
  const int i = blockIdx.x, h = blockIdx.y;  // i: row of the compact q / out of all sequences
  int si = 0;
  while (si + 1 < seqs.n && i >= seqs.s[si].row0 + seqs.s[si].nr) ++si;
  const float* __restrict__ kc = (const float*)seqs.s[si].k;
  const float* __restrict__ vc = (const float*)seqs.s[si].v;
  const int64_t HD = (int64_t)H * Dh;
  for (int d = threadIdx.x; d < Dh; d += kThreads) sq[d] = q[(int64_t)i * HD + h * Dh + d];
  __syncthreads();
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < L; j += kThreads) {
    const float* kr = kc + (int64_t)j * HD + h * Dh;
    float s = 0.f;
    for (int d = 0; d < Dh; ++d) s = fmaf(sq[d], kr[d], s);
    s *= scale;
    sc[j] = s;
    mx = fmaxf(mx, s);
  }
  __shared__ float red[kThreads];
  red[threadIdx.x] = mx;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  mx = red[0];
  __syncthreads();
  float sum = 0.f;
  for (int j = threadIdx.x; j < L; j += kThreads) {
    const float e = __expf(sc[j] - mx);
    sc[j] = e;
    sum += e;
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const float inv = 1.0f / red[0];
  for (int d = threadIdx.x; d < Dh; d += kThreads) {
    float acc = 0.f;
    for (int j = 0; j < L; ++j) acc = fmaf(sc[j], vc[(int64_t)j * HD + h * Dh + d], acc);
    out[(int64_t)i * HD + h * Dh + d] = acc * inv;
  }
}

// fp32 path on the matrix unit (v_mfma_f32_32x32x2_f32): one wavefront per 32 queries of
// one sequence and one head, transposed like the bf16 kernel so that the probabilities
// feed the second product from the registers that hold the scores:
//   S^T[32 keys, 32 queries] = K Q^T   (lane l: query l % 32; keys 8 (v / 4) + 4 (l / 32) + v % 4)
//   O^T[Dh, 32 queries]     += V^T P^T (register v of a lane is the B operand of one MFMA
//                                       over the key pair {8 (v / 4) + v % 4, + 4})
// over blocks of 32 keys with an online softmax (running max and sum per query, kept by
// the two lanes l and l ^ 32 that share a query). The K and Q operands use four
// consecutive head dimensions per lane, 4 (l / 32) into each 8-wide step (MFMA j takes
// dimensions d + j and d + 4 + j). Q stays in registers; K and V come from the cache.
template <int DH>
__global__ void __launch_bounds__(256)
attn_f32_mfma_kernel(const float* __restrict__ q_all, const AttnSeqs seqs, int L, int H, float scale,
                     float* __restrict__ out_all, int waves_total) {
  const int lane = threadIdx.x % 64;
  int w = blockIdx.x * 4 + threadIdx.x / 64;
  if (w >= waves_total) return;  // a whole wavefront
  int si = 0, qtiles = 0;
  for (;;) {
    qtiles = (seqs.s[si].nr + 31) / 32;
    if (w < qtiles * H || si + 1 >= seqs.n) break;
    w -= qtiles * H;
    ++si;
  }
  if (qtiles == 0) return;  // (not reached: the grid counts only sequences with rows)
  const int qt = w % qtiles, h = w / qtiles;
  const int r = seqs.s[si].nr;
  const int64_t HD = (int64_t)H * DH;
  const float* __restrict__ q = q_all + (int64_t)seqs.s[si].row0 * HD + h * DH;
  const float* __restrict__ kc = (const float*)seqs.s[si].k + h * DH;
  const float* __restrict__ vc = (const float*)seqs.s[si].v + h * DH;
  float* __restrict__ out = out_all + (int64_t)seqs.s[si].row0 * HD + h * DH;
  const int c = lane % 32, hf = lane / 32;
  const int qrow = qt * 32 + c;
  float4 fq[DH / 8];
  {
    const float* qr = q + (int64_t)min(qrow, r - 1) * HD + 4 * hf;
#pragma unroll
    for (int j = 0; j < DH / 8; ++j) fq[j] = *reinterpret_cast<const float4*>(qr + 8 * j);
  }
  f32x16 o[DH / 32];
#pragma unroll
  for (int i = 0; i < DH / 32; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) o[i][v] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int kb = 0; kb < L; kb += 32) {
    f32x16 st;
#pragma unroll
    for (int v = 0; v < 16; ++v) st[v] = 0.f;
    const float* kr = kc + (int64_t)min(kb + c, L - 1) * HD + 4 * hf;
#pragma unroll
    for (int j = 0; j < DH / 8; ++j) {
      const float4 k4 = *reinterpret_cast<const float4*>(kr + 8 * j);
      st = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.x, fq[j].x, st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.y, fq[j].y, st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.z, fq[j].z, st, 0, 0, 0);
      st = __builtin_amdgcn_mfma_f32_32x32x2f32(k4.w, fq[j].w, st, 0, 0, 0);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = kb + 8 * (v / 4) + 4 * hf + (v % 4);
      st[v] = key < L ? st[v] * scale : -INFINITY;
      tmax = fmaxf(tmax, st[v]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);  // finite: every block holds a key below L
    const float alpha = __expf(m_run - m_new);  // 0 on the first block
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) o[i][v] *= alpha;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      st[v] = __expf(st[v] - m_new);
      psum += st[v];
    }
    l_run = l_run * alpha + psum + __shfl_xor(psum, 32);
    m_run = m_new;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int key = min(kb + 8 * (v / 4) + 4 * hf + (v % 4), L - 1);  // past L: weight 0
      const float* vr = vc + (int64_t)key * HD + c;
#pragma unroll
      for (int i = 0; i < DH / 32; ++i)
        o[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * i], st[v], o[i], 0, 0, 0);
    }
  }
  // O^T element v of lane l: dimension 8 (v / 4) + 4 (l / 32) + v % 4 of block i, query l % 32
  if (qrow < r) {
    const float inv = 1.0f / l_run;
    float* orow = out + (int64_t)qrow * HD;
#pragma unroll
    for (int i = 0; i < DH / 32; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) orow[32 * i + 8 * (v / 4) + 4 * hf + (v % 4)] = o[i][v] * inv;
  }
}

struct AttnPlan {
  bool narrow;  // AttnNarrow workgroups (64 queries) instead of AttnWide (128)
  int splits, chunk;
};

// Workgroup shape and key-range split by a cost model fitted to MI355X measurements of
// every shape and split count (r = 17 .. 4096 queries, L = 1024 and 4096, 32 heads, K/V
// warm and cold; it picks the fastest candidate or one within 6 % of it on each): waves of
// workgroups x tiles per workgroup x the shape's time per tile, plus, when split, the
// merge launch and the partials' round trip per (split x query), scaled by H / 32. The
// narrow shape wins from 17 to about 600 query rows (skip steps), the wide one above. r is the number of query
// rows over every sequence of the launch and qt_wide / qt_narrow its number of query tiles
// for each shape; splits whose partials would not fit max_ws bytes are skipped.
AttnPlan plan_attn(int r, int qt_wide, int qt_narrow, int L, int H, size_t max_ws = (size_t)-1) {
  AttnPlan best_p{false, 1, 0};
  double best = 1e300;
  for (int nar = 0; nar < 2; ++nar) {
    const int bkv = nar ? AttnNarrow::BKV : AttnWide::BKV;
    const int base = (nar ? qt_narrow : qt_wide) * H;
    const double tile_us = nar ? kNarrowTileUs : kWideTileUs;
    for (int s : {1, 2, 3, 4, 6, 8, 12, 16}) {
      if (s > 1 && L / s < bkv) break;
      const int chunk = ((L + s - 1) / s + bkv - 1) / bkv * bkv;
      const int splits = (L + chunk - 1) / chunk;
      if (splits > 1 && (size_t)splits * r * H * (D + 2) * sizeof(float) + 512 > max_ws) continue;
      const double waves = (double)(((int64_t)base * splits + 255) / 256);
      double us = waves * (chunk / bkv) * tile_us;
      if (splits > 1) us += kMergeUs + kPartialUs * splits * r * (H / 32.0);
      if (us < best) {
        best = us;
        best_p = AttnPlan{nar != 0, splits, chunk};
      }
    }
  }
  return best_p;
}

template <typename SH>
ec_status launch_attn(const AttnPlan& p, const bf16* q, const AttnSeqs& seqs, int L, int H, float sl, int r,
                      int qtiles, void* out, void* ws, hipStream_t s) {
  const unsigned grid = (unsigned)((int64_t)qtiles * H * p.splits);
  // one limit record per kernel (the two instantiations share a function type)
  static LdsLimit whole, split;
  const ec_status st = p.splits == 1 ? whole.ensure((const void*)attn_bf16_kernel<SH, false>, SH::kLds)
                                     : split.ensure((const void*)attn_bf16_kernel<SH, true>, SH::kLds);
  if (st != EC_OK) return st;
  if (p.splits == 1) {
    attn_bf16_kernel<SH, false><<<grid, SH::NT, SH::kLds, s>>>(q, seqs, L, H, sl, p.chunk, 1, r, (bf16*)out,
                                                              nullptr, nullptr);
    EC_CHECK_LAUNCH("attn_bf16_kernel");
    return EC_OK;
  }
  float* po = (float*)ws;
  float* pml = po + (size_t)p.splits * r * H * D;
  attn_bf16_kernel<SH, true><<<grid, SH::NT, SH::kLds, s>>>(q, seqs, L, H, sl, p.chunk, p.splits, r, nullptr, po,
                                                           pml);
  EC_CHECK_LAUNCH("attn_bf16_kernel");
  bf16* o = (bf16*)out;
  switch (p.splits) {
#define EC_MERGE_CASE(n) \
  case n: return launch_merge<n>(po, pml, p.splits, r, H, D, o, s);
    EC_MERGE_CASE(2) EC_MERGE_CASE(3) EC_MERGE_CASE(4) EC_MERGE_CASE(5) EC_MERGE_CASE(6) EC_MERGE_CASE(7)
    EC_MERGE_CASE(8) EC_MERGE_CASE(9) EC_MERGE_CASE(10) EC_MERGE_CASE(11) EC_MERGE_CASE(12)
    EC_MERGE_CASE(13) EC_MERGE_CASE(14) EC_MERGE_CASE(15) EC_MERGE_CASE(16)
#undef EC_MERGE_CASE
    default: return launch_merge<-1>(po, pml, p.splits, r, H, D, o, s);
  }
}

}  // namespace

size_t attn_ws_bytes(int r, int L, int H, int Dh) {
  if (r <= 0 || Dh != D) return 0;
  const AttnPlan p = plan_attn(r, (r + AttnWide::BQ - 1) / AttnWide::BQ, (r + AttnNarrow::BQ - 1) / AttnNarrow::BQ,
                               L, H);
  if (p.splits <= 1) return 0;
  return (size_t)p.splits * r * H * (Dh + 2) * sizeof(float) + 512;
}

void attn_plan_query(int r, int L, int H, int* query_tile, int* splits) {
  const AttnPlan p = plan_attn(r, (r + AttnWide::BQ - 1) / AttnWide::BQ, (r + AttnNarrow::BQ - 1) / AttnNarrow::BQ,
                               L, H);
  *query_tile = p.narrow ? AttnNarrow::BQ : AttnWide::BQ;
  *splits = p.splits;
}

ec_status attn(ec_dtype dt, const void* q, const void* k, const void* v, int r, int L, int H,
               int Dh, float scale, void* out, void* ws, size_t ws_bytes, hipStream_t s) {
  AttnSeqs one{};
  one.n = 1;
  one.s[0] = AttnSeq{0, r, k, v};
  return attn_batch(dt, q, one, L, H, Dh, scale, out, ws, ws_bytes, s);
}

ec_status attn_batch(ec_dtype dt, const void* q, const AttnSeqs& seqs, int L, int H, int Dh, float scale, void* out,
                     void* ws, size_t ws_bytes, hipStream_t s) {
  EC_REQUIRE(seqs.n >= 1 && seqs.n <= EC_MAX_SEQ, EC_ERR_ARG, "attn: %d sequences", seqs.n);
  int r = 0, qt_wide = 0, qt_narrow = 0;
  for (int i = 0; i < seqs.n; ++i) {
    EC_REQUIRE(seqs.s[i].nr >= 0 && seqs.s[i].row0 == r, EC_ERR_ARG, "attn: sequence %d rows not contiguous", i);
    EC_REQUIRE(seqs.s[i].nr == 0 || (seqs.s[i].k && seqs.s[i].v), EC_ERR_ARG, "attn: null cache of sequence %d", i);
    r += seqs.s[i].nr;
    qt_wide += (seqs.s[i].nr + AttnWide::BQ - 1) / AttnWide::BQ;
    qt_narrow += (seqs.s[i].nr + AttnNarrow::BQ - 1) / AttnNarrow::BQ;
  }
  if (r == 0) return EC_OK;
  EC_REQUIRE(L >= 1, EC_ERR_ARG, "attn: seq_len must be >= 1");
  if (dt == EC_F32) {
    uintptr_t align = (uintptr_t)q | (uintptr_t)out;
    for (int i = 0; i < seqs.n; ++i) align |= (uintptr_t)seqs.s[i].k | (uintptr_t)seqs.s[i].v;
    if ((Dh == 32 || Dh == 64 || Dh == 128) && align % 16 == 0) {  // matrix-unit path (16-byte row loads)
      int waves = 0;
      for (int i = 0; i < seqs.n; ++i) waves += (seqs.s[i].nr + 31) / 32 * H;
      const int blocks = (waves + 3) / 4;
#define EC_F32_ATTN(DHV)                                                                                     attn_f32_mfma_kernel<DHV><<<blocks, 256, 0, s>>>((const float*)q, seqs, L, H, scale, (float*)out, waves)
      if (Dh == 32) EC_F32_ATTN(32);
      else if (Dh == 64) EC_F32_ATTN(64);
      else EC_F32_ATTN(128);
#undef EC_F32_ATTN
      EC_CHECK_LAUNCH("attn_f32_mfma_kernel");
      return EC_OK;
    }
    EC_REQUIRE(Dh <= 1024 && (size_t)(L + Dh) * 4 <= 64 * 1024, EC_ERR_UNSUPPORTED,
               "attn: f32 path supports L + head_dim <= 16384");
    dim3 grid(r, H);
    attn_f32_kernel<<<grid, kThreads, (L + Dh) * sizeof(float), s>>>((const float*)q, seqs, L, H, Dh, scale,
                                                                     (float*)out);
    EC_CHECK_LAUNCH("attn_f32_kernel");
    return EC_OK;
  }
  EC_REQUIRE(Dh == D, EC_ERR_UNSUPPORTED, "attn: bf16 path needs head_dim 128 (got %d)", Dh);
  // q and the caches are addressed through buffer resources with 32-bit byte offsets
  EC_REQUIRE((int64_t)(L > r ? L : r) * H * Dh * 2 <= 0x7fffffff, EC_ERR_UNSUPPORTED,
             "attn: %d rows of %d x %d bf16 exceed the 2 GiB buffer range", L > r ? L : r, H, Dh);
  const AttnPlan p = plan_attn(r, qt_wide, qt_narrow, L, H, ws ? ws_bytes : 0);
  const float sl = scale * kLog2e;
  if (p.narrow) return launch_attn<AttnNarrow>(p, (const bf16*)q, seqs, L, H, sl, r, qt_narrow, out, ws, s);
  return launch_attn<AttnWide>(p, (const bf16*)q, seqs, L, H, sl, r, qt_wide, out, ws, s);
}

}  // namespace ec
