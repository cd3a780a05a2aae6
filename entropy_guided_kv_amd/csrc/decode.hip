// Decode, decide and plan: the per-step bookkeeping of EntropyCache.
//
// After the entropy reduction of the candidate rows, one workgroup
//   - picks the min(n, #candidates) candidates with the largest confidence
//     (max softmax probability; ties to the lower position) and writes their
//     argmax ids into the token buffer, in ascending position order;
//   - appends them to the decode-time ring, which holds the last k decoded
//     positions (O(k) extra memory, Italian summary section 4; the record of
//     decode times from which the k most recent tokens are taken, Arabic
//     technical summary section 2, phase 3);
//   - takes E = max entropy over the decoded rows (the decision signal);
//   - builds the next step's lists: R = still-masked positions + ring
//     (ascending), the candidates (masked positions of the lowest block that
//     still has a mask; or, in sliding-window mode, the masked positions of the
//     B positions from the lowest masked one) and each candidate's index in R.
// It then writes a small result record that the host copies back once.
#include "ec_internal.h"

#include <math.h>

#include <algorithm>

namespace ec {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxL = 65536;

// exclusive prefix sum over the workgroup; *total receives the sum
__device__ int block_excl_scan(int v, int* total, int* sh) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kWaves; ++w) {
      int t = sh[w];
      sh[w] = acc;
      acc += t;
    }
    sh[kWaves] = acc;
  }
  __syncthreads();
  const int res = sh[wave] + x - v;
  *total = sh[kWaves];
  __syncthreads();
  return res;
}

__device__ int block_min(int v, int* sh) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = min(v, __shfl_xor(v, o));
  if (threadIdx.x % 64 == 0) sh[threadIdx.x / 64] = v;
  __syncthreads();
  int m = sh[0];
  for (int w = 1; w < kWaves; ++w) m = min(m, sh[w]);
  __syncthreads();
  return m;
}

// Build R, candidates and candidate indices from masked[] and the ring.
__device__ void build_plan(const uint8_t* masked, int32_t* plan, int L, int P, int B, int k, int window,
                           StepResult* res) {
  __shared__ uint32_t ringbits[kMaxL / 32];
  __shared__ int sh[kWaves + 1];
  const PlanLayout lay(L, k);
  const int words = (L + 31) / 32;
  for (int w = threadIdx.x; w < words; w += kThreads) ringbits[w] = 0;
  __syncthreads();
  const int count = plan[0];
  const int nring = min(count, k);
  for (int e = threadIdx.x; e < nring; e += kThreads) {
    const int p = plan[8 + e];
    atomicOr(&ringbits[p / 32], 1u << (p % 32));
  }
  __syncthreads();

  // contiguous range of positions per thread
  const int per = (L + kThreads - 1) / kThreads;
  const int lo = min(L, threadIdx.x * per), hi = min(L, lo + per);
  int cnt = 0, mcnt = 0, mmin = L;
  for (int p = lo; p < hi; ++p) {
    const int m = masked[p] != 0;
    const int inr = (ringbits[p / 32] >> (p % 32)) & 1;
    cnt += (m | inr);
    mcnt += m;
    if (m && p < mmin) mmin = p;
  }
  int nR, nM;
  int off = block_excl_scan(cnt, &nR, sh);
  block_excl_scan(mcnt, &nM, sh);
  int32_t* R = plan + lay.R0;
  for (int p = lo; p < hi; ++p) {
    const int m = masked[p] != 0;
    const int inr = (ringbits[p / 32] >> (p % 32)) & 1;
    if (m | inr) R[off++] = p;
  }
  // candidates: masked positions of the lowest open block [P + bB, P + (b+1)B), or
  // of the window [first, first + B) that starts at the lowest masked position
  const int first = block_min(mmin, sh);
  int clo = L, chi = L;
  if (first < L) {
    clo = window ? first : P + ((first - P) / B) * B;
    chi = min(L, clo + B);
  }
  int ccnt = 0;
  for (int p = max(lo, clo); p < min(hi, chi); ++p) ccnt += masked[p] != 0;
  int nC;
  int coff = block_excl_scan(ccnt, &nC, sh);
  int32_t* C = plan + lay.C0;
  for (int p = max(lo, clo); p < min(hi, chi); ++p)
    if (masked[p]) C[coff++] = p;
  __syncthreads();
  // index of each candidate in R (R ascending): lower bound
  int32_t* I = plan + lay.I0;
  for (int i = threadIdx.x; i < nC; i += kThreads) {
    const int p = C[i];
    int a = 0, z = nR;
    while (a < z) {
      const int mid = (a + z) / 2;
      if (R[mid] < p) a = mid + 1;
      else z = mid;
    }
    I[i] = a;
  }
  if (threadIdx.x == 0) {
    plan[1] = nR;
    plan[2] = nC;
    plan[3] = nM;
    res->next_rows = nR;
    res->next_cand = nC;
    res->n_masked = nM;
  }
}

__global__ void __launch_bounds__(kThreads)
reset_kernel(int32_t* tokens, uint8_t* masked, int32_t* plan, int L, int P, int B, int k, int window,
             int mask_id, StepResult* res) {
  const PlanLayout lay(L, k);
  for (int p = threadIdx.x; p < L; p += kThreads) {
    masked[p] = p >= P ? 1 : 0;
    if (p >= P) tokens[p] = mask_id;
    plan[lay.J0 + p] = p;
  }
  if (threadIdx.x == 0) plan[0] = 0;
  for (int e = threadIdx.x; e < lay.K; e += kThreads) plan[8 + e] = -1;
  __syncthreads();
  build_plan(masked, plan, L, P, B, k, window, res);
  if (threadIdx.x == 0) {
    res->n_picked = 0;
    res->has_nan = 0;
    res->emax = -INFINITY;
  }
}

__global__ void __launch_bounds__(kThreads)
select_kernel(const float* __restrict__ H, const int32_t* __restrict__ amax,
              const float* __restrict__ conf, int n_cand, int32_t* tokens, uint8_t* masked,
              int32_t* plan, int L, int P, int B, int k, int window, int n, StepResult* res) {
  const PlanLayout lay(L, k);
  __shared__ int by_rank[EC_MAX_TOKENS_PER_STEP];
  __shared__ float emax_sh[EC_MAX_TOKENS_PER_STEP];
  __shared__ int nan_sh[EC_MAX_TOKENS_PER_STEP];
  const int32_t* C = plan + lay.C0;
  const int npick = min(n, n_cand);
  const int count0 = plan[0];
  // rank of every candidate in (confidence desc, position asc); NaN ranks lowest
  for (int i = threadIdx.x; i < n_cand; i += kThreads) {
    float ci = conf[i];
    if (ci != ci) ci = -1.f;
    const int pi = C[i];
    int rank = 0;
    for (int j = 0; j < n_cand; ++j) {
      float cj = conf[j];
      if (cj != cj) cj = -1.f;
      rank += (cj > ci) || (cj == ci && C[j] < pi);
    }
    if (rank < npick) by_rank[rank] = i;
  }
  __syncthreads();
  if (threadIdx.x < npick) {
    const int i = by_rank[threadIdx.x];
    const int p = C[i];
    int slot = 0;
    for (int t = 0; t < npick; ++t) slot += C[by_rank[t]] < p;
    const int id = amax[i];
    tokens[p] = id;
    masked[p] = 0;
    // The step's positions enter the decode record in ascending order (slots 0 ..
    // npick-1 after the count0 earlier entries). Only the last k of them can be among
    // the k most recent entries, so only those write the ring: they are at most k
    // consecutive record indices, hence distinct ring slots (one writer per slot).
    if (k > 0 && slot >= npick - k) plan[8 + (count0 + slot) % lay.K] = p;
    res->pos[slot] = p;
    res->ids[slot] = id;
    res->ent[slot] = H[i];
    res->conf[slot] = conf[i];
    const float h = H[i];
    nan_sh[threadIdx.x] = h != h;
    emax_sh[threadIdx.x] = h;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float e = -INFINITY;
    int nan = 0;
    for (int t = 0; t < npick; ++t) {
      nan |= nan_sh[t];
      if (!nan_sh[t]) e = fmaxf(e, emax_sh[t]);
    }
    res->n_picked = npick;
    res->has_nan = nan;
    res->emax = nan ? NAN : e;
    plan[0] = count0 + npick;
  }
  __syncthreads();
  build_plan(masked, plan, L, P, B, k, window, res);
}

}  // namespace

ec_status plan_reset(int32_t* tokens, uint8_t* masked, int32_t* plan, const ec_params& p,
                     StepResult* res, hipStream_t s) {
  EC_REQUIRE(p.seq_len <= kMaxL, EC_ERR_UNSUPPORTED, "seq_len %d > %d", p.seq_len, kMaxL);
  reset_kernel<<<1, kThreads, 0, s>>>(tokens, masked, plan, p.seq_len, p.prompt_len, p.block_len,
                                      p.k_recent, p.candidates == EC_CAND_WINDOW, p.mask_id, res);
  EC_CHECK_LAUNCH("reset_kernel");
  return EC_OK;
}

__global__ void __launch_bounds__(kThreads)
batch_gather_kernel(BatchSegs b, int32_t* __restrict__ rows_all, int32_t* __restrict__ row_seq,
                    int32_t* __restrict__ out_all) {
  const BatchSeg g = b.seg[blockIdx.y];
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < g.n_rows; i += gridDim.x * kThreads) {
    rows_all[g.row_off + i] = g.rows[i];
    row_seq[g.row_off + i] = g.seq;
  }
  for (int j = blockIdx.x * kThreads + threadIdx.x; j < g.n_cand; j += gridDim.x * kThreads)
    out_all[g.cand_off + j] = g.row_off + g.cidx[j];
}

ec_status batch_gather(const BatchSegs& b, int max_rows, int32_t* rows_all, int32_t* row_seq,
                       int32_t* out_all, hipStream_t s) {
  if (b.n == 0) return EC_OK;
  dim3 grid((unsigned)std::max(1, std::min((max_rows + kThreads - 1) / kThreads, 64)), (unsigned)b.n);
  batch_gather_kernel<<<grid, kThreads, 0, s>>>(b, rows_all, row_seq, out_all);
  EC_CHECK_LAUNCH("batch_gather_kernel");
  return EC_OK;
}

ec_status select_decode(const float* H, const int32_t* amax, const float* conf, int n_cand,
                        int32_t* tokens, uint8_t* masked, int32_t* plan, const ec_params& p,
                        StepResult* res, hipStream_t s) {
  select_kernel<<<1, kThreads, 0, s>>>(H, amax, conf, n_cand, tokens, masked, plan, p.seq_len,
                                       p.prompt_len, p.block_len, p.k_recent,
                                       p.candidates == EC_CAND_WINDOW, p.tokens_per_step, res);
  EC_CHECK_LAUNCH("select_kernel");
  return EC_OK;
}

}  // namespace ec
