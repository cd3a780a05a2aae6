// Internal declarations shared by the HIP sources of libec.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <atomic>

#include "ec.h"

namespace ec {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------- direct-to-LDS loads
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}
// buffer resource over [base, base + bytes) (raw buffer, no stride, gfx9 dword3)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from rsrc at voffset + soffset into LDS at lds + 16 * lane
// (buffer_load_dwordx4 ... lds: tracked by vmcnt alone, no staging registers)
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset,
                                                  int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)lds, 16, voffset, soffset, 0, 0);
}

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each with its
// own L2: workgroup pid runs on XCD pid % 8. The remapped id gives each XCD a contiguous
// range of the logical order (XCD x takes ids [x per, (x+1) per) when nblk = 8 per), so
// neighbours in the logical order share an L2.
__device__ __forceinline__ int xcd_remap(int pid, int nblk) {
  const int per = nblk / 8, rem = nblk % 8;
  const int x = pid % 8, local = pid / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + local;
}

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
ec_status hip_fail(hipError_t e, const char* what);

#define EC_CHECK_HIP(call)                                   \
  do {                                                       \
    hipError_t _e = (call);                                  \
    if (_e != hipSuccess) return ::ec::hip_fail(_e, #call);  \
  } while (0)
#define EC_CHECK_LAUNCH(what)                                \
  do {                                                       \
    hipError_t _e = hipGetLastError();                       \
    if (_e != hipSuccess) return ::ec::hip_fail(_e, what);   \
  } while (0)
#define EC_REQUIRE(cond, code, ...)                          \
  do {                                                       \
    if (!(cond)) { ::ec::set_error(__VA_ARGS__); return code; } \
  } while (0)

// Raises a kernel's dynamic LDS limit once per device (the attribute belongs to the
// device the call is made on); safe with several host threads launching at once.
struct LdsLimit {
  std::atomic<uint64_t> done{0};  // bit d: set on device d (devices >= 64 set it on every call)
  ec_status ensure(const void* kern, int bytes) {
    int dev = 0;
    EC_CHECK_HIP(hipGetDevice(&dev));
    const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return EC_OK;
    EC_CHECK_HIP(hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
    done.fetch_or(bit, std::memory_order_release);
    return EC_OK;
  }
};

// ---------------------------------------------------------------- workspace carving
struct Carver {
  char* base;
  size_t off = 0;
  size_t cap;
  Carver(void* b, size_t c) : base((char*)b), cap(c) {}
  template <typename T> T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = (T*)(base ? base + off : nullptr);
    off += n * sizeof(T);
    return p;
  }
};

// ---------------------------------------------------------------- GEMM
// C[M,N] = A[M,K] . B[N,K]^T with fused epilogues.
enum EpiKind { EPI_STORE = 0, EPI_RESID = 1, EPI_QKV = 2, EPI_SWIGLU = 3, EPI_ENTROPY = 4 };

// Partial softmax state of one slice of a row: m = max, z = sum e^(x-m),
// s = sum (x-m) e^(x-m) (natural units), idx = first index of m.
struct EntPart {
  float m, z, s;
  int idx;
  int nan;
  int pad[3];
};

// one pointer per sequence of a batched forward, passed by value in kernel arguments
// (no device table to upload per step)
struct SeqPtrs {
  const void* p[EC_MAX_SEQ];
};

struct EpiArgs {
  int kind;
  void* out;          // STORE: T[M, ldo]; SWIGLU: T[M, ldo]; QKV: q rows T[M, d]
  float* resid;       // RESID: float[M, ldo] updated in place (h += acc)
  // RESID with split K: when norm_out is set, the split-K reduction also writes
  // norm_out[m] = T(RMSNorm(h[m]) * norm_gain) (the next projection's input), and
  // gemm() reports it through *normed
  const void* norm_gain;
  void* norm_out;
  float norm_eps;
  int64_t ldo;
  // QKV: k/v cache rows at positions rows[m]
  void* k_cache;
  void* v_cache;
  const int32_t* rows;
  const float* rope_cos;
  const float* rope_sin;
  int d_model, head_dim;
  int seq_len;        // QKV: rows[m] outside [0, seq_len) are not written
  // ENTROPY: no logits are stored; parts[m * ntiles + tile] gets the partial state
  // of row m over the tile's columns (logits rounded to bf16 first)
  EntPart* parts;
  int ntiles;
  // QKV over rows of several sequences: row m writes its K / V row into the cache of
  // sequence row_seq[m] (k_seq / v_seq hold this layer's cache of each sequence, by
  // value in the kernel arguments); row_seq == nullptr: every row uses k_cache / v_cache
  const int32_t* row_seq;
  SeqPtrs k_seq, v_seq;
};

// K / V destination of row m for the QKV epilogues
template <typename T>
__device__ __forceinline__ T* kv_dst(const EpiArgs& e, int m, bool v) {
  // selects between values held in registers (a select between the two fields'
  // addresses would make the compiler spill them to a private array)
  const uintptr_t kc = (uintptr_t)e.k_cache, vc = (uintptr_t)e.v_cache;
  if (e.row_seq) {
    const int q = e.row_seq[m];
    const uintptr_t kt = (uintptr_t)e.k_seq.p[q], vt = (uintptr_t)e.v_seq.p[q];
    return (T*)(v ? vt : kt);
  }
  return (T*)(v ? vc : kc);
}

size_t gemm_splitk_ws_bytes(int M, int N, int K, int kind, bool bf16);
// column tiles of the bf16 GEMM's plan for M x N x K (the EPI_ENTROPY parts per row)
int gemm_col_tiles(int M, int N, int K, int kind);
// f32: plain weights (QKV [3d, K]; SwiGLU B = gate [N, K], B2 = up [N, K]).
// bf16: packed weights (QKV rotary-interleaved [3d, K]; SwiGLU B = [2N, K] gate/up
// interleave, B2 unused). N is the number of output columns.
ec_status gemm(ec_dtype dt, const void* A, const void* B, const void* B2, int M, int N, int K,
               const EpiArgs& epi, float* splitk_ws, size_t splitk_ws_bytes, hipStream_t s,
               bool* normed = nullptr);
ec_status pack_weights(int elem_bytes, int d, int head_dim, int F, const void* wqkv,
                       const void* w_gate, const void* w_up, void* wqkv_packed,
                       void* gateup_packed, hipStream_t s);

// ---------------------------------------------------------------- attention
// Sequences of one batched attention launch: sequence i owns query rows [row0, row0 + nr)
// of the compact q / out arrays and attends over its own cache k, v (all L rows).
struct AttnSeq {
  int row0, nr;
  const void* k;
  const void* v;
};
struct AttnSeqs {
  AttnSeq s[EC_MAX_SEQ];
  int n;
};
size_t attn_ws_bytes(int r, int L, int H, int D);
// bf16 launch plan of one sequence's attention: queries per workgroup and key splits
void attn_plan_query(int r, int L, int H, int* query_tile, int* splits);
ec_status attn(ec_dtype dt, const void* q, const void* k, const void* v, int r, int L, int H, int D,
               float scale, void* out, void* ws, size_t ws_bytes, hipStream_t s);
// every sequence's rows in one launch (plus one merge launch when the keys are split)
ec_status attn_batch(ec_dtype dt, const void* q, const AttnSeqs& seqs, int L, int H, int D, float scale, void* out,
                     void* ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- entropy
size_t entropy_ws_bytes(int rows, int vocab);
// merge parts[rows][splits] (the fused LM-head epilogue's states) in order into entropy /
// argmax / confidence
ec_status entropy_merge(const EntPart* parts, int rows, int splits, float* H, int32_t* amax, float* c,
                        hipStream_t s);
// ec_entropy_max_noalloc: the same reduction with its scratch in the library's device array
constexpr size_t kEntropyScratchBytes = (size_t)1 << 20;
ec_status entropy_noalloc(ec_dtype dt, const void* logits, int rows, int vocab, int64_t stride, const int32_t* sel,
                          int n_sel, float* H, int32_t* amax, float* c, float* emax, hipStream_t s);
ec_status entropy(ec_dtype dt, const void* logits, int rows, int vocab, int64_t stride,
                  const int32_t* sel, int n_sel, float* H, int32_t* amax, float* c, float* emax,
                  void* ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- elementwise
// h[i] = table[tokens[rows[i]]]; with row_seq, the token array of row i is tok.p[row_seq[i]]
ec_status embed(ec_dtype dt, const void* table, int vocab, const int32_t* tokens, int L,
                const int32_t* rows, int n, int d, float* h, hipStream_t s,
                const SeqPtrs* tok = nullptr, const int32_t* row_seq = nullptr);
ec_status rmsnorm(ec_dtype dt, const float* h, int n_src, const int32_t* idx, int n, int d,
                  const void* gain, float eps, void* out, hipStream_t s);
// h[m] += sum_s part[s][m] (s ascending), then out[m] = T(RMSNorm(h[m]) * gain), m < M: the
// split-K reduction of a residual projection fused with the next RMSNorm. It performs the
// float operations of the split-K residual epilogue followed by rmsnorm(), in their order.
ec_status resid_norm(ec_dtype dt, const float* part, int S, int M, int d, float* h, const void* gain,
                     float eps, void* out, hipStream_t s);
// ao[i] = a[idx[i]] and bo[i] = b[idx[i]] for i < n (rows of a_row_bytes / b_row_bytes,
// multiples of 16, 16-byte aligned buffers), one launch
ec_status gather_rows2(const int32_t* idx, int n, const void* a, void* ao, size_t a_row_bytes, const void* b,
                       void* bo, size_t b_row_bytes, hipStream_t s);
ec_status scatter(ec_dtype dt, void* kc, void* vc, int64_t L, int width, const void* kr,
                  const void* vr, const int32_t* idx, int n, hipStream_t s);

// ---------------------------------------------------------------- KV-drift probe
// old K / V rows of `rows` before a layer's QKV GEMM; per-row cosine distances after
// it (dist[c * n + i], c = 0 K, 1 V); per layer mean / max over valid rows into
// out[4 l + 2 c + {0, 1}] (dist of layer l at dist + l * layer_stride)
ec_status drift_gather(ec_dtype dt, const void* kc, const void* vc, const int32_t* rows, int n, int L, int d,
                       void* ok, void* ov, hipStream_t s);
ec_status drift_rows(ec_dtype dt, const void* ok, const void* ov, const void* kc, const void* vc,
                     const int32_t* rows, int n, int L, int d, float* dist, hipStream_t s);
ec_status drift_reduce(const float* dist, int n_layers, int n, int64_t layer_stride, float* out, hipStream_t s);

// ---------------------------------------------------------------- batch of sequences
// per-sequence segments of the concatenated row / candidate lists of ec_step_batch
struct BatchSeg {
  const int32_t* rows;  // positions recomputed (device, in the sequence's plan)
  const int32_t* cidx;  // candidate indices into rows (device)
  int n_rows, row_off, n_cand, cand_off, seq;
};
struct BatchSegs {
  BatchSeg seg[EC_MAX_SEQ];
  int n;
};
// rows_all[row_off + i] = rows[i], row_seq[...] = seq; out_all[cand_off + j] = row_off + cidx[j]
ec_status batch_gather(const BatchSegs& b, int max_rows, int32_t* rows_all, int32_t* row_seq,
                       int32_t* out_all, hipStream_t s);

// ---------------------------------------------------------------- decode / plan
// plan buffer layout (int32 words), L = seq_len, k = k_recent (ring size max(k,1)):
//   [0]            ring count (decoded so far)
//   [1]            rows in the recompute list R
//   [2]            candidates
//   [3]            masked positions left
//   [8 .. 8+K)     ring of decoded positions (K = max(k,1))
//   [R0 .. R0+L)   R (ascending positions), R0 = 8 + K
//   [C0 .. C0+L)   candidate positions (ascending)
//   [I0 .. I0+L)   candidate indices into R
//   [J0 .. J0+L)   iota 0..L-1 (rows of a full forward)
//   [RES ..)       StepResult record of the last reset / step
struct StepResult;
struct PlanLayout {
  int K, R0, C0, I0, J0, RES, words;
  __host__ __device__ inline PlanLayout(int L, int k);
};

// device result of one step, copied to the host once per step
struct StepResult {
  int32_t n_picked;
  int32_t has_nan;
  float emax;
  int32_t next_rows;
  int32_t next_cand;
  int32_t n_masked;
  int32_t pad[2];
  int32_t pos[EC_MAX_TOKENS_PER_STEP];
  int32_t ids[EC_MAX_TOKENS_PER_STEP];
  float ent[EC_MAX_TOKENS_PER_STEP];
  float conf[EC_MAX_TOKENS_PER_STEP];
};

__host__ __device__ inline PlanLayout::PlanLayout(int L, int k) {
  K = k > 0 ? k : 1;
  R0 = 8 + K;
  C0 = R0 + L;
  I0 = C0 + L;
  J0 = I0 + L;
  RES = J0 + L;
  words = RES + (int)(sizeof(StepResult) / sizeof(int32_t));
}

ec_status plan_reset(int32_t* tokens, uint8_t* masked, int32_t* plan, const ec_params& p,
                     StepResult* res, hipStream_t s);
ec_status select_decode(const float* H, const int32_t* amax, const float* conf, int n_cand,
                        int32_t* tokens, uint8_t* masked, int32_t* plan, const ec_params& p,
                        StepResult* res, hipStream_t s);

ec_status rope_table(float* c, float* sn, int max_pos, int head_dim, double base, hipStream_t s);

}  // namespace ec
