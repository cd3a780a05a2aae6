/*
 * ec.h -- EntropyCache denoising step for bidirectional diffusion LMs on
 * AMD Instinct MI355X (gfx950). C ABI of libec.so.
 *
 * The method (EntropyCache explainer pages for paper 2603.18489: Italian
 * summary "Algoritmo di Funzionamento"; Arabic technical summary, section 2
 * "Algorithm workflow" and its E_{t+1} equation): at every denoising step,
 * decode new tokens, take E_{t+1} = the largest softmax entropy (nats) among
 * the newly decoded tokens' distributions, and compare it with a threshold
 * tau. E > tau makes the next step a full forward that rewrites every
 * layer's K/V cache (refresh); E <= tau makes it a partial forward that
 * recomputes only the still-masked positions plus the k most recently
 * decoded positions and reuses the cached K/V of every other position.
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the comment says "host".
 *  - Matrices are row-major. Projection weights are stored [out, in], so a
 *    projection computes y = x W^T.
 *  - All tensors of one model (weights, K/V cache, q/k/v rows, logits) share
 *    one storage dtype (ec_dtype). Every dot product, softmax, norm and
 *    entropy accumulates in fp32; the residual stream is fp32.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Calls enqueue work on it and return without waiting, except ec_step,
 *    which waits once per step for the decision (see there).
 *  - The caller owns and frees every buffer (weights, cache, state,
 *    workspace). The library allocates no device memory and keeps no pointer
 *    after a call returns; buffers must stay alive until the stream has run
 *    the enqueued work.
 *  - Calls return an ec_status and never throw. Argument errors are found
 *    before anything is enqueued (nothing runs). A failed HIP call returns
 *    EC_ERR_HIP; ec_last_error() gives the message of the calling thread's
 *    last failure.
 */
#ifndef EC_H_
#define EC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EC_VERSION 10200            /* 1.2.0: timing group EC_T_LAST, last layer over the output rows */
#define EC_MAX_TOKENS_PER_STEP 64   /* upper bound on tokens decoded per step */
#define EC_MAX_LAYERS 256
#define EC_MAX_SEQ 16               /* upper bound on sequences per ec_step_batch call */

typedef enum ec_status {
  EC_OK = 0,
  EC_ERR_ARG = 1,         /* null pointer, negative or inconsistent size */
  EC_ERR_DTYPE = 2,       /* dtype not EC_F32 / EC_BF16 */
  EC_ERR_WORKSPACE = 3,   /* workspace null or smaller than the *_workspace_size query */
  EC_ERR_HIP = 4,         /* a HIP runtime call failed */
  EC_ERR_NAN = 5,         /* ec_step: E was NaN; the next step is forced to refresh */
  EC_ERR_UNSUPPORTED = 6  /* shape the kernels do not support (see each call) */
} ec_status;

typedef enum ec_dtype { EC_F32 = 0, EC_BF16 = 1 } ec_dtype;

/* ------------------------------------------------------------------------
 * ec_entropy_max -- fused softmax entropy / argmax / confidence reduction.
 *
 * For each row i of `logits` (x_i0 .. x_i,V-1), with m = max_j x_ij,
 * Z = sum_j exp(x_ij - m), S = sum_j (x_ij - m) exp(x_ij - m):
 *   entropy[i] = ln Z - S / Z   (= -sum_j p_ij ln p_ij, nats)
 *   argmax[i]  = lowest j with x_ij = m
 *   maxprob[i] = 1 / Z          (= max_j p_ij)
 *   *emax      = max of entropy[] over the rows listed in sel[0..n_sel)
 *                (all rows when sel is NULL); NaN if any of them is NaN.
 * This is the decision signal E_{t+1} of the pages (Arabic technical summary,
 * section 2, "Decode and evaluate entropy" equation); its cost is O(V) per
 * row and independent of sequence length and depth.
 *
 * logits:   [rows, row_stride] of dtype, only the first `vocab` of each row
 *           are read. -inf entries contribute nothing; a NaN entry makes the
 *           row's entropy and maxprob NaN.
 * entropy, maxprob: float[rows]; argmax: int32[rows]; emax: float[1] or NULL.
 * workspace: >= ec_entropy_max_workspace_size(rows, vocab) bytes.
 * Errors: EC_ERR_ARG for rows < 0, vocab < 1, row_stride < vocab, null
 * outputs; rows == 0 enqueues nothing except *emax = -inf.
 * ---------------------------------------------------------------------- */
size_t ec_entropy_max_workspace_size(int32_t rows, int32_t vocab);
ec_status ec_entropy_max(const void* logits, ec_dtype dtype, int32_t rows, int32_t vocab,
                         int64_t row_stride, const int32_t* sel, int32_t n_sel,
                         float* entropy, int32_t* argmax, float* maxprob, float* emax,
                         void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * ec_entropy_max_noalloc -- ec_entropy_max for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments and results as ec_entropy_max
 * (bit-identical outputs), without the workspace: the reduction's scratch lives in a
 * device array of the library, EC_ENTROPY_NOALLOC_SCRATCH_BYTES per GPU, held until the
 * process ends. The call allocates nothing. Every call on one GPU shares that GPU's
 * array (each word a call uses is left cleared for the next call): calls on one GPU
 * must be ordered (one stream, or streams with events between them); calls that overlap
 * in time on one GPU race.
 * Errors: as ec_entropy_max; EC_ERR_UNSUPPORTED (nothing enqueued) when
 * ec_entropy_max_workspace_size(rows, vocab) exceeds EC_ENTROPY_NOALLOC_SCRATCH_BYTES
 * (about 26000 rows at any vocabulary up to 2^31).
 * ---------------------------------------------------------------------- */
#define EC_ENTROPY_NOALLOC_SCRATCH_BYTES (1u << 20)
ec_status ec_entropy_max_noalloc(const void* logits, ec_dtype dtype, int32_t rows, int32_t vocab,
                                 int64_t row_stride, const int32_t* sel, int32_t n_sel, float* entropy,
                                 int32_t* argmax, float* maxprob, float* emax, void* stream);

/* ------------------------------------------------------------------------
 * ec_cache_scatter -- write recomputed K/V rows into one layer's cache.
 *
 * k_cache[idx[i], :] = k_rows[i, :] and v_cache[idx[i], :] = v_rows[i, :]
 * for i < n_rows; every other cache row is untouched. This is the partial
 * forward's cache update: only the recomputed positions get fresh K/V, all
 * other positions keep their cached K/V (Arabic technical summary, section 2,
 * phase 1).
 *
 * k_cache, v_cache: [seq_len, width]; k_rows, v_rows: [n_rows, width], all of
 * dtype; idx: int32[n_rows], distinct positions. A row whose idx is outside
 * [0, seq_len) is skipped (not written). Duplicate positions: unspecified
 * which row lands. Errors: EC_ERR_ARG for null pointers or sizes < 0.
 * ---------------------------------------------------------------------- */
ec_status ec_cache_scatter(void* k_cache, void* v_cache, int64_t seq_len, int32_t width,
                           ec_dtype dtype, const void* k_rows, const void* v_rows,
                           const int32_t* idx, int32_t n_rows, void* stream);

/* ------------------------------------------------------------------------
 * ec_partial_attn -- bidirectional attention of r query rows over all L rows
 * of one layer's K/V cache (no mask: every position attends to every other,
 * Italian summary section 1).
 *
 * out[i, h, :] = softmax_j(q[i,h,:] . k_cache[j,h,:] * scale) @ v_cache[:,h,:]
 * q, out: [r, n_heads * head_dim]; k_cache, v_cache: [seq_len, n_heads *
 * head_dim]; all of dtype; scale > 0. bf16 runs on MFMA with fp32 softmax: with
 * t_j = q . k_j * scale * log2(e) and M an integer >= max_j t_j, the weights
 * w_j = 2^(t_j - M) enter the P.V product rounded to bf16 and the row sum
 * unrounded, out = sum_j bf16(w_j) v_j / sum_j w_j (bf16 rounding commutes with
 * powers of two, so the result does not depend on M).
 * Supported: head_dim == 128 for bf16, with max(r, seq_len) * n_heads * 256
 * bytes below 2 GiB (32-bit buffer offsets). f32: head_dim 32, 64 or 128 with
 * 16-byte aligned q, caches and out runs on the matrix unit at any seq_len;
 * otherwise head_dim <= 1024 with (seq_len + head_dim) * 4 <= 65536.
 * EC_ERR_UNSUPPORTED otherwise.
 * workspace: >= ec_partial_attn_workspace_size(...) bytes (may be 0 -> NULL ok).
 * ---------------------------------------------------------------------- */
size_t ec_partial_attn_workspace_size(int32_t r, int32_t seq_len, int32_t n_heads,
                                      int32_t head_dim);
ec_status ec_partial_attn(const void* q, const void* k_cache, const void* v_cache, int32_t r,
                          int32_t seq_len, int32_t n_heads, int32_t head_dim, float scale,
                          ec_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ec_partial_attn_plan -- the launch plan of the bf16 path of ec_partial_attn (the
 * attention above, Italian summary section 1) for these sizes (host only, no device
 * work): *query_tile = queries per workgroup
 * (64 for the skip-step shape, 128 for the refresh-sized one), *splits = key-range
 * splits merged after the launch (1 = none). Workgroups = ceil(r / query_tile) *
 * n_heads * splits. For diagnostics and tests; ec_partial_attn takes the same plan
 * with its workspace at least ec_partial_attn_workspace_size(...) bytes.
 * Errors: EC_ERR_ARG for null outputs or sizes < 1, EC_ERR_UNSUPPORTED for
 * head_dim != 128. */
ec_status ec_partial_attn_plan(int32_t r, int32_t seq_len, int32_t n_heads, int32_t head_dim,
                               int32_t* query_tile, int32_t* splits);

/* ------------------------------------------------------------------------
 * Model, cache and decoding descriptors (plain structs; struct_size must be
 * set to sizeof(the struct) by the caller).
 *
 * Architecture (not given on the pages; the reading taken): pre-norm blocks
 * with RMSNorm (gain, eps), fused QKV projection, rotary embedding on q and
 * k (pairs (i, i + head_dim/2), angle pos * base^(-2i/head_dim)), softmax
 * attention scaled by 1/sqrt(head_dim), output projection + residual,
 * RMSNorm, SwiGLU MLP (silu(gate) * up, then down) + residual; final RMSNorm
 * and an untied LM head. Logits of position p come from row p.
 * ---------------------------------------------------------------------- */
/* Weight layout of the QKV and gate/up matrices.
 * EC_LAYOUT_PLAIN  (fp32 models): wqkv [3d, d] with rows [0,d) q, [d,2d) k,
 *   [2d,3d) v in natural order; w_gate and w_up [F, d].
 * EC_LAYOUT_PACKED (bf16 models): the layout the MFMA kernels read, built from
 *   the plain one by ec_pack_weights. wqkv keeps [3d, d] but inside each head's
 *   head_dim rows, group g of 32 rows holds rows 16g .. 16g+15 followed by their
 *   rotary partners head_dim/2 + 16g .. head_dim/2 + 16g + 15. w_gate points at
 *   a [2F, d] matrix whose group g of 32 rows holds gate rows 16g .. 16g+15
 *   followed by up rows 16g .. 16g+15; w_up is unused (may be NULL).
 * The math is unchanged: the packed matrices hold the same rows, reordered. */
typedef enum ec_weight_layout { EC_LAYOUT_PLAIN = 0, EC_LAYOUT_PACKED = 1 } ec_weight_layout;

typedef struct ec_layer_weights {
  const void* attn_norm; /* [d] */
  const void* wqkv;      /* [3d, d]: q | k | v rows (packed order for EC_LAYOUT_PACKED) */
  const void* wo;        /* [d, d] */
  const void* mlp_norm;  /* [d] */
  const void* w_gate;    /* PLAIN: [F, d] gate; PACKED: [2F, d] gate/up interleave */
  const void* w_up;      /* PLAIN: [F, d] up; PACKED: unused */
  const void* w_down;    /* [d, F] */
} ec_layer_weights;

/* Every device array of the model and of the cache must be 16-byte aligned (hipMalloc
 * returns 256-byte aligned memory); ec_forward / ec_step return EC_ERR_ARG otherwise.
 * bf16 models run on kernels that address weights, activations and caches through
 * 32-bit byte offsets, and need: head_dim 128; d a multiple of 256; F and V multiples
 * of 128; every weight matrix (V x d, 3d x d, 2F x d) below 2 GiB; seq_len * max(d, F)
 * * 2 bytes below 2 GiB (n_seq times that for ec_step_batch). The calls and their
 * workspace queries return EC_ERR_UNSUPPORTED (size 0) otherwise, before any work. */
typedef struct ec_model_desc {
  uint32_t struct_size;
  ec_dtype dtype;
  int32_t n_layers, d_model, n_heads, head_dim, ffn_dim, vocab;
  float rms_eps;
  const void* embed;               /* [V, d] */
  const ec_layer_weights* layers;  /* HOST array of n_layers entries */
  const void* final_norm;          /* [d] */
  const void* lm_head;             /* [V, d] */
  const float* rope_cos;           /* [rope_max_pos, head_dim/2] fp32, from ec_rope_table */
  const float* rope_sin;           /* same shape */
  int32_t rope_max_pos;            /* >= seq_len */
  int32_t weight_layout;           /* ec_weight_layout: PACKED for bf16, PLAIN for fp32 */
} ec_model_desc;

/* ec_pack_weights -- build the EC_LAYOUT_PACKED matrices of one layer from the
 * plain ones (device to device, out of place, enqueued on `stream`).
 * wqkv [3d, d] -> wqkv_packed [3d, d]; w_gate, w_up [F, d] -> gateup_packed
 * [2F, d]. Either output may be NULL to skip it (its inputs are then ignored).
 * Needs head_dim % 32 == 0 and d % head_dim == 0 for wqkv, F % 16 == 0 for gate/up.
 * Errors: EC_ERR_DTYPE, EC_ERR_ARG (null input of a requested output, bad sizes). */
ec_status ec_pack_weights(ec_dtype dtype, int32_t d_model, int32_t head_dim, int32_t ffn_dim,
                          const void* wqkv, const void* w_gate, const void* w_up,
                          void* wqkv_packed, void* gateup_packed, void* stream);

typedef struct ec_cache_desc {
  uint32_t struct_size;
  int32_t seq_len;        /* L */
  void* const* k;         /* HOST array of n_layers device pointers, each [L, d] */
  void* const* v;         /* same */
} ec_cache_desc;

/* ec_rope_table -- fill cos/sin tables [max_pos, head_dim/2] (fp32) with
 * cos/sin(pos * base^(-2i/head_dim)), evaluated in fp64 on the device. */
ec_status ec_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                        double base, void* stream);

/* ------------------------------------------------------------------------
 * ec_forward -- forward pass over the positions rows[0..n_rows) against the
 * per-layer cache (the partial forward of a skip step; with rows = every
 * position 0..L-1 it is the full forward of a refresh step).
 *
 * Per layer, K/V of the listed rows are computed (RoPE at their absolute
 * positions) and written into the cache at those positions before the
 * queries of the same rows attend over all L cached rows; rows not listed
 * keep (and are read with) whatever the cache holds.
 * tokens: int32[L]; rows: int32[n_rows], distinct positions in [0, L);
 * out_idx: int32[n_out], indices INTO rows whose logits are produced;
 * logits: [n_out, V] of dtype; hidden: NULL or float[n_rows, d] receiving the
 * residual stream after the last layer.
 * The logits need the last layer's output only at the out_idx rows: with hidden
 * == NULL and n_out < n_rows, the last layer writes K/V of every row but runs
 * its attention, O-projection and MLP over the out_idx rows alone (ec_step and
 * ec_step_batch always take this path). The logits are those of the whole
 * forward up to the summation order of the smaller launches.
 * Supported: bf16 needs head_dim == 128, d % 256 == 0, F % 128 == 0,
 * V % 256 == 0; f32 any even head_dim <= 256.
 * ---------------------------------------------------------------------- */
size_t ec_forward_workspace_size(const ec_model_desc* model, int32_t max_rows, int32_t max_out,
                                 int32_t seq_len);
ec_status ec_forward(const ec_model_desc* model, const ec_cache_desc* cache,
                     const int32_t* tokens, const int32_t* rows, int32_t n_rows,
                     const int32_t* out_idx, int32_t n_out, void* logits, float* hidden,
                     void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Denoising state and ec_step.
 * ---------------------------------------------------------------------- */
/* Candidates of a step (the pages note the entropy-guided skipping applies to
 * different decoding strategies, sliding windows and blocks among them; EntropyCache
 * explainer, Italian summary, section 5):
 * EC_CAND_BLOCKS: the masked positions of the lowest block [P + bB, P + (b+1)B) that
 *   still has a masked position (semi-autoregressive blocks of length B);
 * EC_CAND_WINDOW: the masked positions among the B positions starting at the lowest
 *   masked position (a window that slides as soon as its first position is decoded). */
typedef enum ec_candidates { EC_CAND_BLOCKS = 0, EC_CAND_WINDOW = 1 } ec_candidates;

typedef struct ec_params {
  uint32_t struct_size;
  float tau;               /* threshold in nats; E > tau -> refresh next step */
  int32_t k_recent;        /* k: most recently decoded positions recomputed on skip steps */
  int32_t tokens_per_step; /* n: tokens decoded per step, 1..EC_MAX_TOKENS_PER_STEP */
  int32_t block_len;       /* B: candidates = masked positions of the lowest open block */
  int32_t prompt_len;      /* P */
  int32_t seq_len;         /* L = P + masked positions */
  int32_t mask_id;         /* token id written at masked positions */
  int32_t candidates;      /* ec_candidates: which masked positions may be decoded */
} ec_params;

typedef struct ec_state {
  uint32_t struct_size;
  int32_t* tokens;     /* device int32[L]: prompt ids, decoded ids, mask_id elsewhere */
  uint8_t* masked;     /* device uint8[L]: 1 = still masked */
  int32_t* plan;       /* device int32[ec_state_plan_words(L, k)]: decode-time ring of
                          the last k decoded positions, recompute and candidate lists */
  int32_t t;           /* host: steps done */
  int32_t refresh_next;/* host: 1 -> next step is a full forward (set 1 to force) */
  int32_t n_masked;    /* host: positions still masked */
  int32_t n_decoded;   /* host: positions decoded so far */
  int32_t next_rows;   /* host: rows the next skip step recomputes */
  int32_t next_cand;   /* host: candidates of the next step */
} ec_state;

typedef struct ec_step_out {
  uint32_t struct_size;
  int32_t status;        /* EC_OK or EC_ERR_NAN */
  int32_t refreshed;     /* 1 if this step ran the full forward */
  int32_t rows;          /* positions recomputed this step (L on a refresh) */
  int32_t n_cand;        /* candidates this step */
  int32_t n_decoded;     /* tokens decoded this step */
  int32_t refresh_next;  /* E > tau (or E NaN) */
  float emax;            /* E_{t+1}: max entropy over the tokens decoded this step */
  int32_t positions[EC_MAX_TOKENS_PER_STEP]; /* decoded positions, ascending */
  int32_t ids[EC_MAX_TOKENS_PER_STEP];       /* decoded token ids */
  float entropy[EC_MAX_TOKENS_PER_STEP];     /* their entropies (nats) */
  float maxprob[EC_MAX_TOKENS_PER_STEP];     /* their confidences */
} ec_step_out;

/* Words of device int32 storage that ec_state.plan needs. */
size_t ec_state_plan_words(int32_t seq_len, int32_t k_recent);

/* ec_state_reset -- start a new sequence: tokens[0..P) must already hold the
 * prompt; sets tokens[P..L) = mask_id, masked = (pos >= P), clears the
 * decode ring, builds the first plan, and sets the host fields (t = 0,
 * refresh_next = 1, n_masked = L - P, n_decoded = 0, next_*). Synchronizes
 * the stream once. */
ec_status ec_state_reset(ec_state* state, const ec_params* params, void* stream);

/* ec_step -- one denoising step (Arabic technical summary, section 2: forward,
 * decode and evaluate entropy, skip decision and recent-token selection).
 *   1. t == 0 or refresh_next: full forward over all L rows; otherwise a
 *      partial forward over R = still-masked positions plus the last k
 *      decoded positions (the decode-time ring), ascending.
 *   2. Candidates = masked positions of the lowest block
 *      [P + bB, P + (b+1)B) that still has a mask; their logits go through
 *      the entropy/argmax/confidence reduction.
 *   3. The min(n, #candidates) candidates with the largest confidence (ties:
 *      lower position) are decoded with their argmax ids, in ascending
 *      position order, and appended to the decode ring.
 *   4. E = max entropy of the decoded rows; refresh_next = E > tau (strict),
 *      or E is NaN (then out->status = EC_ERR_NAN and the call returns it).
 * The host reads E and the decoded ids once per step (one stream sync),
 * because E selects the next step's path. A state with no masked position
 * left returns EC_OK with n_decoded = 0 and enqueues nothing.
 * out: HOST pointer. workspace: >= ec_step_workspace_size(model, params).
 * ---------------------------------------------------------------------- */
size_t ec_step_workspace_size(const ec_model_desc* model, const ec_params* params);
ec_status ec_step(const ec_model_desc* model, const ec_cache_desc* cache, ec_state* state,
                  const ec_params* params, void* workspace, size_t workspace_bytes,
                  void* stream, ec_step_out* out);

/* ec_step_probe -- ec_step plus the KV-drift probe (the pages' drift measure: the
 * cosine distance of cached vs freshly computed value vectors between consecutive
 * steps, which they report tracks the previous step's E; EntropyCache explainer,
 * Arabic technical summary, section 2, key observations). For every row the step
 * recomputes (all L on a refresh) and every layer, dist = 1 - <old, new> / (|old| |new|)
 * between the K (and the V) the cache held before the step and the one the step
 * writes; drift (device float[4 * n_layers]) receives per layer l:
 *   drift[4l] = mean K distance, drift[4l+1] = max K distance,
 *   drift[4l+2] = mean V distance, drift[4l+3] = max V distance,
 * over the rows whose old and new vectors are both non-zero (NaN if none: the
 * first step of a zero-filled cache). Same workspace as ec_step (ec_step_workspace_size
 * covers the probe's buffers); otherwise identical to ec_step. */
ec_status ec_step_probe(const ec_model_desc* model, const ec_cache_desc* cache, ec_state* state,
                        const ec_params* params, void* workspace, size_t workspace_bytes, void* stream,
                        ec_step_out* out, float* drift);

/* ec_step_batch -- one denoising step of n_seq independent sequences of the same
 * model with the same params (every field but the state and cache is shared),
 * decided per sequence exactly as ec_step decides it: sequence s refreshes when
 * its own t == 0 or its refresh_next is set, otherwise it recomputes its own
 * recompute set, and it reads its own E. All sequences' rows go through one
 * forward (one launch per GEMM over the concatenated rows, so every weight is
 * read once per step for the whole batch; attention runs per sequence against
 * that sequence's cache); one LM head over all candidates with the entropy
 * reduction fused for bf16; selection per sequence.
 * (EntropyCache explainer, Arabic technical summary, section 2, with the
 * decision taken per sequence; the batching itself is not on the pages.)
 * caches, states, outs: HOST arrays of n_seq entries (1 <= n_seq <= EC_MAX_SEQ);
 * a sequence with no masked position left is not stepped (its out has
 * n_decoded = 0). Synchronises `stream` once. Returns EC_ERR_NAN if any
 * sequence's E is NaN (that sequence's out->status says which). */
size_t ec_step_batch_workspace_size(const ec_model_desc* model, int32_t n_seq, const ec_params* params);
ec_status ec_step_batch(const ec_model_desc* model, int32_t n_seq, const ec_cache_desc* caches,
                        ec_state* states, const ec_params* params, void* workspace,
                        size_t workspace_bytes, void* stream, ec_step_out* outs);

/* ------------------------------------------------------------------------
 * Measurement aid: per-kernel-group timing with HIP events.
 *
 * While enabled, ec_forward and ec_step bracket each kernel group with a pair
 * of hipEvents recorded on the caller's stream and accumulate, per group, the
 * elapsed time, the number of launches and the algorithmic work of those
 * launches (flops of the contraction, bytes the method must move). Process-
 * wide state, for one thread at a time; it costs two event records per
 * timed group launch. ec_timing_select restricts the recording to the groups
 * whose bit (1 << EC_T_*) is set in `kinds` (all groups by default), so that a
 * single group can be timed inside a throughput run at the cost of two event
 * records per launch of that group. ec_timing_read synchronizes the recorded
 * events, fills `out` and optionally clears the totals.
 * ---------------------------------------------------------------------- */
enum {
  EC_T_EMBED = 0, EC_T_NORM, EC_T_QKV, EC_T_ATTN, EC_T_OPROJ, EC_T_GATEUP, EC_T_DOWN,
  EC_T_LMHEAD, EC_T_ENTROPY, EC_T_SELECT,
  EC_T_LAST,  /* last layer past its QKV projection, over the output rows only (see ec_forward) */
  EC_T_KINDS
};
typedef struct ec_timing {
  uint32_t struct_size;
  int32_t n_kinds;
  double ms[EC_T_KINDS];        /* summed event time per group */
  int64_t launches[EC_T_KINDS]; /* number of timed launches per group */
  double flops[EC_T_KINDS];     /* algorithmic flops (2*M*N*K for a GEMM) */
  double bytes[EC_T_KINDS];     /* algorithmic bytes (weights + activations read / written) */
} ec_timing;
ec_status ec_timing_enable(int on);
ec_status ec_timing_select(uint32_t kinds);
ec_status ec_timing_read(ec_timing* out, int reset);

/* Message of the calling thread's last failed call ("" if none). */
const char* ec_last_error(void);
int ec_version(void);

#ifdef __cplusplus
}
#endif
#endif /* EC_H_ */
