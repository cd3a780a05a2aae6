// C ABI of libec.so: argument checks, workspace planning, and the per-step
// orchestration of the EntropyCache denoising step (include/ec.h).
#include "ec_internal.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <vector>

namespace ec {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

ec_status hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return EC_ERR_HIP;
}

namespace {

// ---------------------------------------------------------------- timing aid
struct TimingState {
  bool on = false;
  uint32_t mask = ~0u;  // groups recorded while on
  std::vector<hipEvent_t> ev;  // pairs: 2*i start, 2*i+1 stop
  struct Rec {
    int kind, slot;
    double flops, bytes;
  };
  std::vector<Rec> pending;
  int used = 0;
  double ms[EC_T_KINDS] = {}, flops[EC_T_KINDS] = {}, bytes[EC_T_KINDS] = {};
  int64_t launches[EC_T_KINDS] = {};
};
TimingState g_tm;

struct TScope {
  int kind, slot = -1;
  hipStream_t s;
  double fl, by;
  TScope(int k, hipStream_t st, double f, double b) : kind(k), s(st), fl(f), by(b) {
    if (!g_tm.on || !((g_tm.mask >> k) & 1u)) return;
    if ((int)g_tm.ev.size() < 2 * (g_tm.used + 1)) {
      hipEvent_t a, z;
      if (hipEventCreate(&a) != hipSuccess) return;
      if (hipEventCreate(&z) != hipSuccess) return;
      g_tm.ev.push_back(a);
      g_tm.ev.push_back(z);
    }
    slot = g_tm.used++;
    hipEventRecord(g_tm.ev[2 * slot], s);
  }
  ~TScope() {
    if (slot < 0) return;
    hipEventRecord(g_tm.ev[2 * slot + 1], s);
    g_tm.pending.push_back({kind, slot, fl, by});
  }
};

void timing_collect() {
  for (const auto& r : g_tm.pending) {
    float ms = 0.f;
    hipEventSynchronize(g_tm.ev[2 * r.slot + 1]);
    if (hipEventElapsedTime(&ms, g_tm.ev[2 * r.slot], g_tm.ev[2 * r.slot + 1]) == hipSuccess) {
      g_tm.ms[r.kind] += ms;
      g_tm.launches[r.kind] += 1;
      g_tm.flops[r.kind] += r.flops;
      g_tm.bytes[r.kind] += r.bytes;
    }
  }
  g_tm.pending.clear();
  g_tm.used = 0;
}

size_t esize(ec_dtype dt) { return dt == EC_BF16 ? 2 : 4; }
bool dtype_ok(ec_dtype dt) { return dt == EC_F32 || dt == EC_BF16; }

ec_status check_model(const ec_model_desc* m) {
  EC_REQUIRE(m && m->struct_size >= sizeof(ec_model_desc), EC_ERR_ARG, "model: null or struct_size too small");
  EC_REQUIRE(dtype_ok(m->dtype), EC_ERR_DTYPE, "model: bad dtype %d", (int)m->dtype);
  EC_REQUIRE(m->n_layers >= 1 && m->n_layers <= EC_MAX_LAYERS, EC_ERR_ARG, "model: n_layers %d", m->n_layers);
  EC_REQUIRE(m->d_model > 0 && m->n_heads > 0 && m->head_dim > 0 && m->ffn_dim > 0 && m->vocab > 0,
             EC_ERR_ARG, "model: non-positive dimension");
  EC_REQUIRE(m->n_heads * m->head_dim == m->d_model, EC_ERR_ARG, "model: n_heads*head_dim != d_model");
  EC_REQUIRE(m->head_dim % 2 == 0, EC_ERR_ARG, "model: head_dim must be even");
  EC_REQUIRE(m->embed && m->layers && m->final_norm && m->lm_head && m->rope_cos && m->rope_sin,
             EC_ERR_ARG, "model: null pointer");
  const bool packed = m->dtype == EC_BF16;
  EC_REQUIRE(m->weight_layout == (packed ? EC_LAYOUT_PACKED : EC_LAYOUT_PLAIN), EC_ERR_ARG,
             "model: weight_layout must be %s for %s models (see ec_pack_weights)",
             packed ? "EC_LAYOUT_PACKED" : "EC_LAYOUT_PLAIN", packed ? "bf16" : "fp32");
  auto a16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
  EC_REQUIRE(a16(m->embed) && a16(m->final_norm) && a16(m->lm_head) && a16(m->rope_cos) && a16(m->rope_sin),
             EC_ERR_ARG, "model: device arrays must be 16-byte aligned");
  for (int l = 0; l < m->n_layers; ++l) {
    const ec_layer_weights& w = m->layers[l];
    EC_REQUIRE(w.attn_norm && w.wqkv && w.wo && w.mlp_norm && w.w_gate && (packed || w.w_up) && w.w_down,
               EC_ERR_ARG, "model: null weight in layer %d", l);
    EC_REQUIRE(a16(w.attn_norm) && a16(w.wqkv) && a16(w.wo) && a16(w.mlp_norm) && a16(w.w_gate) &&
                   a16(w.w_up) && a16(w.w_down),
               EC_ERR_ARG, "model: weights of layer %d must be 16-byte aligned", l);
  }
  if (m->dtype == EC_BF16) {
    EC_REQUIRE(m->head_dim == 128, EC_ERR_UNSUPPORTED, "bf16 model: head_dim must be 128");
    EC_REQUIRE(m->d_model % 256 == 0 && m->ffn_dim % 128 == 0 && m->vocab % 128 == 0,
               EC_ERR_UNSUPPORTED, "bf16 model: need d %% 256, F %% 128, V %% 128 == 0");
    EC_REQUIRE(m->d_model % 64 == 0 && m->ffn_dim % 64 == 0, EC_ERR_UNSUPPORTED,
               "bf16 model: d and F must be multiples of 64");
    // the bf16 kernels address every weight matrix through 32-bit byte offsets
    const int64_t widest = std::max<int64_t>({3 * (int64_t)m->d_model, 2 * (int64_t)m->ffn_dim, m->vocab});
    EC_REQUIRE(widest * m->d_model * 2 <= 0x7fffffff, EC_ERR_UNSUPPORTED,
               "bf16 model: a %lld x %d weight matrix exceeds the 2 GiB buffer range", (long long)widest,
               m->d_model);
  } else {
    EC_REQUIRE(m->d_model % 4 == 0, EC_ERR_UNSUPPORTED, "f32 model: d_model %% 4 != 0");
  }
  return EC_OK;
}

// bf16 forwards over up to `rows` rows: activations [rows, max(d, F)] and the K / V caches
// [rows, d] are addressed through 32-bit byte offsets
ec_status check_rows_fit(const ec_model_desc* m, int64_t rows) {
  if (m->dtype != EC_BF16) return EC_OK;
  EC_REQUIRE(rows * std::max(m->d_model, m->ffn_dim) * 2 <= 0x7fffffff, EC_ERR_UNSUPPORTED,
             "bf16 model: %lld rows of width %d exceed the 2 GiB buffer range", (long long)rows,
             std::max(m->d_model, m->ffn_dim));
  return EC_OK;
}

ec_status check_cache(const ec_cache_desc* c, const ec_model_desc* m) {
  EC_REQUIRE(c && c->struct_size >= sizeof(ec_cache_desc), EC_ERR_ARG, "cache: null or struct_size too small");
  EC_REQUIRE(c->seq_len >= 1 && c->k && c->v, EC_ERR_ARG, "cache: bad seq_len or null arrays");
  EC_REQUIRE(c->seq_len <= m->rope_max_pos, EC_ERR_ARG, "cache: seq_len %d > rope_max_pos %d",
             c->seq_len, m->rope_max_pos);
  for (int l = 0; l < m->n_layers; ++l) {
    EC_REQUIRE(c->k[l] && c->v[l], EC_ERR_ARG, "cache: null pointer for layer %d", l);
    EC_REQUIRE((((uintptr_t)c->k[l] | (uintptr_t)c->v[l]) & 15) == 0, EC_ERR_ARG,
               "cache: layer %d arrays must be 16-byte aligned", l);
  }
  return EC_OK;
}

struct FwdWs {
  float* h;
  void* a;
  void* q;
  void* o;
  void* s;
  void* xn;
  float* hc;  // [max_out, d] fp32 residual rows of the outputs in the last layer
  void* qc;   // [max_out, d] their queries
  float* splitk;
  size_t splitk_bytes;
  void* attn;
  size_t attn_bytes;
};

size_t splitk_max(const ec_model_desc* m, int max_rows, int max_out) {
  if (m->dtype != EC_BF16) return 0;
  const int d = m->d_model, F = m->ffn_dim, V = m->vocab;
  // memo of the last query (the bound is recomputed only when a shape changes)
  static thread_local int key[5] = {-1, -1, -1, -1, -1};
  static thread_local size_t memo = 0;
  if (key[0] == d && key[1] == F && key[2] == V && key[3] == max_rows && key[4] == max_out) return memo;
  size_t best = 0;
  for (int M = 1; M <= max_rows; ++M) {
    best = std::max(best, gemm_splitk_ws_bytes(M, 3 * d, d, EPI_QKV, true));
    best = std::max(best, gemm_splitk_ws_bytes(M, d, d, EPI_RESID, true));
    best = std::max(best, gemm_splitk_ws_bytes(M, F, d, EPI_SWIGLU, true));
    best = std::max(best, gemm_splitk_ws_bytes(M, d, F, EPI_RESID, true));
  }
  for (int M = 1; M <= max_out; ++M) best = std::max(best, gemm_splitk_ws_bytes(M, V, d, EPI_STORE, true));
  key[0] = d; key[1] = F; key[2] = V; key[3] = max_rows; key[4] = max_out;
  memo = best;
  return best;
}

size_t attn_max(const ec_model_desc* m, int max_rows, int L) {
  static thread_local int key[4] = {-1, -1, -1, -1};
  static thread_local size_t memo = 0;
  if (key[0] == m->n_heads && key[1] == m->head_dim && key[2] == max_rows && key[3] == L) return memo;
  size_t best = 0;
  for (int r = 1; r <= max_rows; ++r)
    best = std::max(best, attn_ws_bytes(r, L, m->n_heads, m->head_dim));
  key[0] = m->n_heads; key[1] = m->head_dim; key[2] = max_rows; key[3] = L;
  memo = best;
  return best;
}

// carve the forward's workspace; with base == nullptr only computes the size
size_t carve_fwd(const ec_model_desc* m, int max_rows, int max_out, int L, void* base, size_t cap,
                 FwdWs* w) {
  Carver c(base, cap);
  const size_t es = esize(m->dtype);
  const int d = m->d_model, F = m->ffn_dim;
  FwdWs x;
  x.h = c.take<float>((size_t)max_rows * d);
  x.a = c.take<char>((size_t)max_rows * d * es);
  x.q = c.take<char>((size_t)max_rows * d * es);
  x.o = c.take<char>((size_t)max_rows * d * es);
  x.s = c.take<char>((size_t)max_rows * F * es);
  x.xn = c.take<char>((size_t)std::max(max_out, 1) * d * es);
  x.hc = c.take<float>((size_t)std::max(max_out, 1) * d);
  x.qc = c.take<char>((size_t)std::max(max_out, 1) * d * es);
  x.splitk_bytes = splitk_max(m, max_rows, max_out);
  x.splitk = c.take<float>(x.splitk_bytes / sizeof(float) + 1);
  x.attn_bytes = attn_max(m, max_rows, L);
  x.attn = c.take<char>(x.attn_bytes + 1);
  if (w) *w = x;
  return c.off + 256;
}

// The forward over `rows` (see ec_forward). All pointers validated by the caller.
// Rows of several sequences in one forward (ec_step_batch): sequence s owns rows
// [row_off[s], row_off[s+1]) of the concatenated row list.
struct BatchRows {
  int n_seq;
  const int32_t* row_seq;          // device [rows]: sequence of each row
  SeqPtrs tok;                     // token array of each sequence (kernel arguments)
  const int* row_off;              // host [n_seq + 1]
  const int* out_off;              // host [n_seq + 1]: sequence s owns outputs [out_off[s], out_off[s+1])
  const ec_cache_desc* caches;     // host [n_seq]
};

// KV-drift probe buffers of a forward (ec_step_probe)
struct DriftProbe {
  void* old_k;   // [rows, d] cached K of the rows before the layer's QKV GEMM
  void* old_v;
  float* dist;   // [n_layers][2][rows] per-row cosine distances
  float* out;    // device [4 * n_layers]
};

// Entropy outputs of a forward whose LM head reduces its logits on the fly (bf16).
struct FusedEnt {
  EntPart* parts;  // [n_out, column tiles of the LM head]
  float* H;
  int32_t* amax;
  float* conf;
};

ec_status run_forward(const ec_model_desc* m, const ec_cache_desc* c, const int32_t* tokens,
                      const int32_t* rows, int n_rows, const int32_t* out_idx, int n_out,
                      void* logits, float* hidden, const FwdWs& w, hipStream_t s,
                      const FusedEnt* fe = nullptr, const BatchRows* b = nullptr,
                      const DriftProbe* probe = nullptr) {
  const ec_dtype dt = m->dtype;
  const int d = m->d_model, F = m->ffn_dim, V = m->vocab, H = m->n_heads, Dh = m->head_dim;
  const int L = c->seq_len;
  const float scale = 1.0f / sqrtf((float)Dh);
  ec_status st;
#define EC_TRY(x)            \
  do {                       \
    st = (x);                \
    if (st != EC_OK) return st; \
  } while (0)
  const double es = (double)esize(dt);
  const double M = n_rows, Lq = L, dd = d, FF = F, VV = V, NO = n_out;
  if (n_rows > 0) {
    {
      TScope t(EC_T_EMBED, s, 0.0, M * dd * (es + 4));
      EC_TRY(embed(dt, m->embed, V, tokens, L, rows, n_rows, d, w.h, s, b ? &b->tok : nullptr,
                   b ? b->row_seq : nullptr));
    }
    // normed: w.a already holds this layer's attention-norm input (the previous layer's
    // down projection fused its split-K reduction with the norm)
    bool normed = false;
    // Only the output rows' final hidden states are read (by the LM head), unless the
    // caller asks for every row's. The last layer then computes K/V of every row (the
    // cache update), but its attention, O-proj and MLP only for the output rows: their
    // queries and residual rows are gathered after the QKV projection.
    const bool prune = hidden == nullptr && n_out > 0 && n_out < n_rows && m->n_layers > 0;
    float* hres = w.h;  // residual rows of the current layer
    int Mr = n_rows;    // rows past the QKV projection
    const void* qin = w.q;
    for (int l = 0; l < m->n_layers; ++l) {
      const ec_layer_weights& lw = m->layers[l];
      if (!normed) {
        TScope t(EC_T_NORM, s, 0.0, M * dd * (4 + es));
        EC_TRY(rmsnorm(dt, w.h, n_rows, nullptr, n_rows, d, lw.attn_norm, m->rms_eps, w.a, s));
      }
      EpiArgs e{};
      e.kind = EPI_QKV;
      e.out = w.q;
      e.ldo = d;
      if (b) {
        e.row_seq = b->row_seq;
        for (int q = 0; q < b->n_seq; ++q) {
          e.k_seq.p[q] = b->caches[q].k[l];
          e.v_seq.p[q] = b->caches[q].v[l];
        }
      } else {
        e.k_cache = c->k[l];
        e.v_cache = c->v[l];
      }
      e.rows = rows;
      e.rope_cos = m->rope_cos;
      e.rope_sin = m->rope_sin;
      e.d_model = d;
      e.head_dim = Dh;
      e.seq_len = L;
      if (probe)
        EC_TRY(drift_gather(dt, c->k[l], c->v[l], rows, n_rows, L, d, probe->old_k, probe->old_v, s));
      {
        TScope t(EC_T_QKV, s, 2 * M * 3 * dd * dd, (3 * dd * dd + M * dd + 3 * M * dd) * es);
        EC_TRY(gemm(dt, w.a, lw.wqkv, nullptr, n_rows, 3 * d, d, e, w.splitk, w.splitk_bytes, s));
      }
      if (probe)
        EC_TRY(drift_rows(dt, probe->old_k, probe->old_v, c->k[l], c->v[l], rows, n_rows, L, d,
                          probe->dist + (size_t)l * 2 * n_rows, s));
      const bool outputs_only = prune && l + 1 == m->n_layers;
      if (outputs_only) {
        TScope t(EC_T_LAST, s, 0.0, (double)n_out * dd * (4 + es) * 2);
        EC_TRY(gather_rows2(out_idx, n_out, w.q, w.qc, (size_t)d * esize(dt), w.h, w.hc, (size_t)d * 4, s));
        hres = w.hc;
        Mr = n_out;
        qin = w.qc;
      }
      const double Ml = Mr;
      const int* off = outputs_only ? (b ? b->out_off : nullptr) : (b ? b->row_off : nullptr);
      {
        TScope t(outputs_only ? EC_T_LAST : EC_T_ATTN, s, 4 * Ml * Lq * dd, (2 * Lq * dd + 2 * Ml * dd) * es);
        if (b) {
          // one launch for every sequence: each sequence's rows attend to its own cache
          AttnSeqs as{};
          as.n = b->n_seq;
          for (int q = 0; q < b->n_seq; ++q)
            as.s[q] = AttnSeq{off[q], off[q + 1] - off[q], b->caches[q].k[l], b->caches[q].v[l]};
          EC_TRY(attn_batch(dt, qin, as, L, H, Dh, scale, w.o, w.attn, w.attn_bytes, s));
        } else {
          EC_TRY(attn(dt, qin, c->k[l], c->v[l], Mr, L, H, Dh, scale, w.o, w.attn, w.attn_bytes, s));
        }
      }
      EpiArgs r{};
      r.kind = EPI_RESID;
      r.resid = hres;
      r.ldo = d;
      r.norm_gain = lw.mlp_norm;
      r.norm_out = w.a;
      r.norm_eps = m->rms_eps;
      {
        TScope t(outputs_only ? EC_T_LAST : EC_T_OPROJ, s, 2 * Ml * dd * dd, (dd * dd + Ml * dd) * es + 8 * Ml * dd);
        EC_TRY(gemm(dt, w.o, lw.wo, nullptr, Mr, d, d, r, w.splitk, w.splitk_bytes, s, &normed));
      }
      if (!normed) {
        TScope t(outputs_only ? EC_T_LAST : EC_T_NORM, s, 0.0, Ml * dd * (4 + es));
        EC_TRY(rmsnorm(dt, hres, Mr, nullptr, Mr, d, lw.mlp_norm, m->rms_eps, w.a, s));
      }
      EpiArgs g{};
      g.kind = EPI_SWIGLU;
      g.out = w.s;
      g.ldo = F;
      {
        TScope t(outputs_only ? EC_T_LAST : EC_T_GATEUP, s, 4 * Ml * FF * dd, (2 * FF * dd + Ml * dd + Ml * FF) * es);
        EC_TRY(gemm(dt, w.a, lw.w_gate, lw.w_up, Mr, F, d, g, w.splitk, w.splitk_bytes, s));
      }
      // the next layer's attention norm rides on the down projection's split-K reduction
      const bool has_next = l + 1 < m->n_layers;
      r.norm_gain = has_next ? m->layers[l + 1].attn_norm : nullptr;
      r.norm_out = has_next ? w.a : nullptr;
      {
        TScope t(outputs_only ? EC_T_LAST : EC_T_DOWN, s, 2 * Ml * dd * FF, (dd * FF + Ml * FF) * es + 8 * Ml * dd);
        EC_TRY(gemm(dt, w.s, lw.w_down, nullptr, Mr, d, F, r, w.splitk, w.splitk_bytes, s, &normed));
      }
    }
  }
  // the last layer ran over the gathered output rows (w.hc) only
  const bool pruned = hidden == nullptr && n_out > 0 && n_out < n_rows && m->n_layers > 0;
  if (probe && n_rows > 0) EC_TRY(drift_reduce(probe->dist, m->n_layers, n_rows, 2 * (int64_t)n_rows, probe->out, s));
  if (hidden && n_rows > 0)
    EC_CHECK_HIP(hipMemcpyAsync(hidden, w.h, (size_t)n_rows * d * sizeof(float),
                                hipMemcpyDeviceToDevice, s));
  if (n_out > 0) {
    TScope t(EC_T_LMHEAD, s, 2 * NO * VV * dd, (VV * dd + NO * dd + (fe ? 0.0 : NO * VV)) * es + NO * dd * 4);
    if (pruned) EC_TRY(rmsnorm(dt, w.hc, n_out, nullptr, n_out, d, m->final_norm, m->rms_eps, w.xn, s));
    else EC_TRY(rmsnorm(dt, w.h, n_rows, out_idx, n_out, d, m->final_norm, m->rms_eps, w.xn, s));
    EpiArgs o{};
    if (fe) {
      // LM head with the entropy / argmax / confidence reduction in its epilogue: one
      // partial state per (row, column tile) instead of a logits tensor
      o.kind = EPI_ENTROPY;
      o.parts = fe->parts;
      EC_TRY(gemm(dt, w.xn, m->lm_head, nullptr, n_out, V, d, o, w.splitk, w.splitk_bytes, s));
    } else {
      o.kind = EPI_STORE;
      o.out = logits;
      o.ldo = V;
      EC_TRY(gemm(dt, w.xn, m->lm_head, nullptr, n_out, V, d, o, w.splitk, w.splitk_bytes, s));
    }
  }
  if (fe && n_out > 0) {
    TScope t(EC_T_ENTROPY, s, 0.0, NO * (VV / 128.0) * sizeof(EntPart));
    EC_TRY(entropy_merge(fe->parts, n_out, gemm_col_tiles(n_out, V, d, EPI_ENTROPY), fe->H, fe->amax,
                         fe->conf, s));
  }
#undef EC_TRY
  return EC_OK;
}

// ec_step workspace: forward (rows up to L, outputs up to B) + logits + reduction + result
struct StepWs {
  FwdWs fwd;
  void* logits;
  float* H;
  int32_t* amax;
  float* conf;
  void* ent_ws;
  size_t ent_bytes;
  void* old_k;   // KV-drift probe (ec_step_probe)
  void* old_v;
  float* dist;
};

int max_cand(const ec_params* p) {
  return std::max(1, std::min(p->block_len, p->seq_len - p->prompt_len));
}

size_t carve_step(const ec_model_desc* m, const ec_params* p, void* base, size_t cap, StepWs* w) {
  const int L = p->seq_len, O = max_cand(p);
  StepWs x;
  const size_t fwd = carve_fwd(m, L, O, L, base, cap, &x.fwd);
  Carver c(base, cap);
  c.off = fwd;
  x.logits = c.take<char>((size_t)O * m->vocab * esize(m->dtype));
  x.H = c.take<float>(O);
  x.amax = c.take<int32_t>(O);
  x.conf = c.take<float>(O);
  x.ent_bytes = std::max(entropy_ws_bytes(O, m->vocab),
                         (size_t)O * ((m->vocab + 127) / 128) * sizeof(EntPart));
  x.ent_ws = c.take<char>(x.ent_bytes + 1);
  x.old_k = c.take<char>((size_t)L * m->d_model * esize(m->dtype));
  x.old_v = c.take<char>((size_t)L * m->d_model * esize(m->dtype));
  x.dist = c.take<float>((size_t)m->n_layers * 2 * L);
  if (w) *w = x;
  return c.off + 256;
}

// Apply a step's device result to the state and the host record; false if E is NaN.
bool finish_step(const StepResult& h, const ec_params& p, bool full, int n_rows, int n_cand, ec_state* state,
                 ec_step_out* out) {
  const bool nan = h.has_nan != 0;
  const bool refresh = nan || (h.emax > p.tau);
  out->status = nan ? EC_ERR_NAN : EC_OK;
  out->refreshed = full ? 1 : 0;
  out->rows = n_rows;
  out->n_cand = n_cand;
  out->n_decoded = h.n_picked;
  out->refresh_next = refresh ? 1 : 0;
  out->emax = h.emax;
  for (int i = 0; i < h.n_picked && i < EC_MAX_TOKENS_PER_STEP; ++i) {
    out->positions[i] = h.pos[i];
    out->ids[i] = h.ids[i];
    out->entropy[i] = h.ent[i];
    out->maxprob[i] = h.conf[i];
  }
  state->t += 1;
  state->refresh_next = refresh ? 1 : 0;
  state->n_masked = h.n_masked;
  state->n_decoded += h.n_picked;
  state->next_rows = h.next_rows;
  state->next_cand = h.next_cand;
  return !nan;
}

// ec_step_batch workspace: the forward over every sequence's rows, candidates of all
// sequences, the concatenated row / candidate lists and the device pointer tables
struct BatchWs {
  FwdWs fwd;
  void* logits;  // fp32 models only
  float* H;
  int32_t* amax;
  float* conf;
  void* ent_ws;
  size_t ent_bytes;
  int32_t* rows_all;
  int32_t* row_seq;
  int32_t* out_all;
};

size_t carve_batch(const ec_model_desc* m, int n_seq, const ec_params* p, void* base, size_t cap, BatchWs* w) {
  const int L = p->seq_len, O = max_cand(p);
  const int MR = n_seq * L, MO = n_seq * O;
  BatchWs x;
  const size_t fwd = carve_fwd(m, MR, MO, L, base, cap, &x.fwd);
  Carver c(base, cap);
  c.off = fwd;
  x.logits = c.take<char>(m->dtype == EC_F32 ? (size_t)MO * m->vocab * 4 : 1);
  x.H = c.take<float>(MO);
  x.amax = c.take<int32_t>(MO);
  x.conf = c.take<float>(MO);
  x.ent_bytes = std::max(entropy_ws_bytes(MO, m->vocab), (size_t)MO * ((m->vocab + 127) / 128) * sizeof(EntPart));
  x.ent_ws = c.take<char>(x.ent_bytes + 1);
  x.rows_all = c.take<int32_t>(MR);
  x.row_seq = c.take<int32_t>(MR);
  x.out_all = c.take<int32_t>(MO);
  if (w) *w = x;
  return c.off + 256;
}

ec_status check_params(const ec_params* p, const ec_model_desc* m, const ec_cache_desc* c) {
  EC_REQUIRE(p && p->struct_size >= sizeof(ec_params), EC_ERR_ARG, "params: null or struct_size too small");
  EC_REQUIRE(p->seq_len >= 1 && p->prompt_len >= 0 && p->prompt_len <= p->seq_len, EC_ERR_ARG,
             "params: bad seq_len / prompt_len");
  EC_REQUIRE(p->block_len >= 1, EC_ERR_ARG, "params: block_len must be >= 1");
  EC_REQUIRE(p->k_recent >= 0, EC_ERR_ARG, "params: k_recent must be >= 0");
  EC_REQUIRE(p->tokens_per_step >= 1 && p->tokens_per_step <= EC_MAX_TOKENS_PER_STEP, EC_ERR_ARG,
             "params: tokens_per_step must be in [1, %d]", EC_MAX_TOKENS_PER_STEP);
  EC_REQUIRE(!(p->tau != p->tau), EC_ERR_ARG, "params: tau is NaN");
  EC_REQUIRE(p->candidates == EC_CAND_BLOCKS || p->candidates == EC_CAND_WINDOW, EC_ERR_ARG,
             "params: candidates must be EC_CAND_BLOCKS or EC_CAND_WINDOW");
  if (m) EC_REQUIRE(p->mask_id >= 0 && p->mask_id < m->vocab, EC_ERR_ARG, "params: mask_id out of range");
  if (c) EC_REQUIRE(c->seq_len == p->seq_len, EC_ERR_ARG, "params: seq_len differs from cache");
  if (m) return check_rows_fit(m, p->seq_len);
  return EC_OK;
}

}  // namespace
}  // namespace ec

using namespace ec;

// One step of one sequence (ec_step, and with drift != NULL ec_step_probe).
ec_status step_impl(const ec_model_desc* model, const ec_cache_desc* cache, ec_state* state,
                    const ec_params* params, void* workspace, size_t workspace_bytes, void* stream,
                    ec_step_out* out, float* drift) {
  ec_status st = check_model(model);
  if (st != EC_OK) return st;
  st = check_cache(cache, model);
  if (st != EC_OK) return st;
  st = check_params(params, model, cache);
  if (st != EC_OK) return st;
  EC_REQUIRE(state && state->struct_size >= sizeof(ec_state) && state->tokens && state->masked &&
                 state->plan,
             EC_ERR_ARG, "ec_step: bad state");
  EC_REQUIRE(out && out->struct_size >= sizeof(ec_step_out), EC_ERR_ARG, "ec_step: bad out");
  const size_t need = carve_step(model, params, nullptr, 0, nullptr);
  EC_REQUIRE(workspace && workspace_bytes >= need, EC_ERR_WORKSPACE,
             "ec_step: workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  const uint32_t osz = out->struct_size;
  memset(out, 0, sizeof(ec_step_out));
  out->struct_size = osz;
  if (state->n_masked <= 0) return EC_OK;

  StepWs w;
  carve_step(model, params, workspace, workspace_bytes, &w);
  const PlanLayout lay(params->seq_len, params->k_recent);
  StepResult* res = (StepResult*)(state->plan + lay.RES);
  const bool full = state->t == 0 || state->refresh_next;
  const int L = params->seq_len;
  const int n_rows = full ? L : state->next_rows;
  const int n_cand = state->next_cand;
  const int32_t* rows = state->plan + (full ? lay.J0 : lay.R0);
  // candidate indices into rows: positions themselves on a full step
  const int32_t* cidx = state->plan + (full ? lay.C0 : lay.I0);

  const DriftProbe probe{w.old_k, w.old_v, w.dist, drift};
  const DriftProbe* pr = drift ? &probe : nullptr;
  if (model->dtype == EC_BF16) {
    // the LM head reduces the candidates' logits in its epilogue (no logits tensor)
    const FusedEnt fe{(EntPart*)w.ent_ws, w.H, w.amax, w.conf};
    st = run_forward(model, cache, state->tokens, rows, n_rows, cidx, n_cand, nullptr, nullptr, w.fwd, s,
                     &fe, nullptr, pr);
    if (st != EC_OK) return st;
  } else {
    st = run_forward(model, cache, state->tokens, rows, n_rows, cidx, n_cand, w.logits, nullptr,
                     w.fwd, s, nullptr, nullptr, pr);
    if (st != EC_OK) return st;
    TScope t(EC_T_ENTROPY, s, 0.0, (double)n_cand * model->vocab * esize(model->dtype));
    st = entropy(model->dtype, w.logits, n_cand, model->vocab, model->vocab, nullptr, 0, w.H,
                 w.amax, w.conf, nullptr, w.ent_ws, w.ent_bytes, s);
    if (st != EC_OK) return st;
  }
  {
    TScope t(EC_T_SELECT, s, 0.0, 0.0);
    st = select_decode(w.H, w.amax, w.conf, n_cand, state->tokens, state->masked, state->plan,
                       *params, res, s);
  }
  if (st != EC_OK) return st;
  StepResult h;
  EC_CHECK_HIP(hipMemcpyAsync(&h, res, sizeof(StepResult), hipMemcpyDeviceToHost, s));
  EC_CHECK_HIP(hipStreamSynchronize(s));
  if (g_tm.on) timing_collect();
  if (!finish_step(h, *params, full, n_rows, n_cand, state, out)) {
    set_error("ec_step: E is NaN at step %d; next step refreshes", state->t - 1);
    return EC_ERR_NAN;
  }
  return EC_OK;
}

extern "C" {

const char* ec_last_error(void) { return g_err; }

ec_status ec_timing_enable(int on) {
  if (!on) timing_collect();
  g_tm.on = on != 0;
  return EC_OK;
}

ec_status ec_timing_select(uint32_t kinds) {
  g_tm.mask = kinds;
  return EC_OK;
}

ec_status ec_timing_read(ec_timing* out, int reset) {
  EC_REQUIRE(out && out->struct_size >= sizeof(ec_timing), EC_ERR_ARG, "ec_timing_read: bad out");
  timing_collect();
  const uint32_t sz = out->struct_size;
  memset(out, 0, sizeof(ec_timing));
  out->struct_size = sz;
  out->n_kinds = EC_T_KINDS;
  for (int k = 0; k < EC_T_KINDS; ++k) {
    out->ms[k] = g_tm.ms[k];
    out->launches[k] = g_tm.launches[k];
    out->flops[k] = g_tm.flops[k];
    out->bytes[k] = g_tm.bytes[k];
    if (reset) {
      g_tm.ms[k] = g_tm.flops[k] = g_tm.bytes[k] = 0;
      g_tm.launches[k] = 0;
    }
  }
  return EC_OK;
}
int ec_version(void) { return EC_VERSION; }

ec_status ec_pack_weights(ec_dtype dtype, int32_t d_model, int32_t head_dim, int32_t ffn_dim,
                          const void* wqkv, const void* w_gate, const void* w_up,
                          void* wqkv_packed, void* gateup_packed, void* stream) {
  EC_REQUIRE(dtype_ok(dtype), EC_ERR_DTYPE, "ec_pack_weights: bad dtype %d", (int)dtype);
  EC_REQUIRE(d_model > 0 && head_dim > 0 && ffn_dim > 0, EC_ERR_ARG, "ec_pack_weights: non-positive size");
  if (wqkv_packed) {
    EC_REQUIRE(wqkv, EC_ERR_ARG, "ec_pack_weights: wqkv is NULL");
    EC_REQUIRE(head_dim % 32 == 0 && d_model % head_dim == 0, EC_ERR_ARG,
               "ec_pack_weights: need head_dim %% 32 == 0 and d_model %% head_dim == 0");
  }
  if (gateup_packed) {
    EC_REQUIRE(w_gate && w_up, EC_ERR_ARG, "ec_pack_weights: w_gate or w_up is NULL");
    EC_REQUIRE(ffn_dim % 16 == 0, EC_ERR_ARG, "ec_pack_weights: need ffn_dim %% 16 == 0");
  }
  return pack_weights((int)esize(dtype), d_model, head_dim, ffn_dim, wqkv, w_gate, w_up, wqkv_packed,
                      gateup_packed, (hipStream_t)stream);
}

size_t ec_entropy_max_workspace_size(int32_t rows, int32_t vocab) {
  return entropy_ws_bytes(rows, vocab);
}

ec_status ec_entropy_max(const void* logits, ec_dtype dtype, int32_t rows, int32_t vocab,
                         int64_t row_stride, const int32_t* sel, int32_t n_sel, float* entropy,
                         int32_t* argmax, float* maxprob, float* emax, void* workspace,
                         size_t workspace_bytes, void* stream) {
  EC_REQUIRE(dtype_ok(dtype), EC_ERR_DTYPE, "ec_entropy_max: bad dtype %d", (int)dtype);
  EC_REQUIRE(rows >= 0 && vocab >= 1 && row_stride >= vocab, EC_ERR_ARG,
             "ec_entropy_max: rows %d vocab %d stride %lld", rows, vocab, (long long)row_stride);
  EC_REQUIRE(n_sel >= 0, EC_ERR_ARG, "ec_entropy_max: n_sel < 0");
  if (rows > 0) {
    EC_REQUIRE(logits && entropy && argmax && maxprob, EC_ERR_ARG, "ec_entropy_max: null pointer");
    const size_t need = entropy_ws_bytes(rows, vocab);
    EC_REQUIRE(workspace && workspace_bytes >= need, EC_ERR_WORKSPACE,
               "ec_entropy_max: workspace %zu < %zu bytes", workspace_bytes, need);
  }
  TScope t(EC_T_ENTROPY, (hipStream_t)stream, 0.0, (double)rows * vocab * esize(dtype));
  return ec::entropy(dtype, logits, rows, vocab, row_stride, sel, n_sel, entropy, argmax, maxprob, emax,
                     workspace, workspace_bytes, (hipStream_t)stream);
}

ec_status ec_entropy_max_noalloc(const void* logits, ec_dtype dtype, int32_t rows, int32_t vocab,
                                 int64_t row_stride, const int32_t* sel, int32_t n_sel, float* entropy,
                                 int32_t* argmax, float* maxprob, float* emax, void* stream) {
  static_assert(EC_ENTROPY_NOALLOC_SCRATCH_BYTES == kEntropyScratchBytes, "scratch size mismatch");
  EC_REQUIRE(dtype_ok(dtype), EC_ERR_DTYPE, "ec_entropy_max_noalloc: bad dtype %d", (int)dtype);
  EC_REQUIRE(rows >= 0 && vocab >= 1 && row_stride >= vocab, EC_ERR_ARG,
             "ec_entropy_max_noalloc: rows %d vocab %d stride %lld", rows, vocab, (long long)row_stride);
  EC_REQUIRE(n_sel >= 0, EC_ERR_ARG, "ec_entropy_max_noalloc: n_sel < 0");
  if (rows > 0)
    EC_REQUIRE(logits && entropy && argmax && maxprob, EC_ERR_ARG, "ec_entropy_max_noalloc: null pointer");
  TScope t(EC_T_ENTROPY, (hipStream_t)stream, 0.0, (double)rows * vocab * esize(dtype));
  return ec::entropy_noalloc(dtype, logits, rows, vocab, row_stride, sel, n_sel, entropy, argmax, maxprob, emax,
                             (hipStream_t)stream);
}

ec_status ec_cache_scatter(void* k_cache, void* v_cache, int64_t seq_len, int32_t width,
                           ec_dtype dtype, const void* k_rows, const void* v_rows,
                           const int32_t* idx, int32_t n_rows, void* stream) {
  EC_REQUIRE(dtype_ok(dtype), EC_ERR_DTYPE, "ec_cache_scatter: bad dtype %d", (int)dtype);
  EC_REQUIRE(seq_len >= 0 && width >= 1 && n_rows >= 0, EC_ERR_ARG, "ec_cache_scatter: bad sizes");
  if (n_rows == 0) return EC_OK;
  EC_REQUIRE(k_cache && v_cache && k_rows && v_rows && idx, EC_ERR_ARG, "ec_cache_scatter: null pointer");
  return scatter(dtype, k_cache, v_cache, seq_len, width, k_rows, v_rows, idx, n_rows,
                 (hipStream_t)stream);
}

size_t ec_partial_attn_workspace_size(int32_t r, int32_t seq_len, int32_t n_heads, int32_t head_dim) {
  return attn_ws_bytes(r, seq_len, n_heads, head_dim);
}

ec_status ec_partial_attn_plan(int32_t r, int32_t seq_len, int32_t n_heads, int32_t head_dim,
                               int32_t* query_tile, int32_t* splits) {
  EC_REQUIRE(query_tile && splits, EC_ERR_ARG, "ec_partial_attn_plan: null output");
  EC_REQUIRE(r >= 1 && seq_len >= 1 && n_heads >= 1, EC_ERR_ARG, "ec_partial_attn_plan: bad sizes");
  EC_REQUIRE(head_dim == 128, EC_ERR_UNSUPPORTED, "ec_partial_attn_plan: the bf16 path needs head_dim 128");
  int qt = 0, sp = 0;
  attn_plan_query(r, seq_len, n_heads, &qt, &sp);
  *query_tile = qt;
  *splits = sp;
  return EC_OK;
}

ec_status ec_partial_attn(const void* q, const void* k_cache, const void* v_cache, int32_t r,
                          int32_t seq_len, int32_t n_heads, int32_t head_dim, float scale,
                          ec_dtype dtype, void* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  EC_REQUIRE(dtype_ok(dtype), EC_ERR_DTYPE, "ec_partial_attn: bad dtype %d", (int)dtype);
  EC_REQUIRE(r >= 0 && seq_len >= 1 && n_heads >= 1 && head_dim >= 1, EC_ERR_ARG,
             "ec_partial_attn: bad sizes");
  if (r == 0) return EC_OK;
  EC_REQUIRE(q && k_cache && v_cache && out, EC_ERR_ARG, "ec_partial_attn: null pointer");
  EC_REQUIRE(scale > 0.f, EC_ERR_ARG, "ec_partial_attn: scale must be positive");
  const size_t need = attn_ws_bytes(r, seq_len, n_heads, head_dim);
  EC_REQUIRE(need == 0 || (workspace && workspace_bytes >= need), EC_ERR_WORKSPACE,
             "ec_partial_attn: workspace %zu < %zu bytes", workspace_bytes, need);
  return attn(dtype, q, k_cache, v_cache, r, seq_len, n_heads, head_dim, scale, out, workspace,
              workspace_bytes, (hipStream_t)stream);
}

ec_status ec_rope_table(float* cos_out, float* sin_out, int32_t max_pos, int32_t head_dim,
                        double base, void* stream) {
  EC_REQUIRE(cos_out && sin_out && max_pos >= 1 && head_dim >= 2 && head_dim % 2 == 0 && base > 0,
             EC_ERR_ARG, "ec_rope_table: bad arguments");
  return rope_table(cos_out, sin_out, max_pos, head_dim, base, (hipStream_t)stream);
}

size_t ec_forward_workspace_size(const ec_model_desc* model, int32_t max_rows, int32_t max_out,
                                 int32_t seq_len) {
  if (check_model(model) != EC_OK || max_rows < 0 || max_out < 0 || seq_len < 1) return 0;
  return carve_fwd(model, std::max(max_rows, 1), max_out, seq_len, nullptr, 0, nullptr);
}

ec_status ec_forward(const ec_model_desc* model, const ec_cache_desc* cache, const int32_t* tokens,
                     const int32_t* rows, int32_t n_rows, const int32_t* out_idx, int32_t n_out,
                     void* logits, float* hidden, void* workspace, size_t workspace_bytes,
                     void* stream) {
  ec_status st = check_model(model);
  if (st != EC_OK) return st;
  st = check_cache(cache, model);
  if (st != EC_OK) return st;
  EC_REQUIRE(n_rows >= 0 && n_rows <= cache->seq_len && n_out >= 0 && n_out <= std::max(n_rows, 0),
             EC_ERR_ARG, "ec_forward: n_rows %d n_out %d", n_rows, n_out);
  st = check_rows_fit(model, cache->seq_len);
  if (st != EC_OK) return st;
  EC_REQUIRE(tokens && (rows || n_rows == 0) && (out_idx || n_out == 0) && (logits || n_out == 0),
             EC_ERR_ARG, "ec_forward: null pointer");
  const size_t need = carve_fwd(model, std::max(n_rows, 1), n_out, cache->seq_len, nullptr, 0, nullptr);
  EC_REQUIRE(workspace && workspace_bytes >= need, EC_ERR_WORKSPACE,
             "ec_forward: workspace %zu < %zu bytes", workspace_bytes, need);
  FwdWs w;
  carve_fwd(model, std::max(n_rows, 1), n_out, cache->seq_len, workspace, workspace_bytes, &w);
  return run_forward(model, cache, tokens, rows, n_rows, out_idx, n_out, logits, hidden, w,
                     (hipStream_t)stream);
}

size_t ec_state_plan_words(int32_t seq_len, int32_t k_recent) {
  if (seq_len < 1) return 0;
  return (size_t)PlanLayout(seq_len, k_recent).words;
}

size_t ec_step_workspace_size(const ec_model_desc* model, const ec_params* params) {
  if (check_model(model) != EC_OK || check_params(params, model, nullptr) != EC_OK) return 0;
  return carve_step(model, params, nullptr, 0, nullptr);
}

ec_status ec_state_reset(ec_state* state, const ec_params* params, void* stream) {
  ec_status st = check_params(params, nullptr, nullptr);
  if (st != EC_OK) return st;
  EC_REQUIRE(state && state->struct_size >= sizeof(ec_state) && state->tokens && state->masked &&
                 state->plan,
             EC_ERR_ARG, "ec_state_reset: bad state");
  hipStream_t s = (hipStream_t)stream;
  StepResult* rec = (StepResult*)(state->plan + PlanLayout(params->seq_len, params->k_recent).RES);
  st = plan_reset(state->tokens, state->masked, state->plan, *params, rec, s);
  StepResult h;
  if (st == EC_OK) {
    hipError_t e = hipMemcpyAsync(&h, rec, sizeof(StepResult), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) st = hip_fail(e, "ec_state_reset: readback");
  }
  if (st != EC_OK) return st;
  state->t = 0;
  state->refresh_next = 1;
  state->n_masked = h.n_masked;
  state->n_decoded = 0;
  state->next_rows = h.next_rows;
  state->next_cand = h.next_cand;
  return EC_OK;
}

ec_status ec_step(const ec_model_desc* model, const ec_cache_desc* cache, ec_state* state,
                  const ec_params* params, void* workspace, size_t workspace_bytes, void* stream,
                  ec_step_out* out) {
  return step_impl(model, cache, state, params, workspace, workspace_bytes, stream, out, nullptr);
}

ec_status ec_step_probe(const ec_model_desc* model, const ec_cache_desc* cache, ec_state* state,
                        const ec_params* params, void* workspace, size_t workspace_bytes, void* stream,
                        ec_step_out* out, float* drift) {
  EC_REQUIRE(drift, EC_ERR_ARG, "ec_step_probe: drift is NULL");
  return step_impl(model, cache, state, params, workspace, workspace_bytes, stream, out, drift);
}


size_t ec_step_batch_workspace_size(const ec_model_desc* model, int32_t n_seq, const ec_params* params) {
  if (check_model(model) != EC_OK || check_params(params, model, nullptr) != EC_OK) return 0;
  if (n_seq < 1 || n_seq > EC_MAX_SEQ) return 0;
  return carve_batch(model, n_seq, params, nullptr, 0, nullptr);
}

ec_status ec_step_batch(const ec_model_desc* model, int32_t n_seq, const ec_cache_desc* caches,
                        ec_state* states, const ec_params* params, void* workspace,
                        size_t workspace_bytes, void* stream, ec_step_out* outs) {
  ec_status st = check_model(model);
  if (st != EC_OK) return st;
  EC_REQUIRE(n_seq >= 1 && n_seq <= EC_MAX_SEQ, EC_ERR_ARG, "ec_step_batch: n_seq %d not in [1, %d]",
             n_seq, EC_MAX_SEQ);
  EC_REQUIRE(caches && states && outs, EC_ERR_ARG, "ec_step_batch: null caches, states or outs");
  st = check_params(params, model, &caches[0]);
  if (st != EC_OK) return st;
  st = check_rows_fit(model, (int64_t)n_seq * params->seq_len);
  if (st != EC_OK) return st;
  for (int q = 0; q < n_seq; ++q) {
    st = check_cache(&caches[q], model);
    if (st != EC_OK) return st;
    EC_REQUIRE(caches[q].seq_len == params->seq_len, EC_ERR_ARG, "ec_step_batch: cache %d seq_len differs", q);
    const ec_state& sq = states[q];
    EC_REQUIRE(sq.struct_size >= sizeof(ec_state) && sq.tokens && sq.masked && sq.plan, EC_ERR_ARG,
               "ec_step_batch: bad state %d", q);
    EC_REQUIRE(outs[q].struct_size >= sizeof(ec_step_out), EC_ERR_ARG, "ec_step_batch: bad out %d", q);
  }
  const size_t need = carve_batch(model, n_seq, params, nullptr, 0, nullptr);
  EC_REQUIRE(workspace && workspace_bytes >= need, EC_ERR_WORKSPACE,
             "ec_step_batch: workspace %zu < %zu bytes", workspace_bytes, need);
  hipStream_t s = (hipStream_t)stream;
  for (int q = 0; q < n_seq; ++q) {
    const uint32_t osz = outs[q].struct_size;
    memset(&outs[q], 0, sizeof(ec_step_out));
    outs[q].struct_size = osz;
  }
  BatchWs w;
  carve_batch(model, n_seq, params, workspace, workspace_bytes, &w);
  const PlanLayout lay(params->seq_len, params->k_recent);
  const int L = params->seq_len;

  // this step's rows and candidates of every sequence, concatenated in sequence order
  BatchSegs segs{};
  int row_off[EC_MAX_SEQ + 1], cand_off[EC_MAX_SEQ + 1];
  bool full[EC_MAX_SEQ] = {};
  int nrows[EC_MAX_SEQ] = {}, ncand[EC_MAX_SEQ] = {};
  int M = 0, C = 0;
  for (int q = 0; q < n_seq; ++q) {
    row_off[q] = M;
    cand_off[q] = C;
    const ec_state& sq = states[q];
    if (sq.n_masked <= 0) continue;
    full[q] = sq.t == 0 || sq.refresh_next;
    nrows[q] = full[q] ? L : sq.next_rows;
    ncand[q] = sq.next_cand;
    segs.seg[segs.n++] = BatchSeg{sq.plan + (full[q] ? lay.J0 : lay.R0), sq.plan + (full[q] ? lay.C0 : lay.I0),
                                  nrows[q], M, ncand[q], C, q};
    M += nrows[q];
    C += ncand[q];
  }
  row_off[n_seq] = M;
  cand_off[n_seq] = C;
  if (segs.n == 0) return EC_OK;

  st = batch_gather(segs, L, w.rows_all, w.row_seq, w.out_all, s);
  if (st != EC_OK) return st;

  BatchRows b{n_seq, w.row_seq, SeqPtrs{}, row_off, cand_off, caches};
  for (int q = 0; q < n_seq; ++q) b.tok.p[q] = states[q].tokens;
  if (model->dtype == EC_BF16) {
    const FusedEnt fe{(EntPart*)w.ent_ws, w.H, w.amax, w.conf};
    st = run_forward(model, &caches[0], nullptr, w.rows_all, M, w.out_all, C, nullptr, nullptr, w.fwd, s,
                     &fe, &b);
    if (st != EC_OK) return st;
  } else {
    st = run_forward(model, &caches[0], nullptr, w.rows_all, M, w.out_all, C, w.logits, nullptr, w.fwd, s,
                     nullptr, &b);
    if (st != EC_OK) return st;
    TScope t(EC_T_ENTROPY, s, 0.0, (double)C * model->vocab * esize(model->dtype));
    st = entropy(model->dtype, w.logits, C, model->vocab, model->vocab, nullptr, 0, w.H, w.amax, w.conf,
                 nullptr, w.ent_ws, w.ent_bytes, s);
    if (st != EC_OK) return st;
  }
  StepResult hres[EC_MAX_SEQ];
  {
    TScope t(EC_T_SELECT, s, 0.0, 0.0);
    for (int i = 0; i < segs.n; ++i) {
      const int q = segs.seg[i].seq;
      StepResult* res = (StepResult*)(states[q].plan + lay.RES);
      st = select_decode(w.H + cand_off[q], w.amax + cand_off[q], w.conf + cand_off[q], ncand[q],
                         states[q].tokens, states[q].masked, states[q].plan, *params, res, s);
      if (st != EC_OK) return st;
    }
  }
  for (int i = 0; i < segs.n; ++i) {
    const int q = segs.seg[i].seq;
    EC_CHECK_HIP(hipMemcpyAsync(&hres[i], states[q].plan + lay.RES, sizeof(StepResult),
                                hipMemcpyDeviceToHost, s));
  }
  EC_CHECK_HIP(hipStreamSynchronize(s));
  if (g_tm.on) timing_collect();
  int bad = -1;
  for (int i = 0; i < segs.n; ++i) {
    const int q = segs.seg[i].seq;
    if (!finish_step(hres[i], *params, full[q], nrows[q], ncand[q], &states[q], &outs[q]) && bad < 0) bad = q;
  }
  if (bad >= 0) {
    set_error("ec_step_batch: E of sequence %d is NaN; its next step refreshes", bad);
    return EC_ERR_NAN;
  }
  return EC_OK;
}

}  // extern "C"
