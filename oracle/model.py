"""Bidirectional transformer forward with a per-layer K/V cache (oracle).

What the pages fix (EntropyCache explainer, Italian summary section 1 and
Arabic technical summary section 1): a diffusion LM attends bidirectionally,
every position to every other, so decoding one token changes every position's
representation; vanilla inference therefore runs a full forward over the
whole sequence at every step. EntropyCache keeps the per-layer K/V of every
position and, on a skip step, recomputes K/V only for the still-masked
positions and the k most recently decoded ones while every other position
reuses its cached K/V (Arabic summary section 2, "Algorithm workflow", phase
1; Italian summary "Algoritmo di Funzionamento", step 2).

The pages give no architecture. The reading used here is a pre-norm LLaMA-
style block: RMSNorm (gain vector, eps), one fused QKV projection, rotary
position embedding (half-split pairs, base 10000) on q and k at the rows'
absolute positions, softmax attention with scale 1/sqrt(head_dim) over all L
cached rows with no mask, output projection and residual, RMSNorm, SwiGLU MLP
(silu(gate) * up, then down) and residual; a final RMSNorm and an untied LM
head give the logits of position i at row i. Projection matrices are stored
[out, in], so y = x W^T. No biases.

Precision: all arithmetic in float64. For bf16 models, values are rounded to
bf16 (round to nearest, ties to even) at the points where the device path
holds bf16: the normed GEMM inputs, q/k/v after RoPE (the cache), the
attention weights that multiply V (as 2^(t - M) for an integer M, see
attention()), the attention output, the SwiGLU product and the logits. The
residual stream is kept unrounded (the device keeps it in fp32).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# numeric formats
# --------------------------------------------------------------------------
def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits), ties to even.

    Written from the format's definition: x = m * 2^e with 0.5 <= |m| < 1; keep
    8 bits of m with round-half-even. Zeros, infinities and NaN pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    finite = np.isfinite(x)
    out = np.where(finite, np.ldexp(np.rint(np.ldexp(np.where(finite, m, 0.0), 8)), e - 8), x)
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64 values (exact)."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# building blocks
# --------------------------------------------------------------------------
def rmsnorm(h: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """h / sqrt(mean(h^2) + eps) * g, per row."""
    ms = np.mean(h * h, axis=-1, keepdims=True)
    return h / np.sqrt(ms + eps) * g


def rope_angles(pos: np.ndarray, head_dim: int, base: float) -> np.ndarray:
    """theta[p, i] = p * base^(-2i/head_dim) for i < head_dim/2, in float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]


def rope(u: np.ndarray, pos: np.ndarray, base: float) -> np.ndarray:
    """Rotate pairs (i, i + D/2) of every head by theta(pos, i).

    u: [n, H, D] at absolute positions pos[n].
      u'_i       = u_i cos t - u_{i+D/2} sin t
      u'_{i+D/2} = u_i sin t + u_{i+D/2} cos t
    """
    n, H, D = u.shape
    t = rope_angles(pos, D, base)[:, None, :]
    c, s = np.cos(t), np.sin(t)
    lo, hi = u[..., : D // 2], u[..., D // 2:]
    return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)


LOG2E = 1.0 / math.log(2.0)


def softmax(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, round_weights=None) -> np.ndarray:
    """Bidirectional attention of query rows over every cached row.

    q: [r, H, D]; K, V: [L, H, D]. For each head, softmax(q K^T / sqrt(D)) V
    over all L keys, no mask.

    With ``round_weights`` (bf16 models: the P.V product takes its weights in
    bf16), the weights of each query row are written in base 2 as
    w_j = 2^(t_j - M), t_j = s_j log2(e), with M the smallest integer >= max_j t_j;
    the weights that multiply V are round_weights(w_j) and the normaliser is the
    unrounded sum: out = sum_j round(w_j) v_j / sum_j w_j. Without rounding this is
    softmax(s) V exactly. Rounding to bf16 commutes with scaling by powers of two,
    so any integer M >= max t gives the same result.
    """
    r, H, D = q.shape
    out = np.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    for h in range(H):
        s = (q[:, h, :] @ K[:, h, :].T) * scale
        if round_weights is None:
            out[:, h, :] = softmax(s) @ V[:, h, :]
        else:
            t = s * LOG2E
            M = np.ceil(t.max(axis=-1, keepdims=True))
            w = np.exp2(t - M)
            out[:, h, :] = (round_weights(w) @ V[:, h, :]) / w.sum(axis=-1, keepdims=True)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# model
# --------------------------------------------------------------------------
class OracleModel:
    """float64 view of seeded weights (``synth.ModelWeights``)."""

    def __init__(self, weights, keep_f64: Optional[bool] = None):
        self.w = weights
        self.shape = weights.shape
        self.dtype = self.shape.dtype
        self.mirror = self.dtype == "bf16"
        self.n_layers = len(weights.layers)
        if keep_f64 is None:
            keep_f64 = self.shape.param_count() * 8 < (6 << 30)
        self.keep = keep_f64
        self._layers: Dict[int, Dict[str, np.ndarray]] = {}
        self._head: Optional[np.ndarray] = None

    def rnd(self, x: np.ndarray) -> np.ndarray:
        return round_bf16(x) if self.mirror else x

    def layer(self, i: int) -> Dict[str, np.ndarray]:
        if i in self._layers:
            return self._layers[i]
        lw = {k: to_f64(v, self.dtype) for k, v in self.w.layers[i].items()}
        if self.keep:
            self._layers[i] = lw
        return lw

    def lm_head(self) -> np.ndarray:
        if self._head is not None:
            return self._head
        hd = to_f64(self.w.lm_head, self.dtype)
        if self.keep:
            self._head = hd
        return hd

    def embed(self, ids: np.ndarray) -> np.ndarray:
        return to_f64(self.w.embed[np.asarray(ids, dtype=np.int64)], self.dtype)

    def final_norm(self) -> np.ndarray:
        return to_f64(self.w.final_norm, self.dtype)


def new_cache(model: OracleModel, seq_len: int) -> List[List[np.ndarray]]:
    d = model.shape.d_model
    return [[np.zeros((seq_len, d)), np.zeros((seq_len, d))] for _ in range(model.n_layers)]


def layer_forward(model: OracleModel, li: int, h: np.ndarray, rows: np.ndarray, kv) -> np.ndarray:
    """One transformer block (EntropyCache explainer, Italian summary section 1: bidirectional
    attention, no mask) for the residual rows ``h`` [r, d] at positions ``rows``: RMSNorm, q/k/v
    with RoPE at the rows' positions, the rows' K/V written into the layer's cache ``kv`` = [K, V]
    ([L, d] each) before the queries attend over all L rows, O-projection and residual, RMSNorm,
    SwiGLU MLP and residual. Returns the residual stream after the block."""
    m = model.shape
    d, H, D = m.d_model, m.n_heads, m.head_dim
    r = len(rows)
    rnd = model.rnd
    lw = model.layer(li)
    K, V = kv
    a = rnd(rmsnorm(h, lw["attn_norm"], m.rms_eps))
    qkv = a @ lw["wqkv"].T
    q = rnd(rope(qkv[:, :d].reshape(r, H, D), rows, m.rope_base))
    k = rnd(rope(qkv[:, d:2 * d].reshape(r, H, D), rows, m.rope_base))
    v = rnd(qkv[:, 2 * d:])
    K[rows] = k.reshape(r, d)
    V[rows] = v
    o = rnd(attention(q, K.reshape(-1, H, D), V.reshape(-1, H, D),
                      round_weights=rnd if model.mirror else None).reshape(r, d))
    h = h + o @ lw["wo"].T
    b = rnd(rmsnorm(h, lw["mlp_norm"], m.rms_eps))
    s = rnd(silu(b @ lw["w_gate"].T) * (b @ lw["w_up"].T))
    return h + s @ lw["w_down"].T


def forward(model: OracleModel, tokens: np.ndarray, rows: Sequence[int], cache,
            out_rows: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Forward pass over the positions ``rows`` against the per-layer cache.

    For each layer the K/V of ``rows`` are computed and written into the cache
    first; the queries of ``rows`` then attend over all L cached rows, which for
    positions outside ``rows`` are whatever the cache already holds. With
    rows = every position this is the full (refresh) forward and no stale
    value is read.

    Returns a dict with
      hidden -- residual stream after the last layer, [r, d] in rows' order;
      normed -- final-RMSNorm output for out_rows (default: rows), [n, d];
      logits -- LM-head logits for out_rows, [n, V].
    """
    m = model.shape
    rows = np.asarray(rows, dtype=np.int64)
    assert len(np.unique(rows)) == len(rows), "recomputed rows must be distinct"
    rnd = model.rnd
    h = model.embed(np.asarray(tokens)[rows])
    for li in range(model.n_layers):
        h = layer_forward(model, li, h, rows, cache[li])
    if out_rows is None:
        sel = np.arange(len(rows))
    else:
        where = {int(p): i for i, p in enumerate(rows)}
        sel = np.array([where[int(p)] for p in out_rows], dtype=np.int64)
    xn = rnd(rmsnorm(h[sel], model.final_norm(), m.rms_eps))
    logits = rnd(xn @ model.lm_head().T)
    return {"hidden": h, "normed": xn, "logits": logits}


def forward_full(model: OracleModel, tokens: np.ndarray, cache, out_rows=None):
    """Refresh: every position recomputed, every cache row rewritten."""
    return forward(model, tokens, np.arange(len(tokens)), cache, out_rows)


def forward_partial(model: OracleModel, tokens: np.ndarray, rows, cache, out_rows=None):
    """Skip step: only ``rows`` recomputed; the other cache rows are reused as they are."""
    return forward(model, tokens, rows, cache, out_rows)
