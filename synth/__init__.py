"""Seeded synthetic inputs for the EntropyCache denoising step.

This module is shared by the CPU oracle, the tests and the benchmark. It holds
only input generation: model shapes, decoding settings, random weights,
prompts and stand-alone logits. None of the method's arithmetic lives here.

Workloads follow the five shapes the method is exercised on (a tiny fp32
model, a vocabulary-wide entropy reduction alone, a small bf16 model, an
8B-shaped bf16 model at L=1024 and a long-context batch of four sequences at
L=4096). The pages measure on trained LLaDA-8B / Dream-7B models and public
reasoning/code benchmarks (EntropyCache explainer, "Experimental results");
neither weights nor datasets are available, so seeded random weights
N(0, 0.02) and uniform random prompt ids stand in for them.

bf16 tensors are carried as numpy uint16 bit patterns (numpy has no bf16);
they are produced from float32 samples with round-to-nearest-even.
"""
from __future__ import annotations

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

WEIGHT_STD = 0.02
CHUNK_ELEMS = 1 << 22  # elements per independently seeded chunk of a tensor


# --------------------------------------------------------------------------
# shapes and settings
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class ModelShape:
    name: str
    dtype: str  # "f32" or "bf16"
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0

    @property
    def mask_id(self) -> int:
        return self.vocab - 1

    def param_count(self) -> int:
        d, f, v = self.d_model, self.ffn_dim, self.vocab
        per_layer = 4 * d * d + 3 * d * f + 2 * d
        return 2 * v * d + d + self.n_layers * per_layer


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    model: ModelShape
    prompt_len: int
    n_masked: int
    tokens_per_step: int
    block_len: int
    k_recent: int
    taus: Tuple[float, ...]
    batch: int = 1
    seed: int = 0
    window: bool = False  # candidates from a sliding window instead of fixed blocks

    @property
    def seq_len(self) -> int:
        return self.prompt_len + self.n_masked

    @property
    def steps(self) -> int:
        return -(-self.n_masked // self.tokens_per_step)

    @property
    def tau(self) -> float:
        return self.taus[len(self.taus) // 2] if len(self.taus) > 1 else self.taus[0]


TINY = ModelShape("tiny", "f32", 2, 256, 4, 64, 1024, 1024)
SMALL = ModelShape("small", "bf16", 8, 2048, 16, 128, 5632, 32000)
M8B = ModelShape("8b", "bf16", 32, 4096, 32, 128, 12288, 126464)

CONFIGS: Dict[str, DecodeConfig] = {
    # fp32, L = 96 + 32, one token per step, k = 4, tau = 0.5 nats
    "tiny": DecodeConfig("tiny", TINY, 96, 32, 1, 32, 4, (0.5,)),
    # bf16, L = 384 + 128, two tokens per step, k = 8, tau = 1.0
    "small": DecodeConfig("small", SMALL, 384, 128, 2, 128, 8, (1.0,)),
    # bf16 8B-shaped, L = 768 + 256, blocks of 32, k = 16, tau swept
    "8b": DecodeConfig("8b", M8B, 768, 256, 1, 32, 16, (0.25, 0.5, 1.0, 2.0)),
    # bf16 8B-shaped, four independent sequences of L = 3584 + 512, k = 32
    "long": DecodeConfig("long", M8B, 3584, 512, 1, 32, 32, (1.0,), batch=4),
}

ENTROPY_ROWS = 64
ENTROPY_VOCAB = 126464
ENTROPY_TEMP_RANGE = (0.05, 5.0)


# --------------------------------------------------------------------------
# seeding and bf16 encoding of inputs
# --------------------------------------------------------------------------
def _rng(seed: int, name: str, chunk: int = 0) -> np.random.Generator:
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, key, chunk])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Infinities pass through; NaN maps to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_tensor(seed: int, name: str, shape: Tuple[int, ...], std: float, dtype: str,
                   pool: Optional[ThreadPoolExecutor] = None) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)
    n_chunks = -(-n // CHUNK_ELEMS)

    def fill(c: int) -> None:
        lo, hi = c * CHUNK_ELEMS, min(n, (c + 1) * CHUNK_ELEMS)
        z = _rng(seed, name, c).standard_normal(hi - lo, dtype=np.float32)
        z *= np.float32(std)
        out[lo:hi] = f32_to_bf16_bits(z) if dtype == "bf16" else z

    if pool is not None and n_chunks > 1:
        list(pool.map(fill, range(n_chunks)))
    else:
        for c in range(n_chunks):
            fill(c)
    return out.reshape(shape)


def _ones(shape: Tuple[int, ...], dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return np.full(shape, 0x3F80, dtype=np.uint16)
    return np.ones(shape, dtype=np.float32)


# --------------------------------------------------------------------------
# model weights
# --------------------------------------------------------------------------
LAYER_TENSORS = ("attn_norm", "wqkv", "wo", "mlp_norm", "w_gate", "w_up", "w_down")


def layer_shapes(m: ModelShape) -> Dict[str, Tuple[int, ...]]:
    """Per-layer tensors. Projection matrices are stored [out, in] row-major."""
    d, f = m.d_model, m.ffn_dim
    return {
        "attn_norm": (d,),
        "wqkv": (3 * d, d),   # rows [0,d) -> q, [d,2d) -> k, [2d,3d) -> v
        "wo": (d, d),
        "mlp_norm": (d,),
        "w_gate": (f, d),
        "w_up": (f, d),
        "w_down": (d, f),
    }


def make_layer(m: ModelShape, layer: int, seed: int = 0,
               pool: Optional[ThreadPoolExecutor] = None) -> Dict[str, np.ndarray]:
    out = {}
    for name, shape in layer_shapes(m).items():
        if name.endswith("norm"):
            out[name] = _ones(shape, m.dtype)
        else:
            out[name] = _normal_tensor(seed, f"{m.name}.layer{layer}.{name}", shape,
                                       WEIGHT_STD, m.dtype, pool)
    return out


def make_embed(m: ModelShape, seed: int = 0, pool=None) -> np.ndarray:
    return _normal_tensor(seed, f"{m.name}.embed", (m.vocab, m.d_model), WEIGHT_STD, m.dtype, pool)


def make_lm_head(m: ModelShape, seed: int = 0, pool=None, scale: float = 1.0) -> np.ndarray:
    return _normal_tensor(seed, f"{m.name}.lm_head", (m.vocab, m.d_model), WEIGHT_STD * scale,
                          m.dtype, pool)


def make_final_norm(m: ModelShape) -> np.ndarray:
    return _ones((m.d_model,), m.dtype)


@dataclass
class ModelWeights:
    shape: ModelShape
    embed: np.ndarray
    layers: List[Dict[str, np.ndarray]]
    final_norm: np.ndarray
    lm_head: np.ndarray


def make_model(m: ModelShape, seed: int = 0, n_layers: Optional[int] = None,
               lm_head_scale: float = 1.0, threads: Optional[int] = None) -> ModelWeights:
    """All weights of a model (or of its first ``n_layers`` layers) on the host."""
    nl = m.n_layers if n_layers is None else n_layers
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(threads) as pool:
        embed = make_embed(m, seed, pool)
        layers = [make_layer(m, i, seed, pool) for i in range(nl)]
        head = make_lm_head(m, seed, pool, lm_head_scale)
    return ModelWeights(m, embed, layers, make_final_norm(m), head)


def make_hot_token_model(m: ModelShape, seed: int = 0, n_layers: Optional[int] = None, hot_tokens: int = 4,
                         hot_scale: float = 12.0, hot_seed: int = 0) -> ModelWeights:
    """A test fixture whose rows have clear top-1 tokens.

    The model is make_model's, except that the LM-head rows of hot_tokens token ids (drawn
    with hot_seed) are scaled by hot_scale (rounded to bf16 again for bf16 models): every
    row's largest logits come from those few ids, and its top-1 leads its top-2 by a
    sizeable fraction of the top-1 logit, far above the rounding of stored logits. The
    layers are unchanged, so the forward keeps the sensitivity of the plain fixture.
    """
    w = make_model(m, seed, n_layers)
    hot = np.random.default_rng(hot_seed).choice(m.vocab - 1, hot_tokens, replace=False)
    h = bf16_bits_to_f32(w.lm_head[hot]) if m.dtype == "bf16" else w.lm_head[hot]
    h = (h * np.float32(hot_scale)).astype(np.float32)
    w.lm_head[hot] = f32_to_bf16_bits(h) if m.dtype == "bf16" else h
    return w


# --------------------------------------------------------------------------
# sequences
# --------------------------------------------------------------------------
def make_prompt(cfg: DecodeConfig, seq: int = 0) -> np.ndarray:
    """Token ids [L]: prompt ids uniform on [0, V-1), then n_masked copies of mask_id = V-1."""
    m = cfg.model
    ids = _rng(cfg.seed, f"{cfg.name}.prompt{seq}").integers(0, m.vocab - 1, cfg.prompt_len,
                                                              dtype=np.int64)
    return np.concatenate([ids, np.full(cfg.n_masked, m.mask_id, dtype=np.int64)]).astype(np.int32)


# --------------------------------------------------------------------------
# stand-alone logits for the entropy reduction
# --------------------------------------------------------------------------
def make_entropy_logits(rows: int = ENTROPY_ROWS, vocab: int = ENTROPY_VOCAB, seed: int = 0,
                        dtype: str = "bf16") -> Tuple[np.ndarray, np.ndarray]:
    """Logits z / T with z ~ N(0,1) and a per-row temperature T, log-uniform on [0.05, 5].

    Small T gives sharp rows (entropy near 0), large T flat rows (near ln V).
    Returns (logits [rows, vocab] as bf16 bits or float32, temperatures [rows]).
    """
    lo, hi = ENTROPY_TEMP_RANGE
    t = np.exp(_rng(seed, "entropy.temp").uniform(math.log(lo), math.log(hi), rows))
    z = _rng(seed, "entropy.z").standard_normal((rows, vocab), dtype=np.float32)
    x = (z / t[:, None].astype(np.float32)).astype(np.float32)
    return (f32_to_bf16_bits(x) if dtype == "bf16" else x), t


def entropy_edge_rows(vocab: int, dtype: str = "bf16") -> Dict[str, np.ndarray]:
    """Rows with known entropies: flat, one-hot (-inf elsewhere), m-way ties, two-level."""
    neg_inf = np.float32(-np.inf)
    rows = {}
    rows["uniform"] = np.full(vocab, 0.75, dtype=np.float32)
    one = np.full(vocab, neg_inf, dtype=np.float32)
    one[vocab // 3] = 2.5
    rows["one_hot"] = one
    tie = np.full(vocab, neg_inf, dtype=np.float32)
    tie[[5, vocab // 2, vocab - 1, 17]] = 1.0
    rows["tie4"] = tie
    two = np.zeros(vocab, dtype=np.float32)
    two[: vocab // 8] = 3.0
    rows["two_level"] = two
    peak = np.zeros(vocab, dtype=np.float32)
    peak[vocab - 2] = 40.0
    rows["sharp"] = peak
    if dtype == "bf16":
        return {k: f32_to_bf16_bits(v) for k, v in rows.items()}
    return rows
