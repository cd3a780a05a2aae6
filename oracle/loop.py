"""The EntropyCache denoising loop (oracle).

Per step t (EntropyCache explainer: Arabic technical summary, section 2,
"Algorithm workflow", three phases; Italian summary, "Algoritmo di
Funzionamento"):
  1. forward: full if the skip flag is off, otherwise partial over the
     still-masked positions plus the k most recently decoded positions
     (taken from a record of decode times), every other position reusing
     its cached K/V;
  2. decode new tokens from the logits and take E_{t+1}, the largest entropy
     among the newly decoded tokens' distributions;
  3. E_{t+1} > tau turns the skip flag off (full recompute next step);
     otherwise the next step is a partial one.

Readings where the pages are silent (each listed in the design notes):
  * the first step is always a full forward (no cache exists yet);
  * the flag is re-evaluated every step: refresh_next = E > tau, equality
    skips; a NaN E also forces a refresh;
  * every still-masked position is recomputed (not only the current block);
  * "k most recent" = the last k entries of an append-only decode log; the
    positions decoded in one step are appended in ascending order;
  * decoding is greedy argmax; the n tokens of a step are the candidates
    with the largest max-probability, ties to the lower position;
    candidates are the masked positions of the lowest block that still has
    a mask (semi-autoregressive blocks of length B);
  * confidence and E are compared in float32, the device's precision.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .drift import step_drift
from .entropy import entropy_rows
from .model import OracleModel, forward, new_cache


def candidates(masked: np.ndarray, prompt_len: int, block_len: int, window: bool = False) -> np.ndarray:
    """Masked positions of the lowest block [P + bB, P + (b+1)B) that still has a mask;
    with ``window``, the masked positions among the B positions from the lowest masked one
    (a sliding window, one of the decoding strategies the pages name: EntropyCache
    explainer, Italian summary, section 5)."""
    pos = np.flatnonzero(masked)
    if pos.size == 0:
        return pos
    if window:
        lo = int(pos[0])
    else:
        lo = prompt_len + ((int(pos[0]) - prompt_len) // block_len) * block_len
    hi = lo + block_len
    return pos[(pos >= lo) & (pos < hi)]


def select(cand: np.ndarray, conf32: np.ndarray, n: int) -> np.ndarray:
    """The min(n, len(cand)) candidates with the largest confidence, ties to the lower position.

    A NaN confidence ranks below every number. Returned in ascending position order.
    """
    key = lambda i: (-(float(conf32[i]) if conf32[i] == conf32[i] else -1.0), int(cand[i]))
    order = sorted(range(len(cand)), key=key)
    pick = [int(cand[i]) for i in order[: min(n, len(cand))]]
    return np.array(sorted(pick), dtype=np.int64)


def recompute_set(masked: np.ndarray, decode_log: List[int], k: int) -> np.ndarray:
    """Still-masked positions plus the last k entries of the decode log, ascending."""
    recent = decode_log[-k:] if k > 0 else []
    return np.array(sorted(set(np.flatnonzero(masked).tolist()) | set(recent)), dtype=np.int64)


@dataclass
class StepRecord:
    t: int
    refreshed: bool
    rows: np.ndarray          # positions recomputed this step
    cand: np.ndarray          # candidate positions
    entropy: np.ndarray       # float64 entropies of the candidates
    argmax: np.ndarray
    maxprob: np.ndarray
    margin: np.ndarray        # top-1 minus top-2 logit of each candidate row
    top1: np.ndarray          # top-1 logit of each candidate row
    picked: np.ndarray        # decoded positions, ascending
    ids: np.ndarray           # decoded token ids, same order
    emax: float               # E_{t+1} (float32 value)
    refresh_next: bool
    logits: Optional[np.ndarray] = None
    drift: Optional[np.ndarray] = None  # [n_layers, 4] KV drift of the recomputed rows (probe)


@dataclass
class DecodeState:
    tokens: np.ndarray
    masked: np.ndarray
    decode_log: List[int] = field(default_factory=list)
    t: int = 0
    refresh_next: bool = True


def init_state(cfg, prompt: np.ndarray) -> DecodeState:
    masked = np.zeros(cfg.seq_len, dtype=bool)
    masked[cfg.prompt_len:] = True
    return DecodeState(np.asarray(prompt, dtype=np.int64).copy(), masked)


def _top2_margin(logits: np.ndarray) -> np.ndarray:
    if logits.shape[1] < 2:
        return np.full(logits.shape[0], np.inf)
    part = np.sort(logits, axis=1)[:, -2:]
    return part[:, 1] - part[:, 0]


def step(model: OracleModel, cfg, st: DecodeState, cache, tau: float,
         keep_logits: bool = False, probe: bool = False) -> StepRecord:
    """One denoising step; mutates ``st`` and ``cache``. With ``probe`` the record also
    holds the KV drift of the recomputed rows (cache before vs after the forward)."""
    full = st.t == 0 or st.refresh_next
    if full:
        rows = np.arange(cfg.seq_len, dtype=np.int64)
    else:
        rows = recompute_set(st.masked, st.decode_log, cfg.k_recent)
    cand = candidates(st.masked, cfg.prompt_len, cfg.block_len, getattr(cfg, "window", False))
    before = [[k.copy(), v.copy()] for k, v in cache] if probe else None
    out = forward(model, st.tokens, rows, cache, out_rows=cand)
    logits = out["logits"]
    h, a, c = entropy_rows(logits)
    conf32 = c.astype(np.float32)
    picked = select(cand, conf32, cfg.tokens_per_step)
    where = {int(p): i for i, p in enumerate(cand)}
    ids = np.array([a[where[int(p)]] for p in picked], dtype=np.int64)
    for p, tok in zip(picked, ids):
        st.tokens[p] = tok
        st.masked[p] = False
        st.decode_log.append(int(p))
    hp = np.array([h[where[int(p)]] for p in picked])
    if hp.size == 0:
        emax = -math.inf
    elif np.isnan(hp).any():
        emax = math.nan
    else:
        emax = float(np.float32(hp.max()))
    st.refresh_next = bool(math.isnan(emax) or np.float32(emax) > np.float32(tau))
    rec = StepRecord(st.t, full, rows, cand, h, a, c, _top2_margin(logits), logits.max(axis=1),
                     picked, ids, emax, st.refresh_next, logits if keep_logits else None,
                     step_drift(before, cache, rows) if probe else None)
    st.t += 1
    return rec


def run_entropycache(model: OracleModel, cfg, prompt: np.ndarray, tau: float,
                     max_steps: Optional[int] = None, keep_logits: bool = False, probe: bool = False):
    """Run the loop until no mask remains (or ``max_steps``). Returns (records, state, cache)."""
    st = init_state(cfg, prompt)
    cache = new_cache(model, cfg.seq_len)
    recs = []
    while st.masked.any() and (max_steps is None or st.t < max_steps):
        recs.append(step(model, cfg, st, cache, tau, keep_logits, probe))
    return recs, st, cache


def run_vanilla(model: OracleModel, cfg, prompt: np.ndarray, max_steps: Optional[int] = None):
    """Vanilla denoising: a full forward from a fresh (empty) cache at every step."""
    st = init_state(cfg, prompt)
    recs = []
    while st.masked.any() and (max_steps is None or st.t < max_steps):
        cache = new_cache(model, cfg.seq_len)
        st.refresh_next = True
        recs.append(step(model, cfg, st, cache, tau=math.inf))
    return recs, st
