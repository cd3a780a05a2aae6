"""KV-drift measure (oracle) -- TEST INFRASTRUCTURE ONLY.

The pages measure how far the KV cache moves between consecutive denoising
steps as the cosine distance of the value vectors, and report that it tracks
the largest entropy among the tokens decoded in the step before (EntropyCache
explainer, Arabic technical summary, section 2, key observations; Italian
summary, section 2, observation 1). Here, for each row a step recomputes:
    dist = 1 - <old, new> / (|old| |new|)
with old = the vector cached before the step and new = the one the step writes,
for K and for V of every layer, in float64. Rows with a zero-norm old or new
vector (a cache never written) are left out of the per-layer mean and max; a
layer with no row left gives NaN.
"""
from __future__ import annotations

from typing import List, Sequence

import numpy as np


def cosine_distance_rows(old: np.ndarray, new: np.ndarray) -> np.ndarray:
    """1 - cos(old[i], new[i]) for every row i; NaN where either norm is zero."""
    old = np.asarray(old, dtype=np.float64)
    new = np.asarray(new, dtype=np.float64)
    dot = np.einsum("ij,ij->i", old, new)
    n0 = np.sqrt(np.einsum("ij,ij->i", old, old))
    n1 = np.sqrt(np.einsum("ij,ij->i", new, new))
    out = np.full(old.shape[0], np.nan)
    ok = (n0 > 0) & (n1 > 0)
    out[ok] = 1.0 - dot[ok] / (n0[ok] * n1[ok])
    return out


def summarize(dist: np.ndarray) -> np.ndarray:
    """(mean, max) over the rows with a defined distance; (NaN, NaN) if none."""
    v = dist[~np.isnan(dist)]
    if v.size == 0:
        return np.array([np.nan, np.nan])
    return np.array([v.mean(), v.max()])


def step_drift(cache_before: List[List[np.ndarray]], cache_after: List[List[np.ndarray]],
               rows: Sequence[int]) -> np.ndarray:
    """[n_layers, 4]: K mean, K max, V mean, V max of the recomputed rows' distances."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(cache_before), 4))
    for l, ((k0, v0), (k1, v1)) in enumerate(zip(cache_before, cache_after)):
        out[l, 0:2] = summarize(cosine_distance_rows(k0[rows], k1[rows]))
        out[l, 2:4] = summarize(cosine_distance_rows(v0[rows], v1[rows]))
    return out
