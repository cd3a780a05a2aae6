"""Decision signal: softmax entropy, argmax and confidence of a logit row.

The explainer pages define the signal as the largest entropy among the
distributions of the tokens decoded in the current step,
E_{t+1} = max over newly decoded i of ( -sum_j p_ij log p_ij ), with p_i the
softmax of row i over the whole vocabulary (Arabic technical summary, section
2, "Decode and evaluate entropy" equation; Italian summary, "Algoritmo di
Funzionamento" step 1). The log is natural (nats).

The decoding rule itself is not on the pages; greedy argmax per row with the
maximum softmax probability as confidence is the reading taken here.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np


def entropy_stats(row: np.ndarray) -> Tuple[float, int, float]:
    """(entropy in nats, argmax, max softmax probability) of one logit row.

    p_j = exp(x_j) / sum_k exp(x_k), evaluated as exp(x_j - max) / Z for range
    safety. Entries equal to -inf have p_j = 0 and add nothing to the entropy
    (0 log 0 = 0). The argmax is the lowest index holding the maximum. A row
    with no finite maximum, or any NaN, gives NaN entropy and confidence.
    """
    x = np.asarray(row, dtype=np.float64)
    if x.size == 0 or np.isnan(x).any():
        return float("nan"), 0, float("nan")
    m = x.max()
    idx = int(np.flatnonzero(x == m)[0])
    if not np.isfinite(m):
        return float("nan"), idx, float("nan")
    e = np.exp(x - m)
    z = e.sum()
    p = e / z
    live = p > 0
    logp = (x[live] - m) - math.log(z)
    h = float(-(p[live] * logp).sum())
    return h, idx, float(p[idx])


def entropy_rows(x: np.ndarray):
    """Row-wise ``entropy_stats`` for a [rows, V] array.

    Returns float64 entropies, int64 argmax and float64 max-probabilities.
    """
    x = np.asarray(x)
    n = x.shape[0]
    h = np.empty(n)
    a = np.empty(n, dtype=np.int64)
    c = np.empty(n)
    for i in range(n):
        h[i], a[i], c[i] = entropy_stats(x[i])
    return h, a, c


def max_entropy(h: np.ndarray, chosen=None) -> float:
    """E = max of the entropies of the chosen rows (all rows if ``chosen`` is None).

    NaN anywhere among them makes E NaN.
    """
    h = np.asarray(h, dtype=np.float64)
    if chosen is not None:
        h = h[np.asarray(chosen, dtype=np.int64)]
    if h.size == 0:
        return float("-inf")
    if np.isnan(h).any():
        return float("nan")
    return float(h.max())
