"""Pins of the oracle's KV-drift measure (cosine distance of cached vs recomputed rows).

Closed forms: identical or positively scaled vectors are at distance 0, opposite
ones at 2, orthogonal ones at 1, vectors 60 degrees apart at 1/2; a zero vector
has no direction and is left out of the per-layer summary.
"""
import math

import numpy as np

from oracle.drift import cosine_distance_rows, step_drift, summarize


def test_closed_forms():
    a = np.array([[1.0, 2.0, -3.0]] * 4)
    b = np.stack([a[0], -a[0], [2.0, -1.0, 0.0], 3.5 * a[0]])
    d = cosine_distance_rows(a, b)
    np.testing.assert_allclose(d, [0.0, 2.0, 1.0, 0.0], atol=1e-15)
    # 60 degrees: 1 - cos(pi/3) = 1/2
    u = np.array([[1.0, 0.0]])
    v = np.array([[math.cos(math.pi / 3), math.sin(math.pi / 3)]])
    np.testing.assert_allclose(cosine_distance_rows(u, v), [0.5], atol=1e-15)


def test_random_matches_angle_definition():
    rng = np.random.default_rng(0)
    x, y = rng.standard_normal((50, 64)), rng.standard_normal((50, 64))
    ang = np.array([math.acos(np.clip(np.dot(p, q) / np.linalg.norm(p) / np.linalg.norm(q), -1, 1))
                    for p, q in zip(x, y)])
    np.testing.assert_allclose(cosine_distance_rows(x, y), 1 - np.cos(ang), atol=1e-12)
    # symmetric and invariant under positive scaling of either side
    np.testing.assert_allclose(cosine_distance_rows(y, x), cosine_distance_rows(x, y), atol=1e-15)
    np.testing.assert_allclose(cosine_distance_rows(3 * x, 0.25 * y), cosine_distance_rows(x, y), atol=1e-12)


def test_zero_rows_are_left_out():
    old = np.array([[0.0, 0.0], [1.0, 0.0], [1.0, 1.0]])
    new = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    d = cosine_distance_rows(old, new)
    assert math.isnan(d[0]) and d[1] == 1.0 and abs(d[2]) < 1e-15
    np.testing.assert_allclose(summarize(d), [0.5, 1.0])
    assert np.isnan(summarize(np.array([np.nan, np.nan]))).all()


def test_step_drift_layers_and_rows():
    rng = np.random.default_rng(1)
    L, d = 10, 8
    before = [[rng.standard_normal((L, d)), rng.standard_normal((L, d))] for _ in range(2)]
    after = [[k.copy(), v.copy()] for k, v in before]
    rows = [2, 5, 7]
    after[0][1][5] = -before[0][1][5]          # layer 0, V of row 5 flipped: distance 2
    after[1][0][[2, 5, 7]] *= 4.0               # layer 1, K rescaled: distance 0
    after[1][1][3] = rng.standard_normal(d)     # a row outside the set: not measured
    out = step_drift(before, after, rows)
    np.testing.assert_allclose(out[0], [0.0, 0.0, 2.0 / 3.0, 2.0], atol=1e-12)
    np.testing.assert_allclose(out[1], [0.0, 0.0, 0.0, 0.0], atol=1e-12)
