"""Pins for oracle.entropy against closed forms, a library routine and constructed cases.

The signal is the max over newly decoded rows of the softmax entropy in nats
(EntropyCache explainer, Arabic technical summary section 2, the E_{t+1}
equation). Each test below would fail on a plausible mistake: a dropped
normaliser, a wrong log base, a sign error, an argmax that keeps the last of
equal maxima, or mishandled -inf entries.
"""
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle.entropy import entropy_rows, entropy_stats, max_entropy


@pytest.mark.parametrize("V", [1, 2, 7, 1024, 126464])
def test_uniform_row_is_ln_v(V):
    h, a, c = entropy_stats(np.full(V, -3.25))
    assert abs(h - math.log(V)) < 1e-12 * max(1.0, math.log(V))
    assert a == 0
    assert abs(c - 1.0 / V) < 1e-15


def test_one_hot_is_zero():
    x = np.full(1000, -np.inf)
    x[417] = 3.0
    h, a, c = entropy_stats(x)
    assert h == 0.0 and a == 417 and c == 1.0


@pytest.mark.parametrize("m", [2, 3, 5, 64])
def test_m_equal_maxima_is_ln_m(m):
    rng = np.random.default_rng(m)
    x = np.full(500, -np.inf)
    pos = np.sort(rng.choice(500, m, replace=False))
    x[pos] = 1.5
    h, a, c = entropy_stats(x)
    assert abs(h - math.log(m)) < 1e-13
    assert a == pos[0]
    assert abs(c - 1.0 / m) < 1e-15


@pytest.mark.parametrize("n1,n2,a,b", [(1, 99, 2.0, 0.0), (10, 1014, 3.0, -1.0), (500, 500, 0.25, 0.0)])
def test_two_level_closed_form(n1, n2, a, b):
    x = np.concatenate([np.full(n1, a), np.full(n2, b)])
    z = n1 * math.exp(a) + n2 * math.exp(b)
    p1, p2 = math.exp(a) / z, math.exp(b) / z
    want = -(n1 * p1 * math.log(p1) + n2 * p2 * math.log(p2))
    h, idx, c = entropy_stats(x)
    assert abs(h - want) < 1e-12
    assert idx == (0 if a >= b else n1)
    assert abs(c - max(p1, p2)) < 1e-15


def test_random_rows_match_scipy():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((16, 3000)) * rng.uniform(0.05, 8.0, (16, 1))
    h, a, c = entropy_rows(x)
    p = scipy.special.softmax(x, axis=1)
    want = scipy.stats.entropy(p, axis=1)
    np.testing.assert_allclose(h, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(a, np.argmax(x, axis=1))
    np.testing.assert_allclose(c, np.exp(x.max(1) - scipy.special.logsumexp(x, axis=1)), rtol=1e-13)


def test_argmax_keeps_lowest_of_equal_maxima():
    x = np.zeros(50)
    x[[31, 7, 44]] = 2.0
    assert entropy_stats(x)[1] == 7


def test_shift_invariance_and_sharpening():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(777)
    h0 = entropy_stats(x)[0]
    assert abs(entropy_stats(x + 123.5)[0] - h0) < 1e-11
    hs = [entropy_stats(x * beta)[0] for beta in (0.5, 1.0, 2.0, 4.0)]
    assert all(hs[i] > hs[i + 1] for i in range(3))


def test_gaussian_logits_entropy_near_ln_v_minus_half_sigma_squared():
    # For V i.i.d. N(0, s^2) logits with small s, H ~= ln V - s^2/2 (second-order expansion).
    rng = np.random.default_rng(2)
    V, s = 200000, 0.3
    h = entropy_stats(rng.standard_normal(V) * s)[0]
    assert abs(h - (math.log(V) - s * s / 2)) < 2e-3


def test_nan_and_empty_rows():
    x = np.zeros(10)
    x[3] = np.nan
    h, _, c = entropy_stats(x)
    assert math.isnan(h) and math.isnan(c)
    h, _, _ = entropy_stats(np.full(8, -np.inf))
    assert math.isnan(h)


def test_max_entropy_over_chosen_rows():
    h = np.array([0.1, 2.0, 0.7, 5.0])
    assert max_entropy(h) == 5.0
    assert max_entropy(h, [0, 2]) == 0.7
    assert math.isnan(max_entropy(np.array([0.1, np.nan]), [0, 1]))
    assert max_entropy(h, []) == -math.inf
