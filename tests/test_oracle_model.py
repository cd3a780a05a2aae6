"""Pins for oracle.model: format rounding, building blocks and the cached forward.

The forward's structure (bidirectional attention over every cached row,
partial recompute of a row subset against stale K/V, full refresh) follows the
EntropyCache explainer (Arabic technical summary, section 2, phase 1; Italian
summary, "Algoritmo di Funzionamento"). The pins are closed forms, library
routines (torch CPU) and a scalar-loop brute force on tiny shapes.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from tests import bruteforce


# ---------------------------------------------------------------- formats
def test_round_bf16_known_values():
    one = 1.0
    assert om.round_bf16(np.array([one + 2 ** -8]))[0] == 1.0               # tie -> even (down)
    assert om.round_bf16(np.array([one + 3 * 2 ** -8]))[0] == 1 + 2 ** -6   # tie -> even (up)
    assert om.round_bf16(np.array([one + 2 ** -8 + 2 ** -20]))[0] == 1 + 2 ** -7
    assert om.round_bf16(np.array([-(one + 2 ** -8 + 2 ** -20)]))[0] == -(1 + 2 ** -7)
    assert om.round_bf16(np.array([0.0]))[0] == 0.0
    assert om.round_bf16(np.array([np.inf]))[0] == np.inf
    assert math.isnan(om.round_bf16(np.array([np.nan]))[0])
    big = om.round_bf16(np.array([3.0e38]))[0]
    assert np.isfinite(big) and abs(big / 3.0e38 - 1) <= 2 ** -9


def test_round_bf16_matches_bit_rounding_of_float32():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    want = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x)).astype(np.float64)
    np.testing.assert_array_equal(om.round_bf16(x.astype(np.float64)), want)


# ---------------------------------------------------------------- blocks
def test_rmsnorm_closed_form():
    rng = np.random.default_rng(1)
    h = rng.standard_normal((5, 64)) * 3.0
    out = om.rmsnorm(h, np.ones(64), 0.0)
    np.testing.assert_allclose(np.sqrt((out ** 2).mean(1)), 1.0, rtol=1e-14)
    x = np.full((1, 4), 2.0)
    g = np.array([1.0, 2.0, 3.0, 4.0])
    np.testing.assert_allclose(om.rmsnorm(x, g, 0.5)[0], 2.0 / math.sqrt(4.5) * g, rtol=1e-15)


def test_rope_identity_at_zero_and_norm_preserving():
    rng = np.random.default_rng(2)
    u = rng.standard_normal((3, 2, 16))
    np.testing.assert_array_equal(om.rope(u, np.zeros(3), 10000.0), u)
    out = om.rope(u, np.array([1, 77, 4095]), 10000.0)
    pair = lambda a: a[..., :8] ** 2 + a[..., 8:] ** 2
    np.testing.assert_allclose(pair(out), pair(u), rtol=1e-12)


def test_rope_relative_position_and_complex_form():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 8))
    k = rng.standard_normal((1, 1, 8))
    dot = lambda p1, p2: float((om.rope(q, np.array([p1]), 1e4) * om.rope(k, np.array([p2]), 1e4)).sum())
    assert abs(dot(5, 2) - dot(105, 102)) < 1e-11
    assert abs(dot(5, 2) - dot(2, 5)) > 1e-6   # depends on the signed difference
    # complex restatement: z_i = u_i + 1j*u_{i+D/2}, rotated by exp(1j * p * base^(-2i/D))
    p = 37
    z = q[0, 0, :4] + 1j * q[0, 0, 4:]
    zr = z * np.exp(1j * p * 10000.0 ** (-2.0 * np.arange(4) / 8))
    np.testing.assert_allclose(om.rope(q, np.array([p]), 1e4)[0, 0], np.concatenate([zr.real, zr.imag]),
                               rtol=1e-13, atol=1e-14)


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((7, 3, 16))
    K = rng.standard_normal((29, 3, 16))
    V = rng.standard_normal((29, 3, 16))
    got = om.attention(q, K, V)
    tq, tk, tv = (torch.from_numpy(a).permute(1, 0, 2).contiguous() for a in (q, K, V))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def _rounded_weight_attention_loops(q, K, V, rnd, extra):
    """Scalar restatement: weights e^s / 2^M' against M' = (smallest integer >= max s log2 e)
    + extra, rounded by rnd where they multiply V, normalised by the unrounded sum."""
    r, H, D = q.shape
    out = np.zeros_like(q)
    for i in range(r):
        for h in range(H):
            s = [float(np.dot(q[i, h], K[j, h])) / math.sqrt(D) for j in range(K.shape[0])]
            M = math.ceil(max(s) / math.log(2.0)) + extra
            w = [math.exp(x - M * math.log(2.0)) for x in s]
            for e in range(D):
                out[i, h, e] = sum(rnd(w[j]) * V[j, h, e] for j in range(len(w))) / sum(w)
    return out


def test_attention_rounded_weights_independent_of_reference_and_bounded():
    """bf16 attention weights (reading: rounded as 2^(t - M), M integer): the result must not
    depend on which integer M is taken (the device moves its reference by integers, per tile),
    must lie within 2^-8 max|v| of the exact softmax (bf16 unit roundoff 2^-8 on each weight),
    must equal a scalar-loop restatement, and without rounding must equal softmax exactly."""
    rng = np.random.default_rng(11)
    q = om.round_bf16(rng.standard_normal((5, 2, 8)) * 2.0)
    K = om.round_bf16(rng.standard_normal((23, 2, 8)) * 2.0)
    V = om.round_bf16(rng.standard_normal((23, 2, 8)))
    got = om.attention(q, K, V, round_weights=om.round_bf16)
    rnd1 = lambda x: float(om.round_bf16(np.array(x)))
    for extra in (0, 3, 40):
        np.testing.assert_allclose(got, _rounded_weight_attention_loops(q, K, V, rnd1, extra),
                                   rtol=1e-13, atol=1e-15)
    exact = om.attention(q, K, V)
    for h in range(2):
        assert np.abs(got[:, h] - exact[:, h]).max() <= 2.0 ** -8 * np.abs(V[:, h]).max()
    assert np.abs(got - exact).max() > 0  # the rounding is really applied
    np.testing.assert_allclose(om.attention(q, K, V, round_weights=lambda w: w), exact, rtol=1e-13, atol=1e-15)


def test_silu_matches_torch():
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(om.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(),
                               rtol=1e-14, atol=1e-300)


# ---------------------------------------------------------------- forward
BF_SHAPE = synth.ModelShape("bf", "f32", 2, 8, 2, 4, 12, 10)
BF_SHAPE_BF16 = synth.ModelShape("bfh", "bf16", 2, 8, 2, 4, 12, 10)


def _nested(w, dtype):
    f = lambda a: om.to_f64(a, dtype).tolist()
    return {
        "embed": f(w.embed),
        "layers": [{k: f(v) for k, v in lw.items()} for lw in w.layers],
        "final_norm": f(w.final_norm),
        "lm_head": f(w.lm_head),
    }


def _scaled_model(shape, scale=8.0):
    # larger weights than N(0, 0.02) so attention is far from uniform and every term matters
    w = synth.make_model(shape, seed=5)
    if shape.dtype == "f32":
        w.embed = w.embed * scale
        w.layers = [{k: (v * scale if not k.endswith("norm") else v) for k, v in lw.items()} for lw in w.layers]
        w.lm_head = w.lm_head * scale
    return w


@pytest.mark.parametrize("rows_kind", ["full", "partial"])
def test_forward_matches_scalar_bruteforce(rows_kind):
    w = _scaled_model(BF_SHAPE)
    m = om.OracleModel(w)
    L = 6
    tokens = np.array([3, 1, 4, 1, 5, 9])
    rng = np.random.default_rng(6)
    cache = om.new_cache(m, L)
    for K, V in cache:                      # deliberately stale cache contents
        K[:] = rng.standard_normal(K.shape)
        V[:] = rng.standard_normal(V.shape)
    bf_cache = [[K.tolist(), V.tolist()] for K, V in cache]
    rows = np.arange(L) if rows_kind == "full" else np.array([1, 4])
    out = om.forward(m, tokens, rows, cache)
    h_bf, lg_bf = bruteforce.forward(_nested(w, "f32"), tokens.tolist(), rows.tolist(), bf_cache, 2)
    np.testing.assert_allclose(out["hidden"], np.array(h_bf), rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(out["logits"], np.array(lg_bf), rtol=1e-11, atol=1e-12)
    for li in range(2):
        np.testing.assert_allclose(cache[li][0], np.array(bf_cache[li][0]), rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(cache[li][1], np.array(bf_cache[li][1]), rtol=1e-11, atol=1e-12)


def test_forward_bf16_mirror_matches_scalar_bruteforce():
    w = synth.make_model(BF_SHAPE_BF16, seed=7)
    m = om.OracleModel(w)
    assert m.mirror
    L = 5
    tokens = np.array([2, 7, 1, 8, 2])
    cache = om.new_cache(m, L)
    bf_cache = [[K.tolist(), V.tolist()] for K, V in cache]
    rnd32 = lambda v: float(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.array([v], np.float32)))[0])
    out = om.forward(m, tokens, np.arange(L), cache)
    h_bf, lg_bf = bruteforce.forward(_nested(w, "bf16"), tokens.tolist(), list(range(L)), bf_cache, 2, rnd=rnd32)
    # every stored value is a bf16 value; they agree except where fp32 double rounding differs
    np.testing.assert_allclose(out["logits"], np.array(lg_bf), rtol=1e-2, atol=1e-5)
    np.testing.assert_allclose(out["hidden"], np.array(h_bf), rtol=1e-3, atol=1e-6)
    assert np.all(om.round_bf16(cache[0][0]) == cache[0][0])


def test_partial_over_all_rows_equals_full_and_idempotence():
    w = _scaled_model(BF_SHAPE, scale=4.0)
    m = om.OracleModel(w)
    tokens = np.array([3, 1, 4, 1, 5, 9, 2, 6])
    L = len(tokens)
    c_full = om.new_cache(m, L)
    full = om.forward_full(m, tokens, c_full)
    c_all = om.new_cache(m, L)
    part_all = om.forward_partial(m, tokens, np.arange(L), c_all)
    np.testing.assert_array_equal(full["logits"], part_all["logits"])
    # right after a refresh on the same tokens, a partial step reproduces the full forward's rows
    rows = np.array([0, 5, 6])
    c2 = [[K.copy(), V.copy()] for K, V in c_full]
    part = om.forward_partial(m, tokens, rows, c2)
    np.testing.assert_allclose(part["hidden"], full["hidden"][rows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(part["logits"], full["logits"][rows], rtol=1e-12, atol=1e-13)
    for li in range(2):
        np.testing.assert_allclose(c2[li][0], c_full[li][0], rtol=1e-12, atol=1e-13)


def test_partial_reads_stale_rows():
    # after changing a token that is NOT recomputed, the partial result must differ from a full forward
    w = _scaled_model(BF_SHAPE, scale=4.0)
    m = om.OracleModel(w)
    tokens = np.array([3, 1, 4, 1, 5, 9, 2, 6])
    c = om.new_cache(m, len(tokens))
    om.forward_full(m, tokens, c)
    t2 = tokens.copy()
    t2[2] = 7
    rows = np.array([5, 6])
    part = om.forward_partial(m, t2, rows, [[K.copy(), V.copy()] for K, V in c])
    fresh = om.forward_full(m, t2, om.new_cache(m, len(tokens)))
    assert np.abs(part["logits"] - fresh["logits"][rows]).max() > 1e-6
    # and equals a forward over the original tokens for those rows (row 2 was never refreshed)
    same = om.forward_partial(m, tokens, rows, [[K.copy(), V.copy()] for K, V in c])
    np.testing.assert_allclose(part["logits"], same["logits"], rtol=1e-12, atol=1e-13)
