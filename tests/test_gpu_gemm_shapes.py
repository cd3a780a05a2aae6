"""GPU parity of the bf16 MFMA GEMM paths at the 8B layer width, through ec_forward.

One layer with d=4096, 32 heads of 128, SwiGLU width 12288 (the 8B-shaped
model's projection shapes) and a small vocabulary, so the oracle forward
stays fast. The row counts pick every tile configuration and split width the
GEMM planner uses on these shapes: 1024 rows (a refresh: 256x192 tiles for
q|k|v and gate/up, 128x128 for the output projection, 256x128 with two K
splits for down, reduced together with the next RMSNorm), 300 rows (256x128
q|k|v, output projection in two splits, down in four), 144 rows (all-rows
128x96 q|k|v and 256x96 gate/up, output projection in four splits, down in
eight), 48 rows (64x96 q|k|v in two splits, 64x64 output projection in four,
64x96 gate/up), 40 and 17 rows (64x128 output projection and down in eight
splits) and 1 row (q|k|v in eight splits as well).
Bars as in the other forward tests: 2e-2 relative per row for
hidden states, logits and the recomputed K/V rows, every other cache row
bit-identical, argmax exact where the logit margin clears the id gate.

Also: ec_pack_weights moves exactly the rows its layout definition names.
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import bf16_tensor
from tests.test_gpu_forward import _compare, _setup

pytestmark = pytest.mark.gpu

WIDE = synth.ModelShape("wide", "bf16", 1, 4096, 32, 128, 12288, 1024)


@pytest.mark.parametrize("n_rows", [1024, 300, 144, 48, 40, 17, 1])
def test_forward_at_8b_layer_width(n_rows):
    L = 1024
    w, omm, dm, cache, oc = _setup(WIDE, L, seed=11, stale=n_rows < L)
    rng = np.random.default_rng(12)
    tokens = rng.integers(0, WIDE.vocab - 1, L).astype(np.int32)
    rows = np.arange(L) if n_rows == L else np.sort(rng.choice(L, n_rows, replace=False))
    out = rows[np.sort(rng.choice(len(rows), min(len(rows), 32), replace=False))]
    _compare(WIDE, omm, dm, cache, oc, tokens, rows, out)


def _random_rows(n, lo, hi, seed):
    """Row counts drawn from a fixed seed over [lo, hi): other tile and split choices of the
    planner than the hand-picked counts above."""
    rng = np.random.default_rng(seed)
    return sorted(int(x) for x in rng.choice(np.arange(lo, hi), n, replace=False))


@pytest.mark.parametrize("n_rows", _random_rows(10, 2, 1024, 5150) + _random_rows(8, 2, 257, 5151))
def test_forward_at_8b_layer_width_seeded_rows(n_rows):
    L = 1024
    w, omm, dm, cache, oc = _setup(WIDE, L, seed=13, stale=True)
    rng = np.random.default_rng(n_rows)
    tokens = rng.integers(0, WIDE.vocab - 1, L).astype(np.int32)
    rows = np.sort(rng.choice(L, n_rows, replace=False))
    out = rows[np.sort(rng.choice(len(rows), min(len(rows), 32), replace=False))]
    _compare(WIDE, omm, dm, cache, oc, tokens, rows, out)


NARROW_FFN = synth.ModelShape("narrowffn", "bf16", 1, 2048, 16, 128, 512, 1024)


@pytest.mark.parametrize("n_rows", [40, 1])
def test_forward_split_k_swiglu(n_rows):
    """A layer whose packed gate/up matrix is short (2F = 1024 rows) against a deep K
    (d = 2048): the GEMM planner splits K four ways over 64x64 tiles, so the SwiGLU runs in
    the split-K reduction instead of the GEMM epilogue. Same bars as the other forward
    tests."""
    L = 256
    w, omm, dm, cache, oc = _setup(NARROW_FFN, L, seed=31, stale=True)
    rng = np.random.default_rng(32)
    tokens = rng.integers(0, NARROW_FFN.vocab - 1, L).astype(np.int32)
    rows = np.sort(rng.choice(L, n_rows, replace=False))
    _compare(NARROW_FFN, omm, dm, cache, oc, tokens, rows, rows[: min(n_rows, 16)])


WIDE13 = synth.ModelShape("wide13", "bf16", 1, 5120, 40, 128, 13824, 1024)


@pytest.mark.parametrize("n_rows", [256, 77])
def test_forward_wider_than_4096(n_rows):
    """A 13B-shaped layer (d = 5120, 40 heads, SwiGLU width 13824): rows wider than 4096
    take the RMSNorm form that holds eight float4 per thread, and the GEMM planner sees
    projection shapes it was not fitted on. Same bars as at the 8B width, argmax ids under
    the id gate (a margin of exactly two bf16 steps of top-1, as one sampled row of the
    77-row case has, is not above the gate)."""
    L = 256
    w, omm, dm, cache, oc = _setup(WIDE13, L, seed=21, stale=n_rows < L)
    rng = np.random.default_rng(22)
    tokens = rng.integers(0, WIDE13.vocab - 1, L).astype(np.int32)
    rows = np.arange(L) if n_rows == L else np.sort(rng.choice(L, n_rows, replace=False))
    out = rows[np.sort(rng.choice(len(rows), min(len(rows), 24), replace=False))]
    _compare(WIDE13, omm, dm, cache, oc, tokens, rows, out)


def _packed_qkv_order(d, D):
    """Row order of the packed q|k|v matrix: inside each head, group g of 32 rows is
    first-half rows 16g..16g+15 then their rotary partners D/2 + 16g .. D/2 + 16g + 15."""
    order = []
    for hb in range(0, 3 * d, D):
        for g in range(D // 32):
            order += [hb + 16 * g + i for i in range(16)]
            order += [hb + D // 2 + 16 * g + i for i in range(16)]
    return np.array(order)


@pytest.mark.parametrize("d,D,F,dtype", [(256, 128, 512, "bf16"), (4096, 128, 12288, "bf16"),
                                         (256, 64, 1024, "f32")])
def test_pack_weights_layout(d, D, F, dtype):
    from entropy_guided_kv_amd import api
    rng = np.random.default_rng(d + F)
    mk = lambda r: rng.standard_normal((r, d)).astype(np.float32)
    wqkv, wg, wu = mk(3 * d), mk(F), mk(F)
    if dtype == "bf16":
        dev = lambda a: bf16_tensor(synth.f32_to_bf16_bits(a))
        host = lambda a: synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a))
    else:
        dev = lambda a: torch.from_numpy(a).cuda()
        host = lambda a: a
    shape = synth.ModelShape("p", dtype, 1, d, d // D, D, F, 16)
    qp, gu = api.pack_weights(shape, dev(wqkv), dev(wg), dev(wu))
    torch.cuda.synchronize()
    got_q = qp.float().cpu().numpy()
    got_gu = gu.float().cpu().numpy()
    np.testing.assert_array_equal(got_q, host(wqkv)[_packed_qkv_order(d, D)])
    hg, hu = host(wg), host(wu)
    exp_gu = np.empty((2 * F, d), np.float32)
    for g in range(F // 16):
        exp_gu[32 * g: 32 * g + 16] = hg[16 * g: 16 * g + 16]
        exp_gu[32 * g + 16: 32 * g + 32] = hu[16 * g: 16 * g + 16]
    np.testing.assert_array_equal(got_gu, exp_gu)
    # a permutation: every plain row appears exactly once
    assert sorted(_packed_qkv_order(d, D).tolist()) == list(range(3 * d))
