"""GPU parity: ec_entropy_max against the oracle's entropy on identical logits.

Bars: argmax bit-exact (both sides compare the same stored values), entropy
within 1e-3 nats, max-probability within 1e-4 relative, E = max over the
selected rows.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle.entropy import entropy_rows
from oracle.model import bf16_bits_to_f64
from tests.gpu_util import bf16_tensor, to_f64

pytestmark = pytest.mark.gpu
H_TOL = 1e-3


def _check(logits_dev: torch.Tensor, logits_f64: np.ndarray, sel=None):
    import entropy_guided_kv_amd as ek
    H, a, c, e = ek.ec_entropy_max(logits_dev, sel=sel)
    torch.cuda.synchronize()
    h0, a0, c0 = entropy_rows(logits_f64)
    Hg, ag, cg = H.cpu().double().numpy(), a.cpu().numpy(), c.cpu().double().numpy()
    fin = ~np.isnan(h0)
    np.testing.assert_array_equal(np.isnan(Hg), ~fin)
    assert np.abs(Hg[fin] - h0[fin]).max(initial=0) <= H_TOL
    np.testing.assert_array_equal(ag[fin], a0[fin])
    np.testing.assert_allclose(cg[fin], c0[fin], rtol=1e-4, atol=1e-7)
    rows = np.arange(len(h0)) if sel is None else sel.cpu().numpy()
    want = np.nan if np.isnan(h0[rows]).any() else h0[rows].max()
    got = float(e.item())
    if math.isnan(want):
        assert math.isnan(got)
    else:
        assert abs(got - want) <= H_TOL
    return Hg, h0


def test_entropy_rows_at_full_size():
    """64 rows x V = 126464 bf16, per-row temperature log-uniform in [0.05, 5]."""
    bits, temps = synth.make_entropy_logits()
    x = bf16_tensor(bits)
    Hg, h0 = _check(x, bf16_bits_to_f64(bits))
    print(f"entropy range {h0.min():.4f} .. {h0.max():.4f} nats, max |dH| {np.abs(Hg - h0).max():.2e}")
    assert h0.min() < 0.1 and h0.max() > math.log(126464) - 0.1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_entropy_edge_rows(dtype):
    V = 126464
    rows = synth.entropy_edge_rows(V, dtype)
    names = list(rows)
    mat = np.stack([rows[n] for n in names])
    x = bf16_tensor(mat) if dtype == "bf16" else torch.from_numpy(mat).cuda()
    ref = bf16_bits_to_f64(mat) if dtype == "bf16" else mat.astype(np.float64)
    Hg, h0 = _check(x, ref)
    got = dict(zip(names, Hg))
    assert abs(got["uniform"] - math.log(V)) <= H_TOL
    assert abs(got["one_hot"]) <= 1e-6  # 0 up to the rounding of max * log2(e)
    assert abs(got["tie4"] - math.log(4)) <= H_TOL


@pytest.mark.parametrize("rows,V,stride_pad", [(1, 1, 0), (3, 7, 1), (5, 1000, 24), (17, 12345, 3),
                                               (2, 126464, 0), (128, 32000, 0), (0, 10, 0),
                                               (300, 2000, 0), (1000, 4096, 8)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_entropy_ragged_and_strided(rows, V, stride_pad, dtype):
    """Fewer than 256 rows split each row into slices that the last workgroup merges; 256
    rows or more take one workgroup per row, whose entropies the last workgroup gathers for
    E; a row pitch that is not a multiple of 16 bytes takes the element-wise path."""
    rng = np.random.default_rng(rows * 7 + V)
    z = (rng.standard_normal((rows, V + stride_pad)) * rng.uniform(0.1, 6, (rows, 1))).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(z)
        full = bf16_tensor(bits)
        ref = bf16_bits_to_f64(bits)[:, :V]
    else:
        full = torch.from_numpy(z).cuda()
        ref = z.astype(np.float64)[:, :V]
    x = full[:, :V]
    if rows == 0:
        import entropy_guided_kv_amd as ek
        H, a, c, e = ek.ec_entropy_max(x)
        assert e.item() == -math.inf
        return
    _check(x, ref)


def _random_entropy_cases(n=16, seed=77, max_elems=3e7):
    """(rows, V, row-pitch padding, dtype, with a selection) drawn from a fixed seed."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        rows, V = int(rng.integers(1, 700)), int(rng.integers(1, 150000))
        if rows * V > max_elems:
            continue
        pad = int(rng.choice([0, 0, 1, 3, 8, 24]))
        cases.append((rows, V, pad, ("bf16", "f32")[len(cases) % 2], bool(len(cases) % 4 >= 2)))
    return cases


@pytest.mark.parametrize("rows,V,pad,dtype,with_sel", _random_entropy_cases())
def test_entropy_seeded_random_shapes(rows, V, pad, dtype, with_sel):
    """Shapes off the hand-picked list (1 to 256 slices per row, one workgroup per row past 256
    rows, aligned and element-wise row pitches), with per-row temperatures and, for half of
    them, E over a random subset of the rows."""
    rng = np.random.default_rng(rows * 131 + V)
    z = (rng.standard_normal((rows, V + pad)) * rng.uniform(0.05, 6, (rows, 1))).astype(np.float32)
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(z)
        full, ref = bf16_tensor(bits), bf16_bits_to_f64(bits)[:, :V]
    else:
        full, ref = torch.from_numpy(z).cuda(), z.astype(np.float64)[:, :V]
    sel = None
    if with_sel:
        k = int(rng.integers(1, rows + 1))
        sel = torch.from_numpy(np.sort(rng.choice(rows, k, replace=False)).astype(np.int32)).cuda()
    _check(full[:, :V], ref, sel=sel)


def test_entropy_selected_rows_and_nan():
    rng = np.random.default_rng(3)
    z = (rng.standard_normal((6, 5000)) * 2).astype(np.float32)
    z[4, 17] = np.nan
    x = torch.from_numpy(z).cuda()
    sel = torch.tensor([0, 2, 5], dtype=torch.int32, device="cuda")
    _check(x, z.astype(np.float64), sel=sel)
    _check(x, z.astype(np.float64), sel=torch.tensor([1, 4], dtype=torch.int32, device="cuda"))


def test_entropy_deterministic():
    bits, _ = synth.make_entropy_logits(rows=8)
    import entropy_guided_kv_amd as ek
    x = bf16_tensor(bits)
    r1 = [t.cpu() for t in ek.ec_entropy_max(x)]
    r2 = [t.cpu() for t in ek.ec_entropy_max(x)]
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_entropy_row_with_a_whole_block_of_nan(dtype):
    """A NaN logit makes its row's entropy and confidence NaN even when a whole block of
    the row the reduction handles as one piece (2048 aligned columns cover every split the
    kernels use) holds nothing but NaN, or NaN and -inf: the block's maximum is then -inf
    and its sums are empty, so the NaN must travel as a flag. E over those rows is NaN."""
    V = 20000
    rng = np.random.default_rng(5)
    z = (rng.standard_normal((4, V)) * 2).astype(np.float32)
    z[0, 2048:4096] = np.nan
    z[1, 4096:6144] = np.nan
    z[1, 4096:6144:3] = -np.inf
    z[2, :] = -np.inf
    z[2, 8192:10240] = np.nan
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(z)
        x, ref = bf16_tensor(bits), bf16_bits_to_f64(bits)
    else:
        x, ref = torch.from_numpy(z).cuda(), z.astype(np.float64)
    Hg, h0 = _check(x, ref)
    assert np.isnan(Hg[:3]).all() and not np.isnan(Hg[3])
    _check(x, ref, sel=torch.tensor([3], dtype=torch.int32, device="cuda"))
