"""GPU parity: ec_cache_scatter (bit-exact) and ec_partial_attn against the oracle.

Attention: every query row attends over all L cached rows with no mask
(EntropyCache explainer, Italian summary section 1). bf16 bar: 2e-2 relative
per row (probabilities enter the P.V product as bf16); f32 bar: 1e-5.
"""
import math

import numpy as np
import pytest
import torch

from oracle.model import attention, round_bf16
from tests.gpu_util import row_rel_err, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("L,width,n", [(1024, 4096, 143), (512, 2048, 1), (128, 256, 128), (97, 24, 13),
                                     (64, 128, 0)])
def test_cache_scatter_bit_exact(dtype, L, width, n):
    import entropy_guided_kv_amd as ek
    g = torch.Generator().manual_seed(L + n)
    kc = torch.randn(L, width, generator=g).to(dtype).cuda()
    vc = torch.randn(L, width, generator=g).to(dtype).cuda()
    kr = torch.randn(n, width, generator=g).to(dtype).cuda()
    vr = torch.randn(n, width, generator=g).to(dtype).cuda()
    idx = torch.randperm(L, generator=g)[:n].to(torch.int32).cuda()
    k0, v0 = kc.clone(), vc.clone()
    ek.ec_cache_scatter(kc, vc, kr, vr, idx)
    torch.cuda.synchronize()
    untouched = torch.ones(L, dtype=torch.bool)
    untouched[idx.long().cpu()] = False
    assert torch.equal(kc[untouched.cuda()], k0[untouched.cuda()])
    assert torch.equal(vc[untouched.cuda()], v0[untouched.cuda()])
    assert torch.equal(kc[idx.long()], kr) and torch.equal(vc[idx.long()], vr)


def test_cache_scatter_skips_out_of_range_rows():
    import entropy_guided_kv_amd as ek
    kc = torch.zeros(16, 256, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kr = torch.ones(3, 256, dtype=torch.bfloat16, device="cuda")
    idx = torch.tensor([2, 16, -1], dtype=torch.int32, device="cuda")
    ek.ec_cache_scatter(kc, vc, kr, kr.clone(), idx)
    torch.cuda.synchronize()
    assert kc[2].float().sum().item() == 256 and kc.float().sum().item() == 256


def _attn_case(r, L, H, D, dtype, seed=0, scale=1.0, misalign=False):
    import entropy_guided_kv_amd as ek
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((r, H * D)) * scale
    k = rng.standard_normal((L, H * D)) * scale
    v = rng.standard_normal((L, H * D))
    if dtype == torch.bfloat16:
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    dev = [torch.from_numpy(a.astype(np.float32)).to(dtype).cuda() for a in (q, k, v)]
    if misalign:  # the same values one element past a 16-byte boundary
        def shift(t):
            buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
            view = buf[1:].view(t.shape)
            view.copy_(t)
            return view
        dev = [shift(t) for t in dev]
    out = ek.ec_partial_attn(dev[0], dev[1], dev[2], H, D)
    torch.cuda.synchronize()
    want = attention(q.reshape(r, H, D), k.reshape(L, H, D), v.reshape(L, H, D)).reshape(r, H * D)
    return to_f64(out), want


# bf16 cases; with the launch planner of the library (ec_partial_attn_plan) they take:
#   64-query workgroups, whole key range: (256, 1024, 32), (128, 128, 1), (100, 97, 8) and
#     (150, 65, 4) (a 128-key tile over a cache of 97 or 65 rows: its last 32-key quarter, or
#     last two, see one key or none, whose softmax terms must be 0);
#   64-query workgroups with 2 .. 16 key splits: (147, 1024, 32), (257, 512, 3), (17, 1024, 32),
#     (64, 1024, 32), (143, 1024, 4), (1024, 1024, 2), (96, 900, 24), (65, 1025, 32),
#     (1, 1025, 32) and (70, 2500, 2) (ragged last tiles), (33, 4096, 2);
#   128-query workgroups, whole key range: (1024, 1024, 32), (4, 1, 2), (7, 29, 3), (1, 33, 1)
#     (caches of 1, 29 and 33 rows: the upper-key wavefront of the only tile sees no key or
#     one);
#   128-query workgroups with 4 .. 16 key splits: (200, 1800, 24), (200, 4096, 32), (17, 1000, 2),
#     (40, 700, 8), (1, 1024, 2) and, one per merge width, (1, 769, 1), (1, 1025, 1), (3, 1250, 2),
#     (5, 1400, 3), (2, 768, 1), (1, 1600, 1), (1, 1700, 1), (1, 1800, 1) (most with a ragged last
#     tile).
# test_abi.py::test_bf16_attention_cases_cover_both_shapes checks this coverage on the host.
BF16_ATTN_CASES = [(147, 1024, 32), (256, 1024, 32), (257, 512, 3), (128, 128, 1), (100, 97, 8), (150, 65, 4),
                   (200, 1800, 24), (17, 1024, 32), (64, 1024, 32), (143, 1024, 4), (1024, 1024, 2),
                   (96, 900, 24), (65, 1025, 32), (1, 1025, 32), (70, 2500, 2), (33, 4096, 2),
                   (1024, 1024, 32), (4, 1, 2), (7, 29, 3), (1, 33, 1),
                   (200, 4096, 32), (17, 1000, 2), (40, 700, 8), (1, 1024, 2),
                   (1, 769, 1), (1, 1025, 1), (3, 1250, 2), (5, 1400, 3), (2, 768, 1), (1, 1600, 1),
                   (1, 1700, 1), (1, 1800, 1)]


@pytest.mark.parametrize("r,L,H", BF16_ATTN_CASES)
def test_partial_attn_bf16(r, L, H):
    got, want = _attn_case(r, L, H, 128, torch.bfloat16, seed=r + L, scale=0.35)
    err = row_rel_err(got.reshape(r * H, 128), want.reshape(r * H, 128))
    print(f"r={r} L={L} H={H}: max row rel err {err:.2e}")
    assert err < 2e-2


def _random_bf16_cases(n=24, seed=2024, max_work=2.5e7):
    """(r, L, H) drawn from a fixed seed: r in [1, 700), L in [1, 3000), H among 1 .. 32, with
    r L H bounded so that the oracle stays fast."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        r, L = int(rng.integers(1, 700)), int(rng.integers(1, 3000))
        H = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 32]))
        if r * L * H <= max_work:
            cases.append((r, L, H))
    return cases


@pytest.mark.parametrize("r,L,H", _random_bf16_cases())
def test_partial_attn_bf16_seeded_random_shapes(r, L, H):
    """Shapes off the hand-picked list: both workgroup shapes, 1 .. 16 key splits, ragged query
    tiles and key tiles (the plans they take: 64 queries per workgroup with 1 .. 7, 9 or 11
    splits, 128 with 1, 4, 7, 8, 11 or 16)."""
    got, want = _attn_case(r, L, H, 128, torch.bfloat16, seed=7 * r + L, scale=0.35)
    assert row_rel_err(got.reshape(r * H, 128), want.reshape(r * H, 128)) < 2e-2


@pytest.mark.parametrize("r,L,H,D", [(32, 128, 4, 64), (45, 300, 3, 64), (70, 1000, 2, 128), (1, 33, 1, 32),
                                     (5, 300, 2, 16), (1, 1, 1, 8)])
def test_partial_attn_f32(r, L, H, D):
    """head_dim 32, 64 and 128 run on the matrix unit (ragged query tiles and key blocks
    past L masked), other head sizes on the one-workgroup-per-query kernel."""
    got, want = _attn_case(r, L, H, D, torch.float32, seed=3)
    assert row_rel_err(got.reshape(r * H, D), want.reshape(r * H, D)) < 1e-5


def test_partial_attn_f32_unaligned_rows():
    """Operands 4 bytes off a 16-byte boundary take the one-workgroup-per-query kernel
    (the matrix-unit kernel reads 16-byte row pieces)."""
    r, L, H, D = 32, 128, 4, 64
    got, want = _attn_case(r, L, H, D, torch.float32, seed=3, misalign=True)
    assert row_rel_err(got.reshape(r * H, D), want.reshape(r * H, D)) < 1e-5


def test_partial_attn_sharp_softmax_bf16():
    # large logits: the online max rescaling across key tiles and splits must be exact
    got, want = _attn_case(40, 2048, 2, 128, torch.bfloat16, seed=9, scale=1.6)
    assert row_rel_err(got.reshape(80, 128), want.reshape(80, 128)) < 2e-2
