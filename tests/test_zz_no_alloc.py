"""GPU: the allocation-free entry point ec_entropy_max_noalloc against ec_entropy_max.

ec_entropy_max_noalloc is ec_entropy_max for callers that cannot allocate device memory
(its scratch is a device array of the library). Through the C ABI, two calls in a row on
the same stream, the second with a smaller input, must each give exactly the outputs of
ec_entropy_max on the same logits (the same kernel and slice plan: entropy, argmax,
confidence and E bit-identical), and the second call must not see anything the first
left in the shared array. (The host-side rejections are in tests/test_abi.py.)
"""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import bf16_tensor

pytestmark = pytest.mark.gpu


def _both(x, sel=None):
    import entropy_guided_kv_amd as ek
    a = ek.ec_entropy_max(x, sel=sel)
    b = ek.ec_entropy_max_noalloc(x, sel=sel)
    torch.cuda.synchronize()
    return [t.cpu() for t in a], [t.cpu() for t in b]


def _same(a, b):
    for u, v in zip(a, b):
        assert u.dtype == v.dtype and u.shape == v.shape
        assert torch.equal(u.view(torch.int32), v.view(torch.int32)), (u, v)


def test_noalloc_matches_workspace_entry_point_twice():
    bits, _ = synth.make_entropy_logits()              # 64 x 126464 bf16, the entropy workload
    big = bf16_tensor(bits)
    rng = np.random.default_rng(7)
    z = (rng.standard_normal((5, 3001)) * 3).astype(np.float32)
    z[2, 10] = np.nan
    small = torch.from_numpy(z).cuda()                 # fewer rows, shorter rows, one NaN row
    a, b = _both(big)
    _same(a, b)
    sel = torch.tensor([0, 3, 4], dtype=torch.int32, device="cuda")
    a, b = _both(small, sel=sel)
    _same(a, b)
    assert not np.isnan(b[3].item())                   # the NaN row is not selected
    a, b = _both(small)
    _same(a, b)
    assert np.isnan(b[3].item())
