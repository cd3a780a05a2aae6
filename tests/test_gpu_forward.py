"""GPU parity: ec_forward (full and partial) against the oracle's forward.

A refresh step is the forward over every position; a skip step recomputes only
the listed rows against the cached (stale) K/V of the others (EntropyCache
explainer, Arabic technical summary section 2, phase 1). Bars: fp32 models
1e-5 relative (per row) for hidden states, cached K/V and logits; bf16 models
2e-2 relative, with argmax ids bit-exact wherever the top-1/top-2 logit
margin exceeds 1e-2.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import model as om
from oracle.entropy import entropy_rows
from tests.gpu_util import f64_to_bf16_tensor, margin_gate, rel_err, row_rel_err, to_f64

pytestmark = pytest.mark.gpu

MINI_BF16 = synth.ModelShape("mini", "bf16", 2, 256, 2, 128, 512, 1024)


def _tol(shape):
    return 1e-5 if shape.dtype == "f32" else 2e-2


def _setup(shape, L, seed=0, n_layers=None, stale=True):
    from entropy_guided_kv_amd import api
    w = synth.make_model(shape, seed=seed, n_layers=n_layers)
    om_model = om.OracleModel(w)
    dm = api.DeviceModel.from_host(w, rope_max_pos=L)
    cache = api.KVCache(dm, L)
    ocache = om.new_cache(om_model, L)
    if stale:
        rng = np.random.default_rng(seed + 1)
        for li in range(len(w.layers)):
            for j in range(2):
                vals = rng.standard_normal((L, shape.d_model)) * 0.5
                if shape.dtype == "bf16":
                    vals = om.round_bf16(vals)
                ocache[li][j][:] = vals
                tgt = cache.k[li] if j == 0 else cache.v[li]
                src = f64_to_bf16_tensor(vals) if shape.dtype == "bf16" else torch.from_numpy(vals).float().cuda()
                tgt.copy_(src)
    return w, om_model, dm, cache, ocache


def _compare(shape, om_model, dm, cache, ocache, tokens, rows, out_pos, check_ids=True):
    from entropy_guided_kv_amd import api
    L = len(tokens)
    where = {int(p): i for i, p in enumerate(rows)}
    out_idx = np.array([where[int(p)] for p in out_pos], dtype=np.int32)
    logits, hidden = api.ec_forward(dm, cache, torch.from_numpy(tokens).cuda(),
                                    torch.from_numpy(np.asarray(rows, np.int32)).cuda(),
                                    torch.from_numpy(out_idx).cuda(), want_hidden=True)
    torch.cuda.synchronize()
    ref = om.forward(om_model, tokens, rows, ocache, out_rows=out_pos)
    tol = _tol(shape)
    eh = row_rel_err(to_f64(hidden), ref["hidden"])
    el = row_rel_err(to_f64(logits), ref["logits"])
    ek = max(rel_err(to_f64(cache.k[i]), ocache[i][0]) for i in range(len(ocache)))
    ev = max(rel_err(to_f64(cache.v[i]), ocache[i][1]) for i in range(len(ocache)))
    print(f"{shape.name}: rows={len(rows)} hidden {eh:.2e} logits {el:.2e} K {ek:.2e} V {ev:.2e}")
    assert eh <= tol and el <= tol and ek <= tol and ev <= tol
    lg = to_f64(logits)
    if not check_ids:
        return lg, ref
    # argmax ids: identical wherever the oracle's top-1/top-2 margin clears the gate
    srt = np.sort(ref["logits"], axis=1)
    margin = srt[:, -1] - srt[:, -2]
    gate = margin_gate(srt[:, -1], margin) if shape.dtype == "bf16" else margin > 1e-2
    bad = np.flatnonzero(gate & (lg.argmax(1) != ref["logits"].argmax(1)))
    for i in bad:
        print(f"row {i}: device argmax {lg[i].argmax()} oracle {ref['logits'][i].argmax()} "
              f"margin {margin[i]:.4f} top1 {srt[i, -1]:.4f}")
    assert bad.size == 0
    # entropy of the device logits through the oracle vs the oracle's own: end-to-end drift only
    return lg, ref


@pytest.mark.parametrize("kind", ["full", "partial"])
def test_forward_tiny_f32(kind):
    cfg = synth.CONFIGS["tiny"]
    shape, L = cfg.model, cfg.seq_len
    w, omm, dm, cache, oc = _setup(shape, L, stale=(kind == "partial"))
    tokens = synth.make_prompt(cfg)
    rows = np.arange(L) if kind == "full" else np.array(sorted(set(range(100, 128)) | {3, 50, 97}))
    _compare(shape, omm, dm, cache, oc, tokens, rows, rows[-5:] if kind == "partial" else np.arange(96, 128))


@pytest.mark.parametrize("kind", ["full", "partial", "single"])
def test_forward_mini_bf16(kind):
    shape, L = MINI_BF16, 320
    w, omm, dm, cache, oc = _setup(shape, L, seed=2, stale=(kind != "full"))
    rng = np.random.default_rng(4)
    tokens = rng.integers(0, shape.vocab - 1, L).astype(np.int32)
    if kind == "full":
        rows = np.arange(L)
    elif kind == "partial":
        rows = np.sort(rng.choice(L, 157, replace=False))
    else:
        rows = np.array([211])
    _compare(shape, omm, dm, cache, oc, tokens, rows, rows[: min(len(rows), 40)])


@pytest.mark.parametrize("kind", ["full", "partial"])
def test_forward_small_two_layers(kind):
    """Full-width layers of the small bf16 config (d=2048, F=5632, V=32000, L=512)."""
    cfg = synth.CONFIGS["small"]
    shape, L = cfg.model, cfg.seq_len
    w, omm, dm, cache, oc = _setup(shape, L, n_layers=2, stale=(kind == "partial"))
    tokens = synth.make_prompt(cfg)
    rows = np.arange(L) if kind == "full" else np.arange(384 - 8, 512)
    _compare(shape, omm, dm, cache, oc, tokens, rows, np.arange(384, 512))


def test_partial_after_full_is_idempotent_bf16():
    """Right after a refresh, a skip step on the same tokens reproduces the refresh's rows."""
    from entropy_guided_kv_amd import api
    shape, L = MINI_BF16, 256
    w, omm, dm, cache, oc = _setup(shape, L, seed=5, stale=False)
    tokens = np.random.default_rng(6).integers(0, 1000, L).astype(np.int32)
    tk = torch.from_numpy(tokens).cuda()
    allr = torch.arange(L, dtype=torch.int32, device="cuda")
    lg_full, h_full = api.ec_forward(dm, cache, tk, allr, allr, want_hidden=True)
    k0 = [t.clone() for t in cache.k]
    rows = torch.tensor([0, 17, 100, 255], dtype=torch.int32, device="cuda")
    lg_p, h_p = api.ec_forward(dm, cache, tk, rows, torch.arange(4, dtype=torch.int32, device="cuda"),
                               want_hidden=True)
    torch.cuda.synchronize()
    assert row_rel_err(to_f64(h_p), to_f64(h_full)[rows.long().cpu().numpy()]) < 2e-2
    assert row_rel_err(to_f64(lg_p), to_f64(lg_full)[rows.long().cpu().numpy()]) < 2e-2
    for a, b in zip(cache.k, k0):
        assert rel_err(to_f64(a), to_f64(b)) < 2e-2
