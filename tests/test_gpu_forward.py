"""GPU parity: ec_forward (full and partial) against the oracle's forward.

A refresh step is the forward over every position; a skip step recomputes only
the listed rows against the cached (stale) K/V of the others (EntropyCache
explainer, Arabic technical summary section 2, phase 1). Bars, per row: fp32
models 1e-5 relative for hidden states, the recomputed K/V rows and logits;
bf16 models 2e-2 relative; cache rows outside the recomputed set bit-identical;
argmax ids bit-exact wherever the top-1/top-2 logit margin clears the id gate
(1e-2, and two bf16 steps of |top-1| for bf16 models).
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
    """ec_forward over ``rows`` against the oracle's forward on the same (stale) cache.

    Per row: hidden states and logits of the listed rows, and the K / V rows the call wrote
    (the recomputed positions only, so stale rows with zero error do not dilute the bar);
    every cache row outside ``rows`` must be bit-identical to what it held before the call.
    Argmax ids must match where the oracle's margin clears the id gate."""
    from entropy_guided_kv_amd import api
    L = len(tokens)
    rows = np.asarray(rows)
    outside = torch.from_numpy(np.setdiff1d(np.arange(L), rows)).cuda()
    before = [(cache.k[i][outside].clone(), cache.v[i][outside].clone()) for i in range(len(ocache))]
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
    ek = max(row_rel_err(to_f64(cache.k[i])[rows], ocache[i][0][rows]) for i in range(len(ocache)))
    ev = max(row_rel_err(to_f64(cache.v[i])[rows], ocache[i][1][rows]) for i in range(len(ocache)))
    print(f"{shape.name}: rows={len(rows)} worst row: hidden {eh:.2e} logits {el:.2e} K {ek:.2e} V {ev:.2e}")
    assert eh <= tol and el <= tol and ek <= tol and ev <= tol
    for i, (kb, vb) in enumerate(before):
        assert torch.equal(cache.k[i][outside], kb) and torch.equal(cache.v[i][outside], vb), \
            f"layer {i}: a cache row outside the recomputed set changed"
    lg = to_f64(logits)
    if not check_ids:
        return lg, ref
    # argmax ids: identical wherever the oracle's top-1/top-2 margin clears the id gate
    srt = np.sort(ref["logits"], axis=1)
    margin = srt[:, -1] - srt[:, -2]
    gate = margin_gate(srt[:, -1], margin, shape.dtype)
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


@pytest.mark.parametrize("kind", ["full", "partial", "single", "many_out"])
def test_forward_mini_bf16(kind):
    """"many_out": logits of 200 rows, an LM head product (200 x 1024 x 256) that the GEMM
    planner must not give a tile without the stored-logits epilogue."""
    shape, L = MINI_BF16, 320
    w, omm, dm, cache, oc = _setup(shape, L, seed=2, stale=(kind not in ("full", "many_out")))
    rng = np.random.default_rng(4)
    tokens = rng.integers(0, shape.vocab - 1, L).astype(np.int32)
    if kind == "many_out":
        rows = np.arange(L)
        _compare(shape, omm, dm, cache, oc, tokens, rows, np.sort(rng.choice(L, 200, replace=False)))
        return
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
    ri = rows.long().cpu().numpy()
    assert row_rel_err(to_f64(h_p), to_f64(h_full)[ri]) < 2e-2
    assert row_rel_err(to_f64(lg_p), to_f64(lg_full)[ri]) < 2e-2
    outside = np.setdiff1d(np.arange(L), ri)
    for a, b in zip(cache.k, k0):
        assert row_rel_err(to_f64(a)[ri], to_f64(b)[ri]) < 2e-2
        assert torch.equal(a[outside], b[outside])


@pytest.mark.parametrize("case", ["tiny_full", "tiny_partial", "mini_full", "mini_partial", "mini_one_out",
                                  "small_partial"])
def test_forward_last_layer_over_outputs(case):
    """Without the hidden states, the last layer runs its attention, O-proj and MLP over the
    output rows only (their final states are all the LM head reads); its K/V are still
    written for every row. Against the whole forward on the same starting cache: every
    cache row bit-identical (the QKV projections see the same inputs); fp32 logits
    bit-identical (the fp32 kernels sum each output in a fixed order whatever the row
    count); bf16 logits within the bf16 bar of the oracle's, ids where the gate allows."""
    from entropy_guided_kv_amd import api
    if case.startswith("tiny"):
        cfg = synth.CONFIGS["tiny"]
        shape, L = cfg.model, cfg.seq_len
        tokens = synth.make_prompt(cfg)
        seed, n_layers = 0, None
    elif case.startswith("mini"):
        shape, L = MINI_BF16, 320
        tokens = np.random.default_rng(7).integers(0, shape.vocab - 1, L).astype(np.int32)
        seed, n_layers = 3, None
    else:
        cfg = synth.CONFIGS["small"]
        shape, L = cfg.model, cfg.seq_len
        tokens = synth.make_prompt(cfg)
        seed, n_layers = 0, 2
    partial = case.endswith("partial") or case.endswith("one_out")
    w, omm, dm, cache, oc = _setup(shape, L, seed=seed, n_layers=n_layers, stale=partial)
    rng = np.random.default_rng(11)
    rows = np.sort(rng.choice(L, min(150, 3 * L // 4), replace=False)) if partial else np.arange(L)
    if case.endswith("one_out"):
        out_idx = np.array([77], np.int32)
    else:
        out_idx = np.sort(rng.choice(len(rows), 32, replace=False)).astype(np.int32)
    # a second cache with the same starting rows for the whole forward
    cache2 = api.KVCache(dm, L)
    for a, b in zip(cache2.k + cache2.v, cache.k + cache.v):
        a.copy_(b)
    tk = torch.from_numpy(tokens).cuda()
    rt = torch.from_numpy(rows.astype(np.int32)).cuda()
    ot = torch.from_numpy(out_idx).cuda()
    lg_out, h_none = api.ec_forward(dm, cache, tk, rt, ot, want_hidden=False)
    lg_all, _ = api.ec_forward(dm, cache2, tk, rt, ot, want_hidden=True)
    torch.cuda.synchronize()
    assert h_none is None
    for i, (a, b) in enumerate(zip(cache.k + cache.v, cache2.k + cache2.v)):
        assert torch.equal(a, b), f"cache tensor {i} differs between the two paths"
    if shape.dtype == "f32":
        assert torch.equal(lg_out, lg_all)
    ref = om.forward(omm, tokens, rows, oc, out_rows=rows[out_idx])
    lg = to_f64(lg_out)
    el = row_rel_err(lg, ref["logits"])
    print(f"{case}: rows={len(rows)} outputs={len(out_idx)} worst logit row {el:.2e}")
    assert el <= _tol(shape)
    srt = np.sort(ref["logits"], axis=1)
    gate = margin_gate(srt[:, -1], srt[:, -1] - srt[:, -2], shape.dtype)
    assert not np.any(gate & (lg.argmax(1) != ref["logits"].argmax(1)))
