"""GPU parity of the KV-drift probe (ec_step_probe) against the oracle's drift measure.

fp32 model: the probe's per-layer (K mean, K max, V mean, V max) cosine
distances of the recomputed rows follow the oracle's trajectory run with the
same probe within 1e-5 (both caches agree to ~1e-6). bf16 model: the probe's
values equal the oracle's measure applied to the device's own cache before and
after the step, within 1e-4. The probe does not change the step.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import loop as ol
from oracle import model as om
from oracle.drift import step_drift
from tests.gpu_util import to_f64
from tests.test_gpu_step import PEAKED_SCALE, PEAKED_TAU

pytestmark = pytest.mark.gpu


def _decoder(dm, cfg, tau):
    from entropy_guided_kv_amd import api
    return api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len, cfg.k_recent, tau)


def _nan_close(a, b, atol):
    assert np.array_equal(np.isnan(a), np.isnan(b)), f"NaN pattern differs:\n{a}\n{b}"
    m = ~np.isnan(a)
    assert np.abs(a[m] - b[m]).max(initial=0.0) <= atol, f"max diff {np.abs(a[m] - b[m]).max()}"


def test_probe_tiny_f32_trajectory_matches_oracle():
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompt = synth.make_prompt(cfg)
    dec = _decoder(dm, cfg, PEAKED_TAU)
    dec.reset(torch.from_numpy(prompt))
    drift = torch.zeros(4 * cfg.model.n_layers, dtype=torch.float32, device="cuda")
    outs, drifts = [], []
    while not dec.done:
        outs.append(dec.step(drift=drift))
        drifts.append(drift.cpu().numpy().reshape(-1, 4).astype(np.float64))
    recs, _, _ = ol.run_entropycache(om.OracleModel(w), cfg, prompt, PEAKED_TAU, probe=True)
    assert len(outs) == len(recs)
    assert np.isnan(drifts[0]).all()  # first step: the cache was never written
    for t, (o, r, dg) in enumerate(zip(outs, recs, drifts)):
        assert o.positions == [int(p) for p in r.picked], f"step {t}"
        _nan_close(dg, r.drift, 1e-5)
    # E of step t against the V drift step t+1 measures (the pages' correlation), reported
    e = np.array([o.emax for o in outs[:-1]])
    dv = np.array([d[:, 2].mean() for d in drifts[1:]])
    ok = ~np.isnan(dv)
    if ok.sum() > 2:
        print(f"corr(E_t, mean V drift at t+1) = {np.corrcoef(e[ok], dv[ok])[0, 1]:.3f} over {ok.sum()} steps")


def test_probe_bf16_equals_measure_on_device_caches_and_leaves_step_unchanged():
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["small"]
    w = synth.make_model(cfg.model, n_layers=2)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompt = torch.from_numpy(synth.make_prompt(cfg))
    a, b = _decoder(dm, cfg, math.inf), _decoder(dm, cfg, math.inf)
    a.reset(prompt)
    b.reset(prompt)
    drift = torch.zeros(8, dtype=torch.float32, device="cuda")
    for t in range(4):  # refresh, then skip steps
        before = [[to_f64(k), to_f64(v)] for k, v in zip(a.cache.k, a.cache.v)]
        full = a.state.t == 0 or a.state.refresh_next
        rows = np.arange(cfg.seq_len) if full else a.next_rows()
        oa = a.step(drift=drift)
        ob = b.step()
        after = [[to_f64(k), to_f64(v)] for k, v in zip(a.cache.k, a.cache.v)]
        assert (oa.refreshed, oa.positions, oa.ids, oa.emax) == (ob.refreshed, ob.positions, ob.ids, ob.emax)
        assert oa.refreshed == full and oa.rows == len(rows)
        want = step_drift(before, after, rows)
        _nan_close(drift.cpu().numpy().reshape(-1, 4).astype(np.float64), want, 1e-4)
    for x, y in zip(a.cache.k + a.cache.v, b.cache.k + b.cache.v):
        assert torch.equal(x, y)
