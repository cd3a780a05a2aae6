"""GPU parity: ec_step_batch (several sequences in one forward per step).

Each sequence must follow exactly the trajectory ec_step gives it alone, and the
oracle's loop run on that sequence alone (EntropyCache explainer, Arabic
technical summary section 2: the decision is taken per sequence from its own
E). Bars as for ec_step: path, |R|, candidates, decoded positions and ids
identical wherever the margin gate clears; E within 1e-3 nats (fp32 models) or
2e-2 (bf16) of the oracle. Against ec_step alone, fp32 runs are bit-identical
(the fp32 kernels reduce every output in a fixed order whatever the row count).
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import loop as ol
from oracle import model as om
from tests.test_gpu_step import PEAKED_SCALE, PEAKED_TAU, _gate_ok

pytestmark = pytest.mark.gpu


def _prompts(cfg, n):
    base = synth.make_prompt(cfg)
    out = [base]
    for i in range(1, n):
        p = base.copy()
        rng = np.random.default_rng(100 + i)
        p[: cfg.prompt_len] = rng.integers(0, cfg.model.vocab - 1, cfg.prompt_len)
        out.append(p)
    return out


def _batch_run(dm, cfg, tau, prompts, max_steps=None, window=False):
    from entropy_guided_kv_amd import api
    bd = api.BatchDecoder(dm, len(prompts), cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step,
                          cfg.block_len, cfg.k_recent, tau, window=window)
    bd.reset([torch.from_numpy(p) for p in prompts])
    steps = bd.run(max_steps=max_steps)
    return bd, [[st[i] for st in steps] for i in range(len(prompts))]


def _check_vs_oracle(outs, recs, cfg, tau, e_tol):
    compared = 0
    for o, r in zip(outs, recs):
        assert o is not None
        assert o.refreshed == r.refreshed, f"step {r.t}: path differs"
        assert o.rows == len(r.rows) and o.n_cand == len(r.cand)
        same = o.positions == [int(p) for p in r.picked] and o.ids == [int(i) for i in r.ids]
        if not same:
            assert not _gate_ok(r, cfg.tokens_per_step, cfg.model.dtype), f"step {r.t}: decoded differs"
            break
        tol = e_tol(r) if callable(e_tol) else e_tol
        assert abs(o.emax - r.emax) <= tol, f"step {r.t}: E {o.emax} vs {r.emax}"
        if abs(float(np.float32(r.emax)) - tau) > tol:
            assert o.refresh_next == r.refresh_next
        compared += 1
    return compared


def test_batch_tiny_peaked_matches_oracle_and_single():
    """Three fp32 sequences, refresh and skip steps mixed within and across sequences."""
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompts = _prompts(cfg, 3)
    bd, seq_outs = _batch_run(dm, cfg, PEAKED_TAU, prompts)
    mixed_step = False
    for t in range(len(seq_outs[0])):
        flags = {seq_outs[i][t].refreshed for i in range(3)}
        mixed_step |= len(flags) == 2
    assert mixed_step, "no step mixed refresh and skip sequences"
    for i, p in enumerate(prompts):
        recs, _, _ = ol.run_entropycache(om.OracleModel(w), cfg, p, PEAKED_TAU)
        assert len(seq_outs[i]) == len(recs)
        assert _check_vs_oracle(seq_outs[i], recs, cfg, PEAKED_TAU, 1e-3) == len(recs)
        # the same sequence stepped alone by ec_step: bit-identical
        dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                          cfg.k_recent, PEAKED_TAU)
        dec.reset(torch.from_numpy(p))
        single = dec.run()
        assert [(o.refreshed, o.positions, o.ids, o.emax) for o in single] == \
               [(o.refreshed, o.positions, o.ids, o.emax) for o in seq_outs[i]]
        assert torch.equal(dec.tokens, bd.tokens[i])
        for a, b in zip(dec.cache.k + dec.cache.v, bd.caches[i].k + bd.caches[i].v):
            assert torch.equal(a, b)


@pytest.mark.parametrize("tau", [1.0, math.inf])
def test_batch_small_bf16_first_steps(tau):
    """Two bf16 sequences of the small model, whole blocks of 16 per step, on the hot-token
    fixture (every row's top-1 clearly ahead), stepped together (one attention launch per
    layer over both): each sequence must match its own oracle trajectory on every step up to
    its first gated one (E within the first-order bound of the single-sequence test), and the
    first sequence's oracle clears the gates on its first four steps, so at least four
    steps' decoded positions and ids are compared."""
    import dataclasses
    from entropy_guided_kv_amd import api
    from tests.test_gpu_step import HOT, _e_tol_perturbation, _first_gated
    cfg = dataclasses.replace(synth.CONFIGS["small"], tokens_per_step=16, block_len=16)
    w = synth.make_hot_token_model(cfg.model, **HOT)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompts = _prompts(cfg, 2)
    steps = 5
    _, seq_outs = _batch_run(dm, cfg, tau, prompts, max_steps=steps)
    total = 0
    for i, p in enumerate(prompts):
        recs, _, _ = ol.run_entropycache(om.OracleModel(w), cfg, p, tau, max_steps=steps, keep_logits=True)
        first = _first_gated(recs, cfg.tokens_per_step, "bf16")
        compared = _check_vs_oracle(seq_outs[i], recs, cfg, tau, _e_tol_perturbation)
        assert compared >= first
        if i == 0:
            assert first >= 4
        total += compared
        assert seq_outs[i][0].refreshed
    assert total >= 4


def test_batch_sixteen_sequences_tiny():
    """The largest batch: 16 fp32 sequences equal their single-sequence runs."""
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompts = _prompts(cfg, 16)
    _, seq_outs = _batch_run(dm, cfg, PEAKED_TAU, prompts, max_steps=6)
    for i in (0, 7, 15):
        dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                          cfg.k_recent, PEAKED_TAU)
        dec.reset(torch.from_numpy(prompts[i]))
        single = dec.run(max_steps=6)
        assert [(o.refreshed, o.positions, o.ids, o.emax) for o in single] == \
               [(o.refreshed, o.positions, o.ids, o.emax) for o in seq_outs[i]]


def test_batch_sliding_window_tiny():
    """Sliding-window candidates (candidates from the window at each sequence's lowest masked
    position) in a batch of three fp32 sequences, blocks of 8 and two tokens per step, on the
    peaked head (refresh and skip steps mix): each sequence equals its single-sequence run
    bit for bit over its whole decode."""
    import dataclasses
    from entropy_guided_kv_amd import api
    cfg = dataclasses.replace(synth.CONFIGS["tiny"], tokens_per_step=2, block_len=8)
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompts = _prompts(cfg, 3)
    _, seq_outs = _batch_run(dm, cfg, PEAKED_TAU, prompts, window=True)
    for i in range(3):
        dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                          cfg.k_recent, PEAKED_TAU, window=True)
        dec.reset(torch.from_numpy(prompts[i]))
        single = dec.run()
        got = [o for o in seq_outs[i] if o is not None]
        assert len(got) == len(single) == cfg.steps
        assert [(o.refreshed, o.rows, o.positions, o.ids, o.emax) for o in single] == \
               [(o.refreshed, o.rows, o.positions, o.ids, o.emax) for o in got]
    assert any(o.refreshed for o in seq_outs[0][1:]) and not all(o.refreshed for o in seq_outs[0])


def _random_batches():
    from tests.test_gpu_step import _random_tiny_configs
    rng = np.random.default_rng(99)
    out = []
    for p in _random_tiny_configs()[:6]:
        cfg, peaked = p.values
        out.append(pytest.param(cfg, peaked, int(rng.integers(2, 9)), id=p.id))
    return out


@pytest.mark.parametrize("cfg,peaked,n_seq", _random_batches())
def test_batch_seeded_random_tiny(cfg, peaked, n_seq):
    """Batches of 2 to 8 fp32 sequences over the seeded random tiny configurations (ragged
    blocks, k = 0, n > k, sliding windows): each sequence equals its single-sequence run bit
    for bit over its whole decode."""
    from entropy_guided_kv_amd import api
    w = synth.make_model(cfg.model, seed=cfg.seed, lm_head_scale=PEAKED_SCALE if peaked else 1.0)
    tau = PEAKED_TAU if peaked else math.inf
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompts = _prompts(cfg, n_seq)
    bd, seq_outs = _batch_run(dm, cfg, tau, prompts, window=cfg.window)
    for i in range(n_seq):
        dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                          cfg.k_recent, tau, window=cfg.window)
        dec.reset(torch.from_numpy(prompts[i]))
        single = dec.run()
        got = [o for o in seq_outs[i] if o is not None]
        assert [(o.refreshed, o.rows, o.positions, o.ids, o.emax) for o in single] == \
               [(o.refreshed, o.rows, o.positions, o.ids, o.emax) for o in got]
        assert torch.equal(dec.tokens, bd.tokens[i])
