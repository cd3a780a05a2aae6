"""GPU parity: whole denoising trajectories through ec_step against the oracle loop.

Per step (EntropyCache explainer, Arabic technical summary section 2): the
path taken (refresh or skip), the recompute-set size, the decoded positions
and ids, E_{t+1} and the next step's flag. Decoded ids and positions must be
identical wherever the oracle's top-1/top-2 logit margin of the decoded rows
exceeds the id gate (1e-2 for fp32 models, max(1e-2, 2 bf16 ulps of |top-1|)
for bf16 models, whose logits are stored in bf16) and the confidence gap at the
selection cut (log space) exceeds the cut gate (1e-2 for fp32 models; for bf16
the most two rows' log-confidences can move when every stored logit moves by
one bf16 step, tests/gpu_util.py); the first step that
fails that gate ends the comparison (the two trajectories may legitimately
part there). E within 1e-3 nats for fp32 models; for bf16 models E is checked
against the oracle's entropy of the device's own logits (within 1e-3) by the
forward tests, and end to end within 2e-2.
"""
import math

import numpy as np
import pytest
import torch

import synth
from oracle import loop as ol
from oracle import model as om
from tests.gpu_util import bf16_ulp, cut_gate_threshold, margin_gate

pytestmark = pytest.mark.gpu

PEAKED_SCALE, PEAKED_TAU = 24.0, 2.15


def _decoder(dm, cfg, tau):
    from entropy_guided_kv_amd import api
    dec = api.Decoder(dm, cfg.seq_len, cfg.prompt_len, cfg.tokens_per_step, cfg.block_len,
                      cfg.k_recent, tau, window=cfg.window)
    return dec


def _gate_ok(rec, n, dtype):
    """True when the oracle's step is decided by more than the gates: every decoded row's
    top-1/top-2 margin clears id_gate_threshold and the confidence gap at the selection cut
    (log space) clears cut_gate_threshold."""
    where = {int(p): i for i, p in enumerate(rec.cand)}
    idx = [where[int(p)] for p in rec.picked]
    ok = margin_gate(rec.top1, rec.margin, dtype)
    if not all(ok[i] for i in idx):
        return False
    order = np.argsort(-np.log(rec.maxprob), kind="stable")
    if len(order) > n:
        a, b = order[n - 1], order[n]
        gap = abs(np.log(rec.maxprob[a]) - np.log(rec.maxprob[b]))
        if gap <= cut_gate_threshold(rec.maxprob[a], rec.top1[a], rec.maxprob[b], rec.top1[b], dtype):
            return False
    return True


def _first_gated(recs, n, dtype):
    """Index of the oracle's first step that does not clear the gates (len(recs) if none)."""
    for i, r in enumerate(recs):
        if not _gate_ok(r, n, dtype):
            return i
    return len(recs)


def _e_tol_perturbation(rec, steps=2):
    """End-to-end bar on E for a bf16 fixture, from the oracle's own logits: with
    H = -sum p ln p, dH/dx_j = -p_j (x_j - <x>_p), so if every stored logit of a row lies
    within `steps` bf16 steps (at the row's top-1 magnitude) of the oracle's,
    |dH| <= steps ulp(top-1) sum_j p_j |x_j - <x>_p|; E (the max over the decoded rows)
    moves by at most the largest such bound, plus 1e-3 for second-order terms and the fp32
    reduction. Two steps: a skip step's logits also carry the error of cached K/V rows
    computed at earlier steps (one step is the id gate's premise for a single forward)."""
    where = {int(p): i for i, p in enumerate(rec.cand)}
    bound = 0.0
    for p in rec.picked:
        x = rec.logits[where[int(p)]]
        q = np.exp(x - x.max())
        q /= q.sum()
        mad = float(np.sum(q * np.abs(x - np.sum(q * x))))
        bound = max(bound, steps * float(bf16_ulp(x.max())) * mad)
    return bound + 1e-3


def _compare_run(cfg, w, tau, max_steps=None, e_tol=None, expect_full_compare=True, min_compared=None):
    from entropy_guided_kv_amd import api
    if e_tol is None:
        e_tol = 1e-3 if cfg.model.dtype == "f32" else 2e-2
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    dec = _decoder(dm, cfg, tau)
    prompt = synth.make_prompt(cfg)
    dec.reset(torch.from_numpy(prompt))
    outs = dec.run(max_steps=max_steps)
    recs, st, _ = ol.run_entropycache(om.OracleModel(w), cfg, prompt, tau, max_steps=max_steps,
                                      keep_logits=callable(e_tol))
    assert len(outs) == len(recs)
    compared = 0
    for o, r in zip(outs, recs):
        assert o.refreshed == r.refreshed, f"step {r.t}: path differs"
        assert o.rows == len(r.rows), f"step {r.t}: |R| {o.rows} vs {len(r.rows)}"
        assert o.n_cand == len(r.cand)
        gate = _gate_ok(r, cfg.tokens_per_step, cfg.model.dtype)
        same = o.positions == [int(p) for p in r.picked] and o.ids == [int(i) for i in r.ids]
        if not same:
            assert not gate, f"step {r.t}: decoded {o.positions}/{o.ids} vs {list(r.picked)}/{list(r.ids)}"
            print(f"trajectories part at step {r.t} (near tie, gated)")
            break
        tol = e_tol(r) if callable(e_tol) else e_tol
        assert abs(o.emax - r.emax) <= tol, f"step {r.t}: E {o.emax} vs {r.emax}"
        if abs(float(np.float32(r.emax)) - tau) > tol:
            assert o.refresh_next == r.refresh_next
        compared += 1
    if expect_full_compare:
        assert compared == len(recs)
    if min_compared is not None:
        assert compared >= min_compared, f"{compared} steps compared, fewer than {min_compared}"
    return outs, recs


def test_tiny_trajectory_as_configured():
    cfg = synth.CONFIGS["tiny"]
    outs, recs = _compare_run(cfg, synth.make_model(cfg.model), cfg.tau)
    assert len(outs) == cfg.steps and all(o.refreshed for o in outs)


def test_tiny_trajectory_peaked_mixed_branches():
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    outs, recs = _compare_run(cfg, w, PEAKED_TAU)
    flags = [o.refreshed for o in outs]
    assert any(flags[1:]) and not all(flags[1:])


def test_tiny_tau_plus_inf_all_skips():
    cfg = synth.CONFIGS["tiny"]
    outs, recs = _compare_run(cfg, synth.make_model(cfg.model), math.inf)
    assert [o.refreshed for o in outs] == [True] + [False] * (cfg.steps - 1)


def test_tiny_multi_token_steps_and_ring_cut():
    cfg = synth.DecodeConfig("t3", synth.TINY, 96, 32, 3, 8, 5, (math.inf,))
    _compare_run(cfg, synth.make_model(cfg.model), math.inf)


@pytest.mark.parametrize("n,k", [(4, 2), (3, 1)])
@pytest.mark.parametrize("peaked", [False, True])
def test_tiny_more_tokens_per_step_than_recent_budget(n, k, peaked):
    """n > k: a step decodes more positions than the decode-time ring holds, so only the
    step's last k positions (the highest) stay in the ring (the k most recently decoded of
    the decode record, Arabic technical summary section 2, phase 3). At tau = +inf every
    step after the first is a skip step; on the peaked model the path follows E (the
    oracle's path, which mixes refresh and skip steps for n = 4). |R|, path, positions
    and ids must equal the oracle's on every step."""
    cfg = synth.DecodeConfig(f"t{n}{k}", synth.TINY, 96, 32, n, 8, k, (math.inf,))
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE if peaked else 1.0)
    tau = PEAKED_TAU if peaked else math.inf
    outs, recs = _compare_run(cfg, w, tau)
    assert all(o.rows == len(r.rows) for o, r in zip(outs, recs))
    flags = [o.refreshed for o in outs]
    print("paths", "".join("F" if f else "." for f in flags))
    if not peaked:
        assert flags == [True] + [False] * (len(flags) - 1)
    elif n == 4:
        assert any(flags[1:]) and not all(flags[1:])


@pytest.mark.parametrize("name,P,M,n,B,k", [("no_recent", 96, 32, 1, 8, 0), ("no_prompt", 0, 32, 2, 8, 3),
                                            ("ragged_last_block", 90, 30, 2, 8, 4)])
def test_tiny_degenerate_budgets(name, P, M, n, B, k):
    """k = 0: R is the still-masked positions alone and the decode-time ring stays empty;
    P = 0: every position starts masked; M = 30 with B = 8: the last block holds 6 positions.
    Skip steps after the first exercise all three.

    With P = 0 the first step is an exact tie: every row holds the mask token, so every V
    row is the same and every row's attention output is that row whatever the weights;
    all candidates then share one entropy, confidence and argmax, and rounding decides
    which n of them are picked. That step is checked on what is unique (path, set sizes,
    E, the shared id, n distinct candidates), and the trajectories may part after it."""
    cfg = synth.DecodeConfig(name, synth.TINY, P, M, n, B, k, (math.inf,))
    outs, recs = _compare_run(cfg, synth.make_model(cfg.model), math.inf, expect_full_compare=P > 0)
    if k == 0:
        assert [o.rows for o in outs[1:]] == [M - n * t for t in range(1, len(outs))]
    if P == 0:
        o, r = outs[0], recs[0]
        # equal up to the oracle's own float64 rounding
        assert np.ptp(r.entropy) < 1e-9 and np.ptp(np.log(r.maxprob)) < 1e-9 and len(set(r.argmax)) == 1
        assert o.refreshed and o.rows == len(r.rows) and o.n_cand == len(r.cand)
        assert len(set(o.positions)) == n and set(o.positions) <= set(int(c) for c in r.cand)
        assert o.ids == [int(r.argmax[0])] * n
        assert abs(o.emax - r.emax) <= 1e-3


def _random_tiny_configs(n=12, seed=4242):
    """Tiny fp32 decodes drawn from a fixed seed: prompt length, masked count (L <= 128),
    tokens per step, block length, recent budget k, weight and prompt seeds, fixed blocks or a
    sliding window, and either the peaked LM head with its mixing threshold or tau = +inf."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 65))
        P = int(rng.integers(1, 129 - M))
        nt = int(rng.integers(1, 5))
        B = int(rng.choice([2, 4, 8, 16, 32, M]))
        k = int(rng.integers(0, 9))
        peaked = bool(rng.integers(0, 2))
        window = bool(rng.integers(0, 2))
        cfg = synth.DecodeConfig(f"r{i}", synth.TINY, P, M, nt, B, k, (math.inf,), seed=int(rng.integers(0, 1000)),
                                 window=window)
        out.append(pytest.param(cfg, peaked, id=f"P{P}-M{M}-n{nt}-B{B}-k{k}-{'peaked' if peaked else 'inf'}"
                                                f"{'-win' if window else ''}-s{cfg.seed}"))
    return out


@pytest.mark.parametrize("cfg,peaked", _random_tiny_configs())
def test_tiny_seeded_random_decodes(cfg, peaked):
    """Whole tiny fp32 trajectories over configurations off the hand-picked list (ragged last
    blocks, n > k and n <= k, k = 0, sliding windows, mixed and all-skip paths): path, |R|,
    positions, ids, E and the next flag on every step the gates decide."""
    w = synth.make_model(cfg.model, seed=cfg.seed, lm_head_scale=PEAKED_SCALE if peaked else 1.0)
    outs, recs = _compare_run(cfg, w, PEAKED_TAU if peaked else math.inf, expect_full_compare=False,
                              min_compared=1)
    print("paths", "".join("F" if o.refreshed else "." for o in outs))


def test_tau_minus_inf_equals_vanilla_on_gpu():
    """tau = -inf refreshes every step; it must match a run that forces a refresh each step."""
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompt = torch.from_numpy(synth.make_prompt(cfg))
    a = _decoder(dm, cfg, -math.inf)
    a.reset(prompt)
    oa = a.run()
    b = _decoder(dm, cfg, math.inf)
    b.reset(prompt)
    ob = []
    while not b.done:
        b.state.refresh_next = 1
        ob.append(b.step())
    assert [(o.positions, o.ids, o.emax) for o in oa] == [(o.positions, o.ids, o.emax) for o in ob]
    assert torch.equal(a.tokens, b.tokens)


def test_small_bf16_first_steps():
    """bf16 small config (8 layers, d=2048, V=32000, L=512, 2 tokens/step) with its own N(0, 0.02)
    weights: every step's path, recompute-set size and E (2e-2) against the oracle up to the
    first difference of the decoded set, which these flat logits allow at a gated near tie
    (the decoded ids are compared on the separated fixture below)."""
    cfg = synth.CONFIGS["small"]
    _compare_run(cfg, synth.make_model(cfg.model), cfg.tau, max_steps=3, expect_full_compare=False)


HOT = dict(hot_tokens=8, hot_scale=10.0)  # synth.make_hot_token_model fixture


@pytest.mark.parametrize("tau", [1.0, math.inf])
def test_small_bf16_whole_block_steps_hot_token_fixture(tau):
    """The bf16 small model (8 layers, d=2048, V=32000, L=512, k=8) decoding a whole block
    of 16 per step (no confidence cut to decide) on the hot-token fixture (every row's
    top-1 clearly ahead): the oracle clears the id gate on its first six steps (a property
    of the fixture, checked on the oracle alone), so the device must decode exactly its
    positions and ids on at least those, the same path, and E within the first-order bound
    of the entropy's change under one-step logit differences (_e_tol_perturbation: the hot
    rows' logits reach ~11 - 30, where the entropy moves by ~(x_top - <x>) times the
    logits' error); at tau = 1 refresh and skip steps mix."""
    import dataclasses
    cfg = dataclasses.replace(synth.CONFIGS["small"], tokens_per_step=16, block_len=16)
    w = synth.make_hot_token_model(cfg.model, **HOT)
    recs, _, _ = ol.run_entropycache(om.OracleModel(w), cfg, synth.make_prompt(cfg), tau, max_steps=8)
    first = _first_gated(recs, cfg.tokens_per_step, "bf16")
    assert first >= 6, f"fixture: only {first} leading steps clear the gates"
    outs, _ = _compare_run(cfg, w, tau, max_steps=8, e_tol=_e_tol_perturbation, expect_full_compare=False,
                           min_compared=first)
    flags = [o.refreshed for o in outs]
    if tau == math.inf:
        assert flags == [True] + [False] * (len(flags) - 1)
    else:
        assert any(flags[1:]) and not all(flags[1:])


def test_small_bf16_skip_steps():
    """As test_small_bf16_first_steps, at tau = +inf (skip steps after the first)."""
    cfg = synth.CONFIGS["small"]
    _compare_run(cfg, synth.make_model(cfg.model), math.inf, max_steps=6, expect_full_compare=False)


def test_determinism_two_runs_bit_identical():
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompt = torch.from_numpy(synth.make_prompt(cfg))
    res = []
    for _ in range(2):
        d = _decoder(dm, cfg, PEAKED_TAU)
        d.reset(prompt)
        o = d.run()
        res.append(([(x.positions, x.ids, x.emax, x.refreshed) for x in o], d.tokens.cpu(),
                    [k.cpu() for k in d.cache.k]))
    assert res[0][0] == res[1][0]
    assert torch.equal(res[0][1], res[1][1])
    assert all(torch.equal(a, b) for a, b in zip(res[0][2], res[1][2]))


MINI256 = synth.DecodeConfig("mini256", synth.ModelShape("mini", "bf16", 2, 256, 2, 128, 512, 1024),
                             64, 256, 8, 256, 8, (math.inf,))


@pytest.mark.parametrize("n_cand_rows", ["small", "mini256"])
def test_fused_lm_head_entropy_matches_stored_logits(n_cand_rows):
    """bf16 ec_step reduces the LM head's logits in the GEMM epilogue (no logits tensor).
    Its first step must match ec_forward's stored logits reduced by ec_entropy_max: same
    picked positions and ids, entropy within 1e-5 nats, confidence within 1e-5 relative.
    "small": 128 candidate rows of the small model; "mini256": 256 candidate rows of a
    d = 256, V = 1024 model, a product the GEMM planner would price for tiles that have no
    entropy epilogue (it must plan only the 128x128 or 64x128 tile for these)."""
    from entropy_guided_kv_amd import api
    cfg = synth.CONFIGS["small"] if n_cand_rows == "small" else MINI256
    w = synth.make_model(cfg.model, n_layers=2)
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    prompt = synth.make_prompt(cfg)
    dec = _decoder(dm, cfg, math.inf)
    dec.reset(torch.from_numpy(prompt))
    tokens0 = dec.tokens.clone()
    o = dec.step()
    assert o.refreshed
    L, P, B = cfg.seq_len, cfg.prompt_len, cfg.block_len
    cand = np.arange(P, min(P + B, L))
    cache = api.KVCache(dm, L)
    allr = torch.arange(L, dtype=torch.int32, device="cuda")
    logits, _ = api.ec_forward(dm, cache, tokens0, allr, torch.from_numpy(cand.astype(np.int32)).cuda())
    H, a, c, _ = api.ec_entropy_max(logits)
    torch.cuda.synchronize()
    H, a, c = H.cpu().numpy(), a.cpu().numpy(), c.cpu().numpy()
    order = sorted(range(len(cand)), key=lambda i: (-c[i], cand[i]))[: cfg.tokens_per_step]
    picked = sorted(order, key=lambda i: cand[i])
    assert o.positions == [int(cand[i]) for i in picked]
    assert o.ids == [int(a[i]) for i in picked]
    np.testing.assert_allclose(o.entropy, H[picked], rtol=0, atol=1e-5)
    np.testing.assert_allclose(o.maxprob, c[picked], rtol=1e-5, atol=0)


@pytest.mark.parametrize("n,B", [(1, 8), (3, 5)])
def test_tiny_sliding_window_trajectory(n, B):
    """Sliding-window candidates (EC_CAND_WINDOW): the whole trajectory follows the oracle,
    with refresh and skip steps mixed; it differs from block decoding."""
    import dataclasses
    base = synth.CONFIGS["tiny"]
    cfg = dataclasses.replace(base, tokens_per_step=n, block_len=B, window=True)
    w = synth.make_model(cfg.model, lm_head_scale=PEAKED_SCALE)
    outs, recs = _compare_run(cfg, w, PEAKED_TAU)
    flags = [o.refreshed for o in outs]
    assert any(flags[1:]) and not all(flags[1:])
    blk, _, _ = ol.run_entropycache(om.OracleModel(w), dataclasses.replace(cfg, window=False), synth.make_prompt(cfg),
                                    PEAKED_TAU)
    assert [list(r.picked) for r in blk] != [list(r.picked) for r in recs]


@pytest.mark.parametrize("name", ["tiny_trajectory.json", "tiny_peaked_trajectory.json"])
def test_tiny_trajectory_matches_stored_golden(name):
    """The device trajectory against the stored oracle trajectory (tests/golden/): same path,
    recompute-set sizes, positions, ids and final tokens; E within 1e-3 nats (fp32 model)."""
    import json
    import os
    from entropy_guided_kv_amd import api
    stored = json.load(open(os.path.join(os.path.dirname(__file__), "golden", name)))
    cfg = synth.CONFIGS[stored["config"]]
    w = synth.make_model(cfg.model, lm_head_scale=stored["lm_head_scale"])
    dm = api.DeviceModel.from_host(w, rope_max_pos=cfg.seq_len)
    dec = _decoder(dm, cfg, stored["tau"])
    dec.reset(torch.from_numpy(synth.make_prompt(cfg)))
    outs = dec.run()
    assert len(outs) == len(stored["steps"])
    for o, s in zip(outs, stored["steps"]):
        assert (o.refreshed, o.rows, o.positions, o.ids) == \
               (s["refreshed"], s["n_rows"], s["positions"], s["ids"]), f"step {s['t']}"
        assert abs(o.emax - s["emax"]) <= 1e-3, f"step {s['t']}: E {o.emax} vs {s['emax']}"
    assert dec.tokens.cpu().tolist() == stored["final_tokens"]
