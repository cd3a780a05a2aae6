"""Pins for oracle.loop: decision rule, recompute set, selection and trajectory invariants.

Rule (EntropyCache explainer, Arabic technical summary section 2 phases 2-3;
Italian summary "Algoritmo di Funzionamento"): E_{t+1} > tau -> full forward
next step, otherwise a partial forward over the masked positions plus the k
most recently decoded ones; extra memory O(k) (Italian summary, section 4).
"""
import itertools
import math

import numpy as np
import pytest

import synth
from oracle import loop as ol
from oracle import model as om

CFG = synth.CONFIGS["tiny"]
PEAKED_SCALE, PEAKED_TAU = 24.0, 2.15   # lm-head scale and threshold giving mixed branches


@pytest.fixture(scope="module")
def tiny():
    w = synth.make_model(CFG.model)
    return om.OracleModel(w), synth.make_prompt(CFG)


@pytest.fixture(scope="module")
def peaked():
    w = synth.make_model(CFG.model, lm_head_scale=PEAKED_SCALE)
    return om.OracleModel(w), synth.make_prompt(CFG)


def test_tau_minus_inf_reproduces_vanilla(tiny):
    m, p = tiny
    ec, st, _ = ol.run_entropycache(m, CFG, p, -math.inf)
    va, st2 = ol.run_vanilla(m, CFG, p)
    assert len(ec) == len(va) == CFG.steps
    assert all(r.refreshed for r in ec)
    for a, b in zip(ec, va):
        np.testing.assert_array_equal(a.picked, b.picked)
        np.testing.assert_array_equal(a.ids, b.ids)
        np.testing.assert_array_equal(a.entropy, b.entropy)
    np.testing.assert_array_equal(st.tokens, st2.tokens)
    assert not st.masked.any()


def test_tau_plus_inf_refreshes_once_and_recompute_sizes(tiny):
    m, p = tiny
    recs, st, _ = ol.run_entropycache(m, CFG, p, math.inf)
    assert [r.refreshed for r in recs] == [True] + [False] * (CFG.steps - 1)
    for r in recs[1:]:
        decoded = CFG.tokens_per_step * r.t
        assert len(r.rows) == (CFG.n_masked - decoded) + min(CFG.k_recent, decoded)


def test_refresh_sequence_follows_strict_threshold(peaked):
    m, p = peaked
    recs, _, _ = ol.run_entropycache(m, CFG, p, PEAKED_TAU)
    flags = [r.refreshed for r in recs]
    assert any(flags[1:]) and not all(flags[1:]), "fixture must exercise both branches"
    assert flags[0]
    for prev, cur in zip(recs, recs[1:]):
        assert cur.refreshed == (np.float32(prev.emax) > np.float32(PEAKED_TAU))
    # equality skips: rerun with tau equal to one step's E
    tau_eq = float(np.float32(recs[3].emax))
    recs2, _, _ = ol.run_entropycache(m, CFG, p, tau_eq, max_steps=5)
    assert recs2[3].emax == tau_eq and not recs2[4].refreshed


def test_emax_is_max_entropy_of_decoded_rows(peaked):
    m, p = peaked
    cfg2 = synth.DecodeConfig("t2", CFG.model, 96, 32, 3, 32, 4, (PEAKED_TAU,))
    recs, _, _ = ol.run_entropycache(m, cfg2, p, PEAKED_TAU, max_steps=4)
    for r in recs:
        idx = [list(r.cand).index(q) for q in r.picked]
        assert r.emax == float(np.float32(max(r.entropy[i] for i in idx)))
        assert len(r.picked) == 3


def _brute_select(cand, conf, n):
    best = None
    for sub in itertools.combinations(range(len(cand)), min(n, len(cand))):
        s = set(sub)
        ok = all((conf[i] > conf[j]) or (conf[i] == conf[j] and cand[i] < cand[j])
                 for i in s for j in range(len(cand)) if j not in s)
        if ok:
            assert best is None, "selection must be unique"
            best = sorted(cand[i] for i in sub)
    return best


@pytest.mark.parametrize("seed", range(20))
def test_select_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    nc = int(rng.integers(1, 9))
    cand = np.sort(rng.choice(100, nc, replace=False))
    conf = rng.choice([0.1, 0.2, 0.3, 0.5], nc).astype(np.float32)  # many ties
    n = int(rng.integers(1, 5))
    np.testing.assert_array_equal(ol.select(cand, conf, n), _brute_select(cand, conf, n))


def test_window_candidates_start_at_lowest_mask():
    """Sliding window of B positions from the lowest masked position (not block-aligned)."""
    masked = np.zeros(20, dtype=bool)
    masked[[9, 12, 13, 17]] = True
    np.testing.assert_array_equal(ol.candidates(masked, 4, 4, window=True), [9, 12])      # [9, 13)
    np.testing.assert_array_equal(ol.candidates(masked, 4, 8, window=True), [9, 12, 13])  # [9, 17)
    masked[9] = False
    np.testing.assert_array_equal(ol.candidates(masked, 4, 4, window=True), [12, 13])     # [12, 16)
    np.testing.assert_array_equal(ol.candidates(masked, 4, 6, window=True), [12, 13, 17])
    assert ol.candidates(np.zeros(5, dtype=bool), 0, 2, window=True).size == 0


def test_window_candidates_brute_force():
    rng = np.random.default_rng(5)
    for _ in range(200):
        L, P, B = int(rng.integers(2, 40)), 0, int(rng.integers(1, 9))
        P = int(rng.integers(0, L))
        masked = np.zeros(L, dtype=bool)
        masked[P:] = rng.random(L - P) < 0.5
        got = ol.candidates(masked, P, B, window=True)
        pos = [p for p in range(L) if masked[p]]
        want = [p for p in pos if pos and pos[0] <= p < pos[0] + B]
        np.testing.assert_array_equal(got, want)
        # the window always holds the lowest masked position; blocks hold it too
        if pos:
            assert got[0] == pos[0] and ol.candidates(masked, P, B)[0] == pos[0]


def test_candidates_are_lowest_open_block():
    masked = np.zeros(20, dtype=bool)
    masked[[9, 12, 13, 17]] = True
    np.testing.assert_array_equal(ol.candidates(masked, 4, 4), [9])        # block [8,12)
    masked[9] = False
    np.testing.assert_array_equal(ol.candidates(masked, 4, 4), [12, 13])   # block [12,16)
    np.testing.assert_array_equal(ol.candidates(masked, 4, 16), [12, 13, 17])
    assert ol.candidates(np.zeros(5, dtype=bool), 0, 2).size == 0


def test_recompute_set_last_k_of_decode_log():
    masked = np.zeros(12, dtype=bool)
    masked[[10, 11]] = True
    log = [4, 5, 2, 9, 3]
    np.testing.assert_array_equal(ol.recompute_set(masked, log, 2), [3, 9, 10, 11])
    np.testing.assert_array_equal(ol.recompute_set(masked, log, 0), [10, 11])
    np.testing.assert_array_equal(ol.recompute_set(masked, log, 99), [2, 3, 4, 5, 9, 10, 11])


def test_nan_entropy_forces_refresh(tiny, monkeypatch):
    m, p = tiny
    st = ol.init_state(CFG, p)
    cache = om.new_cache(m, CFG.seq_len)
    ol.step(m, CFG, st, cache, math.inf)
    assert not st.refresh_next
    real = ol.entropy_rows

    def nan_rows(x):
        h, a, c = real(x)
        h[:] = np.nan
        return h, a, c

    monkeypatch.setattr(ol, "entropy_rows", nan_rows)
    rec = ol.step(m, CFG, st, cache, math.inf)
    assert math.isnan(rec.emax) and st.refresh_next


def test_decode_log_keeps_order_within_step(tiny):
    m, p = tiny
    cfg = synth.DecodeConfig("t3", CFG.model, 96, 32, 4, 32, 6, (math.inf,))
    recs, st, _ = ol.run_entropycache(m, cfg, p, math.inf, max_steps=3)
    flat = [int(q) for r in recs for q in r.picked]
    assert st.decode_log == flat
    for r in recs:
        assert list(r.picked) == sorted(r.picked)
    # step 2 recomputes the 24 still-masked positions plus the last 6 of the 8 logged ones
    # (the cut falls inside step 0's four picks)
    assert recs[-1].rows.tolist() == sorted(set(range(96, 128)) - set(flat[:8]) | set(flat[2:8]))


def test_select_ranks_nan_confidence_last():
    cand = np.array([3, 5, 9])
    conf = np.array([np.nan, 0.2, 0.1], dtype=np.float32)
    np.testing.assert_array_equal(ol.select(cand, conf, 1), [5])
    np.testing.assert_array_equal(ol.select(cand, conf, 3), [3, 5, 9])


def _device_ring(steps, k):
    """The decode-time ring as the device keeps it (O(k) memory): record index c lives in
    slot c mod k; a step appends its positions in ascending order at indices count0 ..
    count0 + n - 1, and only the indices >= count0 + n - k write their slot (one writer per
    slot). Returns (ring, count)."""
    ring, count = [-1] * k, 0
    for picked in steps:
        n = len(picked)
        for slot, p in enumerate(sorted(picked)):
            if slot >= n - k:
                ring[(count + slot) % k] = p
        count += n
    return ring, count


@pytest.mark.parametrize("n,k", [(4, 2), (3, 1), (5, 5), (7, 3), (1, 4), (2, 4), (64, 16)])
def test_decode_ring_slot_rule_keeps_the_last_k_entries(n, k):
    """With more positions decoded in a step than the recent budget (n > k) a step's own
    positions overflow the ring; the slot rule must still leave exactly the last k entries of
    the decode log (the higher positions of the last step), and the recompute set built from
    the ring must equal the oracle's (masked positions + decode_log[-k:])."""
    rng = np.random.default_rng(n * 100 + k)
    L = 400
    order = rng.permutation(L)
    masked = np.ones(L, dtype=bool)
    log, steps, i = [], [], 0
    while i < L:
        m = int(rng.integers(1, n + 1))  # steps of 1 .. n positions (a block's ragged end)
        picked = sorted(int(p) for p in order[i:i + m])
        i += m
        steps.append(picked)
        log += picked
        masked[picked] = False
        ring, count = _device_ring(steps, k)
        held = set(ring[:min(count, k)])
        assert held == set(log[-k:])
        R = sorted(set(np.flatnonzero(masked).tolist()) | held)
        np.testing.assert_array_equal(R, ol.recompute_set(masked, log, k))


def test_top2_margin_pins():
    """The top-1/top-2 logit margin the id gate uses: a worked row, a tied maximum (margin 0),
    shift invariance, and against a brute force written differently (the smallest gap between
    the row maximum and any other entry, over every index but the first argmax)."""
    np.testing.assert_array_equal(ol._top2_margin(np.array([[1.0, 5.0, 3.0]])), [2.0])
    np.testing.assert_array_equal(ol._top2_margin(np.array([[4.0, 1.0, 4.0]])), [0.0])
    assert ol._top2_margin(np.array([[7.0]]))[0] == np.inf
    rng = np.random.default_rng(5)
    x = np.round(rng.standard_normal((50, 37)) * 4) / 4  # quarter steps: ties happen
    m = ol._top2_margin(x)
    np.testing.assert_allclose(ol._top2_margin(x + 3.25), m, rtol=0, atol=1e-12)
    for row, got in zip(x, m):
        a = int(np.argmax(row))
        brute = min(row[a] - row[j] for j in range(len(row)) if j != a)
        assert got == brute
    assert (m >= 0).all()
