"""The oracle still computes the stored tiny trajectories (tests/golden/, written by
tests/golden/make_golden.py from the oracle alone). The pages print no worked example;
these files pin the oracle against unintended changes: a change to its arithmetic that
moves them has to name, in its commit, the passage or reading that justifies it."""
import json
import os

import pytest

from tests.golden.make_golden import CASES, trajectory

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.mark.parametrize("name,scale,tau", CASES)
def test_oracle_reproduces_stored_trajectory(name, scale, tau):
    stored = json.load(open(os.path.join(HERE, name)))
    now = trajectory(scale, tau)
    assert now["final_tokens"] == stored["final_tokens"]
    assert len(now["steps"]) == len(stored["steps"])
    for a, b in zip(now["steps"], stored["steps"]):
        assert (a["t"], a["refreshed"], a["n_rows"], a["positions"], a["ids"], a["refresh_next"]) == \
               (b["t"], b["refreshed"], b["n_rows"], b["positions"], b["ids"], b["refresh_next"])
        assert a["emax"] == pytest.approx(b["emax"], rel=0, abs=1e-9)


def test_stored_peaked_trajectory_mixes_both_branches():
    stored = json.load(open(os.path.join(HERE, "tiny_peaked_trajectory.json")))
    flags = [s["refreshed"] for s in stored["steps"]]
    assert flags[0] and any(flags[1:]) and not all(flags[1:])
    # a step refreshes exactly when the previous step's E exceeded tau
    for prev, cur in zip(stored["steps"], stored["steps"][1:]):
        assert cur["refreshed"] == (prev["emax"] > stored["tau"])
