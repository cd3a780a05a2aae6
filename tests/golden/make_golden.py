"""Write the stored oracle trajectories under tests/golden/ (run from the repository root).

The pages print no worked example of the method (no intermediate values, no
trajectory), so no stored value here comes from them. These files record what
the CPU oracle computes on two seeded tiny-model inputs, so that a later change
to the oracle's arithmetic shows up as a diff that its commit has to justify.
Only ``oracle`` and the seeded input generators in ``synth`` are called.

    python tests/golden/make_golden.py
"""
import json
import math
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import synth  # noqa: E402
from oracle import loop as ol  # noqa: E402
from oracle import model as om  # noqa: E402

# (file, lm_head_scale, tau): the tiny fp32 config as configured (every step refreshes) and
# the peaked fixture (LM head x 24, tau = 2.15 nats) whose trajectory mixes both branches
CASES = [("tiny_trajectory.json", 1.0, 0.5), ("tiny_peaked_trajectory.json", 24.0, 2.15)]


def trajectory(scale: float, tau: float) -> dict:
    cfg = synth.CONFIGS["tiny"]
    w = synth.make_model(cfg.model, lm_head_scale=scale)
    prompt = synth.make_prompt(cfg)
    recs, st, _ = ol.run_entropycache(om.OracleModel(w), cfg, prompt, tau)
    return {
        "config": "tiny", "lm_head_scale": scale, "tau": tau, "seed": cfg.seed,
        "steps": [{
            "t": r.t, "refreshed": bool(r.refreshed), "n_rows": int(len(r.rows)),
            "positions": [int(p) for p in r.picked], "ids": [int(i) for i in r.ids],
            "emax": float(r.emax), "refresh_next": bool(r.refresh_next),
        } for r in recs],
        "final_tokens": [int(x) for x in st.tokens],
    }


def main() -> None:
    for name, scale, tau in CASES:
        data = trajectory(scale, tau)
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(data, f, indent=1)
            f.write("\n")
        n_ref = sum(s["refreshed"] for s in data["steps"])
        print(f"{name}: {len(data['steps'])} steps, {n_ref} refreshes")


if __name__ == "__main__":
    main()
