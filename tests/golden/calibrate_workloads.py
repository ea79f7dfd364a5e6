"""Fit the two structural constants of the synthetic workloads with the CPU
oracle and write them to ``workload_calibration.json``.

  * TIE_PAIRS: how many twin expert pairs (identical W rows and bias, inside
    one group) the DeepSeek-V3 prefill workload gets, so that an exact tie
    decides the selection (exactly one twin of a pair selected) for about 1%
    of tokens.
  * HOT_SHIFT: the bias shift of the 16 hot experts (2 per group) in the
    skewed DeepSeek-V3 workload, so that 50% +- 1% of all (token, slot) pairs
    go to hot experts.

Both are measured on the first 4096 tokens at seed 0.  Only the oracle and the
seeded input generator are called.  Run: python tests/golden/calibrate_workloads.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from sigmoid_group_limited_amd import workloads as wl  # noqa: E402

N_TOKENS = 4096
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workload_calibration.json")


def decisive_tie_fraction(o, T, pairs):
    cfg = wl.DSV3
    gi = wl.make_gate_inputs(T, wl.D_MODEL, cfg, seed=0, tie_pairs=pairs)
    r = o.gate(gi.x, gi.W, gi.bias, cfg.n_group, cfg.topk_group, cfg.top_k,
               cfg.route_scale)
    decisive = np.zeros(T, dtype=bool)
    for a, b in gi.twins:
        has_a = (r.indices == a).any(axis=1)
        has_b = (r.indices == b).any(axis=1)
        decisive |= has_a ^ has_b
    return float(decisive.mean())


def hot_share(o, logits, bias0, hot, shift):
    cfg = wl.DSV3
    b = bias0.copy()
    b[hot] = (b[hot] + np.float32(shift)).astype(np.float32)
    r = o.select(logits, b, cfg.n_group, cfg.topk_group, cfg.top_k, cfg.route_scale)
    return float(np.isin(r.indices, hot).mean())


def main():
    o = oracle.load()
    ties = {}
    for p in range(1, 7):
        ties[p] = decisive_tie_fraction(o, N_TOKENS, p)
        print(f"tie pairs {p}: decisive fraction {ties[p]:.4f}", flush=True)
    best_p = min(ties, key=lambda p: abs(ties[p] - 0.01))

    cfg = wl.DSV3
    gi = wl.make_gate_inputs(N_TOKENS, wl.D_MODEL, cfg, seed=0, hot_per_group=2,
                             hot_shift=0.0)
    logits = o.logits(gi.x, gi.W)
    lo, hi = 0.0, 1.0
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        if hot_share(o, logits, gi.bias, gi.hot, mid) < 0.5:
            lo = mid
        else:
            hi = mid
    shift = round(0.5 * (lo + hi), 4)
    share = hot_share(o, logits, gi.bias, gi.hot, shift)
    print(f"hot shift {shift}: hot share {share:.4f}", flush=True)

    result = {
        "tokens": N_TOKENS,
        "seed": 0,
        "tie_pairs": best_p,
        "tie_decisive_fraction": ties,
        "hot_shift": shift,
        "hot_share": share,
        "hot_experts": [int(h) for h in gi.hot],
        "produced_by": "tests/golden/calibrate_workloads.py (CPU oracle only)",
    }
    with open(OUT, "w") as f:
        json.dump(result, f, indent=2, sort_keys=True)
        f.write("\n")
    print(json.dumps(result, indent=2, sort_keys=True))


if __name__ == "__main__":
    main()
