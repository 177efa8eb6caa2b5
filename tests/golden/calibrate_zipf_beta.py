"""Derive the bias scale beta of the Zipf-skewed workload.

The skewed long-context workload gives expert e the router bias
b_e = -beta * ln(r_e), r a seeded permutation of 1..E, so that expert
popularity falls off as a power of its rank.  beta is chosen by bisection so
that the least-squares slope of log(top-k count) against log(rank) is -1.1 on
8192 tokens with iid N(0, 1) logits (seed 1).  Exact top-8 Zipf(1.1) shares
are infeasible (the head expert would need more than all tokens), so the
slope is the matched quantity.

Run:  python tests/golden/calibrate_zipf_beta.py   -> writes zipf_beta.json
Uses only the oracle's top-k selection.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
import oracle  # noqa: E402

E, K, T, TARGET = 384, 8, 8192, -1.1


def slope(beta, logits, rank):
    b = (-beta * np.log(rank)).astype(np.float32)
    idx = oracle.route_topk(logits, b, K)
    cnt = np.bincount(idx.reshape(-1), minlength=E)
    used = cnt > 0
    x, y = np.log(rank[used]), np.log(cnt[used])
    return float(np.polyfit(x, y, 1)[0]), int(used.sum())


def main():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    rank = np.arange(1, E + 1, dtype=np.float64)
    lo, hi = 0.0, 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        s, _ = slope(mid, logits, rank)
        if s > TARGET:
            lo = mid
        else:
            hi = mid
    beta = round(0.5 * (lo + hi), 4)
    s, used = slope(beta, logits, rank)
    out = dict(beta=beta, slope=round(s, 4), experts_used=used, tokens=T,
               seed=1, target_slope=TARGET)
    with open(os.path.join(HERE, "zipf_beta.json"), "w") as f:
        json.dump(out, f, indent=1)
    print(out)


if __name__ == "__main__":
    main()
