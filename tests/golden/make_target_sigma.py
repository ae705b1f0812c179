"""Write target_sigma.json: per-position target-noise std for the verify workloads.

The batched-verify workload draws target logits as draft logits plus N(0, sigma_k^2),
with sigma_k chosen so that the mean acceptance probability falls linearly from 0.9 at
position 1 to 0.5 at position 16. The mean acceptance probability of a position is the
mean TV label c* = sum_v min(p_d, p_t) (the analytic acceptance rate of [P3] "DSpark
Speculative Decoding", section "Confidence-Scheduled Verification"), so sigma_k is found
by bisection on the oracle's c* over 32 fixed calibration rows drawn with the workload's
value recipe (N(0, 3^2) logits, 32 ids raised by +8).

Calls only the oracle and the seeded generators. Run from the repository root:
    python tests/golden/make_target_sigma.py
"""
import json
import os
import sys
from multiprocessing import Pool

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth   # noqa: E402

GAMMA = 16
ROWS = 32
CAL_CFG = {151936: 100, 129280: 101}


def targets():
    return [0.9 - 0.4 * (k - 1) / (GAMMA - 1) for k in range(1, GAMMA + 1)]


def _rows(V):
    c = synth.custom(CAL_CFG[V], B=ROWS, V=V, r=1, gamma=0)
    base = np.stack([synth.base_rows(c, b)[0] for b in range(ROWS)])
    z = np.stack([synth.rng(c.seed, synth.T_TNOISE, b).standard_normal(V, dtype=np.float32)
                  for b in range(ROWS)])
    return base, z


def mean_cstar(base, z, sigma):
    tgt = (base + z * np.float32(sigma)).astype(np.float32)
    return float(np.mean([oracle.tv_row_pair(base[i], tgt[i]) for i in range(base.shape[0])]))


def solve(args):
    V, t = args
    base, z = _rows(V)
    lo, hi = 1e-3, 20.0          # c*(lo) > t > c*(hi); c* falls as sigma grows
    for _ in range(24):
        mid = np.sqrt(lo * hi)
        if mean_cstar(base, z, mid) > t:
            lo = mid
        else:
            hi = mid
    return V, t, float(np.sqrt(lo * hi))


def main():
    jobs = [(V, t) for V in CAL_CFG for t in targets()]
    with Pool(min(8, os.cpu_count() or 1)) as pool:
        res = pool.map(solve, jobs)
    sig = {str(V): [s for (VV, _, s) in res if VV == V] for V in CAL_CFG}
    out = dict(
        sigma=sig,
        target_mean_cstar=targets(),
        calibration=f"{ROWS} rows per vocabulary, synth.custom(seed={CAL_CFG}), "
                    "bisection in log sigma, 24 steps",
        written_by="tests/golden/make_target_sigma.py (oracle.tv_row_pair only)",
    )
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "target_sigma.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(sig))


if __name__ == "__main__":
    main()
