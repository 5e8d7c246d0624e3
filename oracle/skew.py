"""Calibration of the skewed-load workload (fp64, oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The troubleshooting table of "Mixture of Experts and Hybrid Architectures"
names the symptom "90% of tokens go to one expert".  The skewed workload
reproduces it: inputs carry a common direction m (u_t = z_t + mu m) and the
router row of expert 0 is alpha m, with alpha chosen here so that the share of
tokens whose top-k contains expert 0 (zero bias) is 0.90.  Expert 0 makes a
token's top-k when its logit ranks among the k largest, ties going to the
lower index, so when alpha * a_t >= the k-th largest of the other logits.
"""
from __future__ import annotations

import numpy as np


def expert0_share(alpha, a, kth_other):
    """Share of tokens selecting expert 0 when its logit is alpha * a."""
    return float(np.mean(alpha * a >= kth_other))


def calibrate_expert0_scale(logits_other, a, k, target=0.90, lo=0.0, hi=64.0, iters=60):
    """alpha with expert0_share(alpha) closest to target (bisection).

    logits_other: [T][E-1] fp64 logits of experts 1..E-1; a: [T] = u_t . m."""
    kth = -np.sort(-np.asarray(logits_other, dtype=np.float64), axis=1)[:, k - 1]
    a = np.asarray(a, dtype=np.float64)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if expert0_share(mid, a, kth) < target:
            lo = mid
        else:
            hi = mid
    return hi
