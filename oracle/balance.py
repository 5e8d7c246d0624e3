"""Auxiliary-loss-free balance loop and routing entropy (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Mixture of Experts and Hybrid Architectures", "Aux-loss-free balance loop":
start from a zero bias; target usage is n_tokens * top_k / n_experts; route by
scores + bias; count how often each expert fires; an expert over target has
its bias lowered by gamma, one under target raised by gamma; the page's demo
uses gamma = 0.15 for 10 iterations; entropy of the usage should rise toward
ln(n_experts).  An expert exactly on target keeps its bias (the page states
only the two strict cases).

Logits do not depend on the bias, so they are computed once and selection is
re-run with each new bias.
"""
from __future__ import annotations

import math

import numpy as np

from . import SOFTMAX, select


def usage(idx, E):
    """How often each expert fires over all (token, slot) pairs."""
    return np.bincount(np.asarray(idx).reshape(-1), minlength=E)


def entropy(counts):
    """Shannon entropy (nats) of the usage distribution; max is ln(E)."""
    c = np.asarray(counts, dtype=np.float64)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log(p)).sum())


def update_bias(bias, counts, target, gamma=0.15):
    """One step: over target -> bias - gamma, under -> bias + gamma."""
    b = np.array(bias, dtype=np.float64)
    b[counts > target] -= gamma
    b[counts < target] += gamma
    return b


def update_step_fp32(idx, E, bias32, gamma32):
    """One balance step in the precision a GPU keeps the bias in.

    idx: the routing of one batch (any shape); entries outside [0, E) are not
    counted but still count in S = idx.size, the number of (token, slot)
    pairs.  target = S / E; the comparisons are made exactly, as count * E
    against S.  The bias update is done in fp64 on the fp32 bias and gamma
    (exact for values of this size) and rounded once to fp32.  The entropy is
    -sum p ln p with p = count / S (0 when S == 0).

    Returns (new bias fp32 [E], counts int64 [E], entropy fp64)."""
    flat = np.asarray(idx).reshape(-1)
    S = flat.size
    counts = np.bincount(flat[(flat >= 0) & (flat < E)].astype(np.int64), minlength=E)
    ce = counts * E
    b = np.asarray(bias32, dtype=np.float32).astype(np.float64)
    g = float(np.float32(gamma32))
    b[ce > S] -= g
    b[ce < S] += g
    if S > 0:
        p = counts[counts > 0] / S
        ent = float(-(p * np.log(p)).sum())
    else:
        ent = 0.0
    return b.astype(np.float32), counts, ent


def balance_bias(logits, k, gamma=0.15, iterations=10, score_fn=SOFTMAX, n_groups=1,
                 topk_groups=1, nthreads=None):
    """Run the loop on fixed logits [T][E].

    Returns (bias fp64 [E], history) where history holds, per iteration, the
    usage counts and entropy measured before that iteration's update, plus the
    final usage after the last update."""
    T, E = logits.shape
    target = T * k / E
    b = np.zeros(E, dtype=np.float64)
    history = []
    for _ in range(iterations):
        idx, _, _, _ = select(logits, k, score_fn, n_groups, topk_groups, 1.0, b,
                              nthreads=nthreads)
        c = usage(idx, E)
        history.append({"counts": c, "entropy": entropy(c)})
        b = update_bias(b, c, target, gamma)
    idx, _, _, _ = select(logits, k, score_fn, n_groups, topk_groups, 1.0, b, nthreads=nthreads)
    c = usage(idx, E)
    history.append({"counts": c, "entropy": entropy(c)})
    return b, history


def max_entropy(E):
    return math.log(E)
