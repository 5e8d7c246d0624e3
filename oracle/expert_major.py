"""Second, independent oracle implementation: expert-major, NumPy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It shares nothing with
``moe_oracle.c`` except that both read the same inputs.

Routing follows "Mixture of experts and architecture families", "The router and
load balancing": softmax over all E logits, top-k of the probabilities,
renormalise the k weights.  At zero bias this selects the same experts as the
raw-logit route of "Mixture of Experts and Hybrid Architectures", "The router in
code" (softmax is monotone) and a renormalised subset of a softmax equals a
softmax over that subset, so the two oracles must agree.

The expert loop is the same page's masked loop: for each expert, take the rows
whose selection contains it, run the expert on those rows, weight and add.
Experts are SwiGLU ("Sparse MoE FFN" (DeepSeek-V3), "How it works"):
W2 (SiLU(W1 x) * W3 x).
"""
from __future__ import annotations

import numpy as np

from . import widen


def silu(x):
    return x / (1.0 + np.exp(-x))


def swiglu(x, W1, W3, W2):
    """Rows x [n][d]; W1, W3 [F][d]; W2 [d][F] -> [n][d] (NumPy matmuls)."""
    return (silu(x @ W1.T) * (x @ W3.T)) @ W2.T


def softmax_router(u, W_router, k):
    """Softmax over all experts, top-k (stable, ties -> lower index), renormalise."""
    logits = u @ W_router.T
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, idx, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w


def layer(u, W_router, W1, W3, W2, k, shared=None, idx=None, gates=None):
    """Expert-major layer output.  With idx/gates None the softmax router above
    chooses; otherwise the given selection and gates are used (so the expert
    loop can also be checked under sigmoid, group-limited routing)."""
    u = widen(u)
    W1, W3, W2 = widen(W1), widen(W3), widen(W2)
    if idx is None:
        idx, gates = softmax_router(u, widen(W_router), k)
    out = np.zeros_like(u)
    for e in range(W1.shape[0]):
        mask = idx == e
        rows = mask.any(axis=1)
        if rows.any():
            w = (gates * mask)[rows].sum(axis=1, keepdims=True)
            out[rows] += w * swiglu(u[rows], W1[e], W3[e], W2[e])
    if shared is not None:
        W1s, W3s, W2s = (widen(a) for a in shared)
        out += swiglu(u, W1s, W3s, W2s)
    return out, idx, gates
