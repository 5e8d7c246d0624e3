"""Second, independent oracle implementation: expert-major, NumPy float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  It shares nothing with
``moe_oracle.c`` except that both read the same inputs.

Routing follows "Mixture of experts and architecture families", "The router and
load balancing": softmax over all E logits, top-k of the probabilities,
renormalise the k weights.  At zero bias this selects the same experts as the
raw-logit route of "Mixture of Experts and Hybrid Architectures", "The router in
code" (softmax is monotone) and a renormalised subset of a softmax equals a
softmax over that subset, so the two oracles must agree.

The expert pass is expert-major, in the dispatch / combine form the "Sparse
MoE FFN" page describes in "Packed forward" (gather each expert's tokens, run
it once on them, scatter-add the weighted result): the T*k (token, slot) pairs
are flattened, grouped by expert, each expert runs once on its gathered rows
as a batched matrix product, and the gate-weighted rows are scattered back
into the output with an unbuffered add.  Experts are SwiGLU ("Sparse MoE FFN"
(DeepSeek-V3), "How it works"):
W2 (SiLU(W1 x) * W3 x); or GEGLU, GELU in place of SiLU (named beside SwiGLU
in the cheat sheet's "Calculator defaults"); or the biased GELU
MLP of "Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2:
W2 GELU(W1 x + b1) + b2, with GELU(x) = x Phi(x) (SciPy's erf here).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

from . import GEGLU, GELU_MLP, SWIGLU, widen


def silu(x):
    return x / (1.0 + np.exp(-x))


def gelu(x):
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def swiglu(x, W1, W3, W2):
    """Rows x [n][d]; W1, W3 [F][d]; W2 [d][F] -> [n][d] (NumPy matmuls)."""
    return (silu(x @ W1.T) * (x @ W3.T)) @ W2.T


def expert(x, kind, W1, W3, W2, b1=None, b2=None):
    """One expert of the given body on rows x [n][d] -> [n][d]."""
    if kind == SWIGLU:
        return swiglu(x, W1, W3, W2)
    if kind == GEGLU:
        return (gelu(x @ W1.T) * (x @ W3.T)) @ W2.T
    assert kind == GELU_MLP
    a = x @ W1.T
    if b1 is not None:
        a = a + b1
    o = gelu(a) @ W2.T
    return o if b2 is None else o + b2


def softmax_router(u, W_router, k):
    """Softmax over all experts, top-k (stable, ties -> lower index), renormalise."""
    logits = u @ W_router.T
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    idx = np.argsort(-p, axis=1, kind="stable")[:, :k]
    w = np.take_along_axis(p, idx, axis=1)
    w = w / w.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w


def _w(a):
    return None if a is None else widen(a)


def layer(u, W_router, W1, W3, W2, k, shared=None, idx=None, gates=None, kind=SWIGLU,
          b1=None, b2=None):
    """Expert-major layer output.  With idx/gates None the softmax router above
    chooses; otherwise the given selection and gates are used (so the expert
    pass can also be checked under sigmoid, group-limited routing).
    shared is (W1s, W3s, W2s[, b1s, b2s]); W3 is None for the GELU MLP."""
    x = widen(u)
    W1, W3, W2, b1, b2 = (_w(a) for a in (W1, W3, W2, b1, b2))
    if idx is None:
        idx, gates = softmax_router(x, widen(W_router), k)
    idx = np.asarray(idx, dtype=np.int64)
    gates = np.asarray(gates, dtype=np.float64)
    n_tok, n_slot = idx.shape
    # dispatch: one entry per (token, slot) pair, flattened
    tok_of = np.repeat(np.arange(n_tok), n_slot)
    exp_of = idx.reshape(-1)
    wgt_of = gates.reshape(-1)
    y = np.zeros((n_tok, x.shape[1]))
    for e in np.unique(exp_of):
        (pairs,) = np.nonzero(exp_of == e)
        toks = tok_of[pairs]
        ye = expert(x[toks], kind, W1[e], None if W3 is None else W3[e], W2[e],
                    None if b1 is None else b1[e], None if b2 is None else b2[e])
        # combine: scatter-add each pair's weighted row into its token
        np.add.at(y, toks, wgt_of[pairs, None] * ye)
    if shared is not None:
        sw = [_w(a) for a in shared]
        sw += [None] * (5 - len(sw))
        y += expert(x, kind, *sw)
    return y, idx.astype(np.int32), gates
