"""The layer inside its pre-norm residual block, y = h + MoE(RMSNorm(h)) (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2: the MoE
layer replaces the FFN of the pre-norm block, H' = H~ + MoE(Norm(H~)).
"Sparse MoE FFN" (DeepSeek-V3), eq. 12 and "How it works": the skip is added
outside the MoE module.  "Mixture of experts and architecture families": the
norm is RMSNorm, a layer normalisation without mean-centering:
RMSNorm(x) = x / sqrt(mean_j x_j^2 + eps) * g.

Two forms: ``block_forward`` evaluates the layer on normalised rows (computed
here, or the ones a GPU stored); ``fused_block_forward`` is the block whose
normalisation is fused into the router and the first expert product: the
router decides on rs * (h . bf16(W_router * g)) (the precision in which that
kernel takes its decisions), while the expert outputs are those of the exact
fp64 RMSNorm.
"""
from __future__ import annotations

import numpy as np

from . import forward, router_logits, select, widen


def rmsnorm(h, g, eps):
    """Rows of h normalised by their root mean square, times g (fp64)."""
    x = widen(h)
    gw = widen(g)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * gw


def block_forward(h, g, eps, W_router, W1, W3, W2, k, *, un=None, **layer_kw):
    """(y, idx, gates, gap_e, gap_g) of the block.

    un: the normalised rows the layer is evaluated on; None computes them here
    in fp64.  A caller checking a GPU that stores them in a narrower type
    passes that GPU's own rows, so that both sides route on the same values.
    """
    u = rmsnorm(h, g, eps) if un is None else widen(un)
    y, idx, gates, gap_e, gap_g = forward(u, W_router, W1, W3, W2, k, **layer_kw)
    return y + widen(h), idx, gates, gap_e, gap_g


def bf16_round(x):
    """Nearest-even bfloat16 value of each element of x (fp64 in, fp64 out),
    for values exactly representable in fp32 (products of two bf16 values
    are): add half a bf16 ulp with ties to even to the fp32 bit pattern, then
    clear the low 16 bits."""
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def _one_expert_rows(x, W1, W3, W2, sel):
    """FFN_{sel[i]}(x[i]) for every row (fp64): the layer oracle at k = 1 with
    the selection forced, softmax gates (a single gate is exactly 1) and
    route scale 1.  The weights are passed as they are (bf16 bits are read
    exactly by the layer oracle)."""
    E, d = W1.shape[0], x.shape[1]
    y, _, g, _, _ = forward(x, np.zeros((E, d), dtype=W1.dtype), W1, W3, W2, 1,
                            forced_idx=np.asarray(sel).reshape(-1, 1), route_scale=1.0)
    assert np.all(g == 1.0)
    return y


def expert_sum(un, W1, W3, W2, idx, gates, shared=None):
    """shared(un) + sum_j gates[:, j] * FFN_{idx[:, j]}(un), j in order (fp64)."""
    x = widen(un)
    y = np.zeros_like(x)
    if shared is not None:
        W1s, W3s, W2s = (np.ascontiguousarray(a)[None] for a in shared)
        y += _one_expert_rows(x, W1s, W3s, W2s, np.zeros(x.shape[0], dtype=np.int64))
    for j in range(np.asarray(idx).shape[1]):
        y += np.asarray(gates, dtype=np.float64)[:, j:j + 1] * _one_expert_rows(x, W1, W3, W2, idx[:, j])
    return y


def fused_route(h, g, eps, W_router, k, *, bias=None, score_fn=0, n_groups=1, topk_groups=1,
                route_scale=1.0):
    """Routing of the block with the normalisation fused into the router: the
    RMSNorm weight folded into the router rows and rounded to bf16 (the
    precision the kernel decides in), and each token's logits scaled by its
    1/rms: l = rs * (h . bf16(W_router * g)), rs = 1 / sqrt(mean h^2 + eps).
    Returns (idx, gates, gap_expert, gap_group, logits)."""
    x = widen(h)
    rs = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    Wg = bf16_round(widen(W_router) * widen(g)[None, :])
    lg = router_logits(x, Wg) * rs[:, None]
    idx, gates, ge, gg = select(lg, k, score_fn, n_groups, topk_groups, route_scale, bias)
    return idx, gates, ge, gg, lg


def fused_block_forward(h, g, eps, W_router, W1, W3, W2, k, *, bias=None, shared=None, score_fn=0,
                        n_groups=1, topk_groups=1, route_scale=1.0, forced_idx=None):
    """(y, idx, gates, gap_e, gap_g) of the fused block: routing by fused_route
    (or forced_idx, gates still from its logits), and
    y = h + shared(RMSNorm(h)) + sum_j gate_j FFN_j(RMSNorm(h)), RMSNorm in
    fp64 with the exact norm weight."""
    idx, gates, ge, gg, lg = fused_route(h, g, eps, W_router, k, bias=bias, score_fn=score_fn,
                                         n_groups=n_groups, topk_groups=topk_groups, route_scale=route_scale)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int32)
        gates = gates_of(lg, idx, score_fn, route_scale)
    un = rmsnorm(h, g, eps)
    y = widen(h) + expert_sum(un, W1, W3, W2, idx, gates, shared)
    return y, idx, gates, ge, gg


def gates_of(logits, idx, score_fn, route_scale):
    """Gates of a given selection from the raw scores: softmax over the chosen
    logits (max-subtracted), or sigmoid scores over their sum, times
    route_scale."""
    lg = np.take_along_axis(np.asarray(logits, dtype=np.float64), np.asarray(idx, dtype=np.int64), 1)
    if score_fn == 1:
        s = 1.0 / (1.0 + np.exp(-lg))
        return route_scale * s / s.sum(axis=1, keepdims=True)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    return route_scale * z / z.sum(axis=1, keepdims=True)
