"""The layer inside its pre-norm residual block, y = h + MoE(RMSNorm(h)) (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

"Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2: the MoE
layer replaces the FFN of the pre-norm block, H' = H~ + MoE(Norm(H~)).
"Sparse MoE FFN" (DeepSeek-V3), eq. 12 and "How it works": the skip is added
outside the MoE module.  "Mixture of experts and architecture families": the
norm is RMSNorm, a layer normalisation without mean-centering:
RMSNorm(x) = x / sqrt(mean_j x_j^2 + eps) * g.
"""
from __future__ import annotations

import numpy as np

from . import forward, widen


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
