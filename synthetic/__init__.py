"""Seeded synthetic workloads for the sparse MoE feed-forward layer.

Shared by the tests, the smoke check and the benchmark.  This module only
draws random tensors of the right shapes and scales; it holds none of the
layer's arithmetic (no routing, no expert, no combine), so the GPU path and
the CPU oracle can both be fed from it without sharing any computation.

Recipe (every tensor):
  * its own ``torch.Generator`` on ``device``, seeded from (seed, tensor id):
    u 0, W_router 1, W1 2, W3 3, W2 4, W1s 5, W3s 6, W2s 7, bias 8, skew
    direction 9;
  * ``torch.randn`` in fp32 (expert weights drawn expert by expert, so the
    transient buffer is one expert's matrix);
  * weights scaled by 1/sqrt(fan_in): d for W_router, W1, W3, W1s, W3s; F for
    W2; Fs for W2s; u ~ N(0, 1);
  * rounded to the workload's dtype (bf16 round-to-nearest-even, or fp32).
  * bias: zero, or U(-0.05, 0.05) fp32 for the DeepSeek-V3-shaped layers, or
    a vector the caller passes in.
  * skewed layer: u_t = z_t + 2 m with m a seeded unit vector, and router row
    0 replaced by ``expert0_scale`` * m when the caller passes that scale.
  * block form: u is the block input h; the RMSNorm weight is 1 + 0.1 N(0, 1)
    (``make_norm_weight``, tensor id 10).
  * biased GELU-MLP experts (``make_ffn_biases``): b1 ~ 0.5 N(0, 1) [E][F],
    b2 ~ 0.1 N(0, 1) [E][d], b1s, b2s likewise for the shared expert (tensor
    ids 11-14), in the workload's dtype.

The same (workload, seed, device) always gives the same tensors.  Draws on
"cpu" and on "cuda" differ from each other; each test states which it uses.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional

import torch

TENSOR_IDS = {"u": 0, "W_router": 1, "W1": 2, "W3": 3, "W2": 4, "W1s": 5, "W3s": 6,
              "W2s": 7, "bias": 8, "skew_dir": 9, "norm_weight": 10, "b1": 11, "b2": 12,
              "b1s": 13, "b2s": 14}


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    Fs: int            # 0: no shared expert
    score_fn: str      # "softmax" | "sigmoid"
    n_groups: int
    topk_groups: int
    route_scale: float
    dtype: str         # "f32" | "bf16"
    bias: str          # "zero" | "uniform"
    skew: bool = False
    skew_shift: float = 2.0

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def flops(self) -> float:
        """Algorithmic FLOPs of one layer call: router + k routed SwiGLUs + shared."""
        return float(self.T) * (2.0 * self.d * self.E + 6.0 * self.d * self.F * self.k
                                + 6.0 * self.d * self.Fs)


WORKLOADS = {
    # small fp32 layer the oracle finishes in milliseconds
    "tiny_fp32": Workload("tiny_fp32", 64, 64, 8, 2, 128, 0, "softmax", 1, 1, 1.0, "f32", "zero"),
    # Mixtral-style: 8 experts, top-2, softmax over the two raw scores
    "mixtral_e8_top2": Workload("mixtral_e8_top2", 4096, 4096, 8, 2, 14336, 0, "softmax", 1, 1,
                                1.0, "bf16", "zero"),
    # DeepSeek-V3-shaped prefill: 256 routed + 1 shared, sigmoid, 8 groups keep 4, x2.5
    "dsv3_prefill": Workload("dsv3_prefill", 8192, 7168, 256, 8, 2048, 2048, "sigmoid", 8, 4, 2.5,
                             "bf16", "uniform"),
    # same layer at decode shape
    "dsv3_decode": Workload("dsv3_decode", 64, 7168, 256, 8, 2048, 2048, "sigmoid", 8, 4, 2.5,
                            "bf16", "uniform"),
    # skewed load: 128 experts, top-8, 1 shared, expert 0 favoured
    "skewed_e128_top8": Workload("skewed_e128_top8", 16384, 2048, 128, 8, 768, 768, "softmax", 1, 1,
                                 1.0, "bf16", "zero", skew=True),
}


# One GPU's share of the DeepSeek-V3 layer under expert parallelism over 8
# GPUs: 32 local experts that receive about 2048 token rows each (8192
# local tokens x top-8 over 32 experts), plus the replicated shared expert on
# the local tokens.  Measured as an extra shape, not a parity workload.
EP_SHARD = Workload("ep_shard_e32", 8192, 7168, 32, 8, 2048, 2048, "sigmoid", 1, 1, 2.5, "bf16", "uniform")


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + TENSOR_IDS[name] + 1)
    return g


def _randn(shape, gen, device, scale, dtype):
    x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def _experts(E, rows, cols, seed, name, device, scale, dtype):
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    g = _gen(seed, name, device)
    for e in range(E):
        out[e].copy_(_randn((rows, cols), g, device, scale, dtype))
    return out


def torch_dtype(w: Workload):
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def _make_u(w: Workload, seed, dev):
    u = _randn((w.T, w.d), _gen(seed, "u", dev), dev, 1.0, torch.float32)
    m = None
    if w.skew:
        m = torch.randn(w.d, generator=_gen(seed, "skew_dir", dev), device=dev,
                        dtype=torch.float32)
        m = m / m.norm()
        u = u + w.skew_shift * m
    return u.to(torch_dtype(w)), m


def make_norm_weight(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """RMSNorm weight of the block form: 1 + 0.1 N(0, 1) per hidden unit, in
    the workload's dtype."""
    dev = torch.device(device)
    g = 1.0 + _randn((w.d,), _gen(seed, "norm_weight", dev), dev, 0.1, torch.float32)
    return g.to(torch_dtype(w))


def make_ffn_biases(w: Workload, seed: int = 0, device="cpu") -> dict:
    """Additive biases of the GELU-MLP expert body: b1 [E][F], b2 [E][d], and
    b1s [Fs], b2s [d] when the layer has a shared expert (else None)."""
    dev = torch.device(device)
    dt = torch_dtype(w)
    out = {"b1": _randn((w.E, w.F), _gen(seed, "b1", dev), dev, 0.5, dt),
           "b2": _randn((w.E, w.d), _gen(seed, "b2", dev), dev, 0.1, dt),
           "b1s": None, "b2s": None}
    if w.Fs > 0:
        out["b1s"] = _randn((w.Fs,), _gen(seed, "b1s", dev), dev, 0.5, dt)
        out["b2s"] = _randn((w.d,), _gen(seed, "b2s", dev), dev, 0.1, dt)
    return out


def make_u(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    """The token inputs of ``w`` alone (same draw as in make_inputs)."""
    return _make_u(w, seed, torch.device(device))[0]


def make_inputs(w: Workload, seed: int = 0, device="cpu", bias: Optional[torch.Tensor] = None,
                expert0_scale: Optional[float] = None) -> dict:
    """All inputs of one layer call as torch tensors on ``device``.

    bias: overrides the workload's bias recipe (fp32 [E]).  expert0_scale: for
    skewed workloads, router row 0 becomes expert0_scale * m."""
    dt = torch_dtype(w)
    dev = torch.device(device)
    T, d, E, F, Fs = w.T, w.d, w.E, w.F, w.Fs
    u, m = _make_u(w, seed, dev)
    Wr = _randn((E, d), _gen(seed, "W_router", dev), dev, 1.0 / math.sqrt(d), torch.float32)
    if w.skew and expert0_scale is not None:
        Wr[0] = float(expert0_scale) * m
    Wr = Wr.to(dt)
    W1 = _experts(E, F, d, seed, "W1", dev, 1.0 / math.sqrt(d), dt)
    W3 = _experts(E, F, d, seed, "W3", dev, 1.0 / math.sqrt(d), dt)
    W2 = _experts(E, d, F, seed, "W2", dev, 1.0 / math.sqrt(F), dt)
    shared = None
    if Fs > 0:
        W1s = _randn((Fs, d), _gen(seed, "W1s", dev), dev, 1.0 / math.sqrt(d), dt)
        W3s = _randn((Fs, d), _gen(seed, "W3s", dev), dev, 1.0 / math.sqrt(d), dt)
        W2s = _randn((d, Fs), _gen(seed, "W2s", dev), dev, 1.0 / math.sqrt(Fs), dt)
        shared = (W1s, W3s, W2s)
    if bias is not None:
        b = bias.to(device=dev, dtype=torch.float32)
    elif w.bias == "uniform":
        b = (torch.rand(E, generator=_gen(seed, "bias", dev), device=dev,
                        dtype=torch.float32) * 0.1 - 0.05)
    else:
        b = torch.zeros(E, dtype=torch.float32, device=dev)
    out = {"u": u, "W_router": Wr, "bias": b, "W1": W1, "W3": W3, "W2": W2, "shared": shared}
    if m is not None:
        out["skew_dir"] = m
    return out


def to_numpy(t: torch.Tensor):
    """Exact host copy for the oracle: bf16 as uint16 bit patterns, fp32 as is."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view("uint16")
    return t.cpu().numpy()
