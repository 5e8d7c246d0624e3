"""GPU parity of the on-device balance update (moe_balance_update) against the
oracle's fp32 step ("Mixture of Experts and Hybrid Architectures",
"Aux-loss-free balance loop"): counts exact, bias bit-exact, entropy to fp32
rounding."""
import math
import sys

import numpy as np
import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
import oracle
from oracle import balance
from synthetic import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu
GAMMA = np.float32(0.15)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


def step_both(idx, E, bias, dev):
    """One update on the GPU and in the oracle from the same routing and bias."""
    b_gpu = torch.from_numpy(bias.copy()).to(dev)
    counts, ent = moe.moe_balance_update(torch.from_numpy(idx).to(dev), b_gpu, E=E, gamma=float(GAMMA))
    torch.cuda.synchronize()
    b_ref, c_ref, h_ref = balance.update_step_fp32(idx, E, bias, GAMMA)
    return (b_gpu.cpu().numpy(), counts.cpu().numpy(), float(ent.cpu()[0])), (b_ref, c_ref, h_ref)


def check(gpu, ref):
    (b, c, h), (br, cr, hr) = gpu, ref
    assert np.array_equal(c, cr), "counts"
    assert np.array_equal(b.view(np.uint32), br.view(np.uint32)), "bias bits"
    assert h == pytest.approx(hr, rel=2e-7, abs=1e-7)


@pytest.mark.parametrize("T,k,E,skew", [(8192, 8, 256, 0.0), (8192, 8, 256, 3.0), (16384, 8, 128, 6.0),
                                        (4096, 2, 8, 0.0), (333, 6, 32, 1.0), (1, 1, 4, 0.0), (64, 4, 1, 0.0)])
def test_balance_step_matches_oracle(dev, T, k, E, skew):
    rng = np.random.default_rng(T * 7 + E)
    w = np.exp(skew * rng.standard_normal(E))
    idx = np.stack([rng.choice(E, size=k, replace=False, p=w / w.sum()) if k <= E else
                    rng.integers(0, E, k) for _ in range(T)]).astype(np.int32)
    bias = (rng.integers(-8, 8, E) * GAMMA).astype(np.float32)
    gpu, ref = step_both(idx, E, bias, dev)
    check(gpu, ref)
    log(f"[balance] T={T} k={k} E={E} skew={skew}: entropy {gpu[2]:.6f} (ln E {math.log(E):.6f})")


def test_balance_step_edge_cases(dev):
    # entries outside [0, E) are not counted but stay in T*k
    idx = np.array([[0, 9], [-3, 1], [1, 1]], np.int32)
    check(*step_both(idx, 4, np.zeros(4, np.float32), dev))
    # no tokens: counts zero, entropy 0, bias kept
    b = torch.full((5,), 0.3, device=dev)
    counts, ent = moe.moe_balance_update(torch.empty((0, 2), dtype=torch.int32, device=dev), b, E=5)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 5 and float(ent.cpu()[0]) == 0.0
    assert torch.equal(b.cpu(), torch.full((5,), 0.3))


def test_balance_loop_on_gpu_routing_raises_entropy(dev):
    """The pages' loop run on the device: route the skewed layer with the
    current bias, update, repeat 10 times.  Every step matches the oracle's
    step on the same routing, and the usage entropy rises toward ln E."""
    w = WORKLOADS["skewed_e128_top8"].with_(T=4096, d=256, F=128, Fs=128)
    inp = make_inputs(w, seed=0, device=dev, expert0_scale=2.5)
    cfg = moe.MoeConfig.from_workload(w)
    bias = torch.zeros(w.E, dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(cfg, dev)
    ents = []
    for it in range(10):
        idx, *_ = moe.moe_route_debug(inp["u"], inp["W_router"], bias, cfg=cfg, workspace=ws)
        b_before = bias.cpu().numpy().copy()
        counts, ent = moe.moe_balance_update(idx, bias, E=w.E)
        torch.cuda.synchronize()
        ref = balance.update_step_fp32(idx.cpu().numpy(), w.E, b_before, GAMMA)
        check((bias.cpu().numpy(), counts.cpu().numpy(), float(ent.cpu()[0])), ref)
        ents.append(float(ent.cpu()[0]))
    log(f"[balance] loop entropies {[round(e, 4) for e in ents]} ln E {math.log(w.E):.4f}")
    assert ents[-1] > ents[0] + 0.02
    assert max(ents) <= math.log(w.E) + 1e-6


def test_balance_step_on_full_size_routing(dev):
    """The DeepSeek-V3-shaped prefill layer's own routing (T = 8192, k = 8,
    E = 256, 8 groups keep 4) through one update."""
    w = WORKLOADS["dsv3_prefill"]
    inp = make_inputs(w, seed=0, device=dev)
    cfg = moe.MoeConfig.from_workload(w)
    idx, *_ = moe.moe_route_debug(inp["u"], inp["W_router"], inp["bias"], cfg=cfg)
    bias = inp["bias"].cpu().numpy().copy()
    check(*step_both(idx.cpu().numpy(), w.E, bias, dev))
