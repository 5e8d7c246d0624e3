"""The allocation-free forward (moe_layer_forward_noalloc), whose workspace is
the library's fixed per-GPU scratch array, against moe_layer_forward with a
caller-provided workspace: bitwise equal outputs on consecutive calls through
the C ABI, a prefill-shaped layer on the streaming kernels, then a smaller
decode-shaped one (which finds the first call's contents in the array), then
the first layer again."""
import sys

import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
from synthetic import Workload, make_inputs

pytestmark = pytest.mark.gpu

FIRST = Workload("noalloc_prefill", 1200, 512, 16, 4, 384, 256, "sigmoid", 4, 2, 2.5, "bf16", "uniform")
SECOND = Workload("noalloc_decode", 40, 256, 16, 4, 256, 256, "sigmoid", 4, 2, 2.5, "bf16", "uniform")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(inp, dev):
    return {k: (None if v is None else tuple(t.to(dev) for t in v) if isinstance(v, tuple) else v.to(dev))
            for k, v in inp.items()}


def both(w, inp, dev):
    cfg = moe.MoeConfig.from_workload(w)
    assert moe.moe_workspace_bytes(cfg) <= moe.NOALLOC_SCRATCH_BYTES
    ref = moe.moe_layer_forward(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                inp["shared"], cfg=cfg)
    # outputs start as garbage: the entry point must write every element
    y = torch.full_like(ref[0], 3.0)
    idx = torch.full_like(ref[1], -7)
    g = torch.full_like(ref[2], float("nan"))
    got = moe.moe_layer_forward_noalloc(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"],
                                        inp["W2"], inp["shared"], cfg=cfg, y=y, topk_idx=idx, gates=g)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_forward_matches_the_workspace_forward_on_calls_in_a_row():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    dev = torch.device("cuda:0")
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(FIRST))[0] == "stream"
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(SECOND))[0] == "stream_decode"
    a = to_dev(make_inputs(FIRST, seed=21, device="cpu"), dev)
    b = to_dev(make_inputs(SECOND, seed=22, device="cpu"), dev)
    for w, inp in ((FIRST, a), (SECOND, b), (FIRST, a)):
        log(f"[noalloc] {w.name} T={w.T}")
        ref, got = both(w, inp, dev)
        for x, y in zip(ref, got):
            assert torch.equal(x, y), w.name
        log(f"[noalloc] {w.name} bitwise equal to moe_layer_forward")
