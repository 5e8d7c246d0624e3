"""The layer forward captured in a HIP graph (through torch.cuda.graph) replays
bitwise equal to the eager call.

The forward allocates nothing, synchronises nothing and clears its own work
counters with a kernel, so a caller can capture it.  Each replay is preceded
by eager work on the same buffers (they are overwritten), and every replay is
checked against the eager result.
"""
import sys

import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
from synthetic import Workload, make_inputs

pytestmark = pytest.mark.gpu

SHAPES = {
    # prefill streaming kernels (packed weights), shared expert, groups
    "stream_groups_shared": (Workload("stream_groups_shared", 1200, 512, 16, 4, 512, 256, "sigmoid", 4, 2, 2.5,
                                      "bf16", "uniform"), "stream", True),
    # decode streaming kernels (packed weights)
    "decode_groups_shared": (Workload("decode_groups_shared", 40, 256, 16, 4, 256, 256, "sigmoid", 4, 2, 2.5,
                                      "bf16", "uniform"), "stream_decode", True),
    # tiled fp32 kernels (plain weights)
    "tiled_fp32": (Workload("tiled_fp32", 200, 128, 16, 3, 128, 64, "sigmoid", 4, 2, 2.5, "f32", "uniform"),
                   "tiled", False),
    # the one-kernel small fp32 layer
    "small_fp32": (Workload("small_fp32", 100, 128, 16, 3, 128, 64, "sigmoid", 4, 2, 2.5, "f32", "uniform"),
                   "small", False),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # fails loudly when libmoe.so is missing
    return torch.device("cuda:0")


@pytest.mark.parametrize("name", list(SHAPES))
def test_captured_layer_replays_bitwise(dev, name):
    w, path, packed_weights = SHAPES[name]
    cfg = moe.MoeConfig.from_workload(w)
    assert moe.moe_plan_describe(cfg)[0] == path
    log(f"[graph] {name} ({path})")
    inp = make_inputs(w, seed=5, device=dev)
    packed = (moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
              if packed_weights else None)
    y = torch.empty((w.T, w.d), dtype=cfg.torch_dtype, device=dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(cfg, dev)

    def step():
        if packed is not None:
            moe.moe_layer_forward_packed(inp["u"], inp["W_router"], inp["bias"], packed, cfg=cfg, y=y,
                                         topk_idx=idx, gates=gates, workspace=ws)
        else:
            moe.moe_layer_forward(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                  inp["shared"], cfg=cfg, y=y, topk_idx=idx, gates=gates, workspace=ws)

    step()
    torch.cuda.synchronize()
    y_ref, idx_ref, g_ref = y.clone(), idx.clone(), gates.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for r in range(3):
        # eager work on the same buffers between replays
        y.fill_(7)
        idx.fill_(-1)
        gates.fill_(-1.0)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, idx_ref), f"replay {r}: topk_idx differs"
        assert torch.equal(gates, g_ref), f"replay {r}: gates differ"
        assert torch.equal(y, y_ref), f"replay {r}: y differs"
    log(f"[graph] {name}: 3 replays bitwise equal to the eager call")
