"""GPU parity of the other expert bodies (GEGLU and the biased GELU MLP)
against the CPU oracle, through moe_layer_forward_ex.

Routing does not depend on the body, so each call's top-k and gates must
equal those of the SwiGLU entry point bitwise (the same router kernel); they
are also checked against the oracle's own routing of every token, and the
outputs token by token against the oracle's, which runs on its own selection
(on the GPU's for a near-tie token that the GPU broke the other way).  Every
kernel path is covered: tiled fp32 and bf16, the streaming prefill kernels and their decode
variant, and the GELU MLP's fallback to the tiled kernels when F is not a
multiple of 256.
"""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
import oracle
from parity import Y_TOL, host, mode_of, oracle_inputs, record, rel_l2, route_parity, widen_gpu
from synthetic import WORKLOADS, Workload, make_ffn_biases, make_inputs

pytestmark = pytest.mark.gpu

KIND = {"geglu": oracle.GEGLU, "gelu_mlp": oracle.GELU_MLP}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # fails loudly when libmoe.so is missing
    return torch.device("cuda:0")


CASES = {
    "tiled_fp32": Workload("tiled_fp32", 200, 128, 16, 3, 128, 64, "sigmoid", 4, 2, 2.5, "f32", "uniform"),
    "tiled_bf16": Workload("tiled_bf16", 300, 192, 16, 4, 192, 128, "softmax", 1, 1, 1.0, "bf16", "uniform"),
    "stream_bf16": Workload("stream_bf16", 1200, 512, 16, 4, 512, 256, "sigmoid", 4, 2, 2.5, "bf16",
                            "uniform"),
    "stream_f384": Workload("stream_f384", 1100, 256, 8, 2, 384, 128, "softmax", 1, 1, 1.0, "bf16", "zero"),
    "decode_bf16": Workload("decode_bf16", 40, 256, 16, 4, 256, 256, "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
}

# gemm path each (case, kind) takes; the GELU MLP needs whole 256-row slabs
PATH = {
    ("tiled_fp32", "geglu"): "tiled", ("tiled_fp32", "gelu_mlp"): "tiled",
    ("tiled_bf16", "geglu"): "tiled", ("tiled_bf16", "gelu_mlp"): "tiled",
    ("stream_bf16", "geglu"): "stream", ("stream_bf16", "gelu_mlp"): "stream",
    ("stream_f384", "geglu"): "stream", ("stream_f384", "gelu_mlp"): "tiled",
    ("decode_bf16", "geglu"): "stream_decode", ("decode_bf16", "gelu_mlp"): "stream_decode",
}


def to_dev(d, dev):
    return {k: (None if v is None else tuple(t.to(dev) for t in v) if isinstance(v, tuple) else v.to(dev))
            for k, v in d.items()}


def run_ex(w, inp, kind, fb):
    cfg = moe.MoeConfig.from_workload(w)
    gated = kind != "gelu_mlp"
    W3 = inp["W3"] if gated else None
    shared = None
    if inp["shared"] is not None:
        W1s, W3s, W2s = inp["shared"]
        shared = (W1s, W3s if gated else None, W2s, fb["b1s"], fb["b2s"])
    y, idx, g = moe.moe_layer_forward_ex(inp["u"], inp["W_router"], inp["bias"], kind, inp["W1"], W3, inp["W2"],
                                         fb["b1"], fb["b2"], shared, cfg=cfg)
    torch.cuda.synchronize()
    return y, idx, g


def oracle_ex(w, inp, kind, fb, forced, tokens=None):
    u, Wr, bias = oracle_inputs(inp)
    gated = kind != "gelu_mlp"
    shared = None
    if inp["shared"] is not None:
        W1s, W3s, W2s = (host(t) for t in inp["shared"])
        shared = (W1s, W3s if gated else None, W2s,
                  None if fb["b1s"] is None else host(fb["b1s"]), None if fb["b2s"] is None else host(fb["b2s"]))
    b1 = None if fb["b1"] is None else host(fb["b1"])
    b2 = None if fb["b2"] is None else host(fb["b2"])
    return oracle.forward(u, Wr, host(inp["W1"]), host(inp["W3"]) if gated else None, host(inp["W2"]), w.k,
                          bias=bias, shared=shared, score_fn=mode_of(w), n_groups=w.n_groups,
                          topk_groups=w.topk_groups, route_scale=w.route_scale, forced_idx=forced, tokens=tokens,
                          kind=KIND[kind], b1=b1, b2=b2)


def no_biases(fb):
    return {k: None for k in fb}


@pytest.mark.parametrize("kind", ["geglu", "gelu_mlp"])
@pytest.mark.parametrize("name", list(CASES))
def test_expert_body_every_token(dev, name, kind):
    w = CASES[name]
    cfg = moe.MoeConfig.from_workload(w)
    path = moe.moe_plan_describe_ex(cfg, kind)[0]
    log(f"[experts] {name} {kind} path={path}")
    assert path == PATH[(name, kind)]
    inp = to_dev(make_inputs(w, seed=11, device="cpu"), dev)
    fb = make_ffn_biases(w, seed=11, device="cpu")
    fb = to_dev(fb, dev) if kind == "gelu_mlp" else no_biases(fb)
    y, idx, g = run_ex(w, inp, kind, fb)
    # routing is the SwiGLU entry point's, bit for bit
    _, idx0, g0 = moe.moe_layer_forward(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                        inp["shared"], cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0) and torch.equal(g, g0)
    gi = idx.cpu().numpy()
    # the oracle routes on its own: same expert sets except counted near-ties
    yr, ir, gr, ge, gg = oracle_ex(w, inp, kind, fb, None)
    u, Wr, bias = oracle_inputs(inp)
    st = route_parity(w, gi, g.cpu().numpy(), ir, gr, ge, gg, oracle.router_logits(u, Wr), bias)
    diff = np.nonzero(~(np.sort(gi, 1) == np.sort(ir, 1)).all(1))[0]
    if diff.size:  # near-ties broken the other way: the oracle on the GPU's choice
        yr[diff] = oracle_ex(w, inp, kind, fb, gi[diff], tokens=diff)[0]
    err = rel_l2(widen_gpu(y), yr)
    log(f"[experts] {name} {kind} rel_l2_max={err.max():.3e} {st}")
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e} at token {err.argmax()}"
    st.update(rel_l2_max=float(err.max()), outputs_checked=int(w.T), gemm_path=path)
    record(f"{name}_{kind}", st)


@pytest.mark.parametrize("name", ["tiled_bf16", "stream_bf16", "decode_bf16"])
def test_gelu_mlp_without_biases(dev, name):
    """NULL b1, b2, b1s, b2s mean zero biases."""
    w = CASES[name]
    log(f"[experts] {name} gelu_mlp no biases")
    inp = to_dev(make_inputs(w, seed=12, device="cpu"), dev)
    fb = no_biases(make_ffn_biases(w, seed=12, device="cpu"))
    y, idx, _ = run_ex(w, inp, "gelu_mlp", fb)
    yr = oracle_ex(w, inp, "gelu_mlp", fb, idx.cpu().numpy())[0]
    err = rel_l2(widen_gpu(y), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e}"


@pytest.mark.parametrize("name", ["tiled_fp32", "stream_bf16", "decode_bf16"])
def test_swiglu_through_ex_is_the_plain_entry_point(dev, name):
    w = CASES[name]
    inp = to_dev(make_inputs(w, seed=13, device="cpu"), dev)
    cfg = moe.MoeConfig.from_workload(w)
    y0, i0, g0 = moe.moe_layer_forward(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                       inp["shared"], cfg=cfg)
    y1, i1, g1 = moe.moe_layer_forward_ex(inp["u"], inp["W_router"], inp["bias"], "swiglu", inp["W1"], inp["W3"],
                                          inp["W2"], None, None, inp["shared"], cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(i0, i1) and torch.equal(g0, g1)


def test_gelu_mlp_output_bias_alone_is_gate_weighted(dev):
    """Zero W2 and W2s: each token's output is sum_j g_j b2[e_j] + b2s, computed
    here from the GPU's own selection and gates (a property at any size)."""
    w = CASES["stream_bf16"]
    inp = to_dev(make_inputs(w, seed=14, device="cpu"), dev)
    fb = to_dev(make_ffn_biases(w, seed=14, device="cpu"), dev)
    inp["W2"] = torch.zeros_like(inp["W2"])
    W1s, W3s, W2s = inp["shared"]
    inp["shared"] = (W1s, W3s, torch.zeros_like(W2s))
    y, idx, g = run_ex(w, inp, "gelu_mlp", fb)
    b2 = fb["b2"].double()
    ref = (g.double().unsqueeze(-1) * b2[idx.long()]).sum(1) + fb["b2s"].double()
    err = rel_l2(widen_gpu(y), ref.cpu().numpy())
    assert err.max() <= 1e-2, f"max rel-L2 {err.max():.3e}"


def test_gelu_mlp_dsv3_decode_shape_sampled(dev):
    """The DeepSeek-V3 decode shape (T = 64, d = 7168, 256 experts of 2048,
    top-8, one shared expert) with GELU-MLP experts, on the decode streaming
    kernels; outputs of 16 sampled tokens against the oracle, which fetches
    only the experts they use."""
    w = WORKLOADS["dsv3_decode"]
    cfg = moe.MoeConfig.from_workload(w)
    assert moe.moe_plan_describe_ex(cfg, "gelu_mlp")[0] == "stream_decode"
    log("[experts] dsv3_decode gelu_mlp: generating weights")
    inp = make_inputs(w, seed=15, device=dev)
    inp["W3"] = None
    inp["shared"] = (inp["shared"][0], None, inp["shared"][2])
    fb = make_ffn_biases(w, seed=15, device=dev)
    y, idx, g = moe.moe_layer_forward_ex(inp["u"], inp["W_router"], inp["bias"], "gelu_mlp", inp["W1"], None,
                                         inp["W2"], fb["b1"], fb["b2"], inp["shared"] + (fb["b1s"], fb["b2s"]),
                                         cfg=cfg)
    torch.cuda.synchronize()
    tokens = np.random.default_rng(15).choice(w.T, 16, replace=False)
    sel = idx.cpu().numpy()[tokens].astype(np.int64)
    used = np.unique(sel)
    remap = np.full(w.E, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    ui = torch.from_numpy(used).to(dev)
    ti = torch.from_numpy(tokens).to(dev)
    W1s, _, W2s = inp["shared"]
    yr, _, gr, _, _ = oracle.forward(
        host(inp["u"].index_select(0, ti)), host(inp["W_router"].index_select(0, ui)),
        host(inp["W1"].index_select(0, ui)), None, host(inp["W2"].index_select(0, ui)), w.k,
        shared=(host(W1s), None, host(W2s), host(fb["b1s"]), host(fb["b2s"])), score_fn=mode_of(w),
        route_scale=w.route_scale, forced_idx=remap[sel], kind=oracle.GELU_MLP,
        b1=host(fb["b1"].index_select(0, ui)), b2=host(fb["b2"].index_select(0, ui)))
    np.testing.assert_allclose(g.cpu().numpy()[tokens], gr, rtol=1e-5, atol=1e-5)
    err = rel_l2(widen_gpu(y)[tokens], yr)
    log(f"[experts] dsv3_decode gelu_mlp sampled rel_l2_max={err.max():.3e}")
    assert err.max() <= Y_TOL["bf16"], f"max rel-L2 {err.max():.3e}"


@pytest.mark.parametrize("kind", ["geglu", "gelu_mlp"])
@pytest.mark.parametrize("name", ["stream_bf16", "decode_bf16"])
def test_packed_expert_bodies_are_bitwise_the_plain_layout(dev, name, kind):
    """moe_pack_weights_ex + moe_layer_forward_packed_ex give exactly the
    plain-layout result (the plain one is checked against the oracle above)."""
    w = CASES[name]
    cfg = moe.MoeConfig.from_workload(w)
    inp = to_dev(make_inputs(w, seed=16, device="cpu"), dev)
    fb = make_ffn_biases(w, seed=16, device="cpu")
    fb = to_dev(fb, dev) if kind == "gelu_mlp" else no_biases(fb)
    ref = run_ex(w, inp, kind, fb)
    gated = kind != "gelu_mlp"
    W1s, W3s, W2s = inp["shared"]
    packed = moe.moe_pack_weights_ex(kind, inp["W1"], inp["W3"] if gated else None, inp["W2"],
                                     (W1s, W3s if gated else None, W2s), cfg=cfg)
    assert packed.numel() == moe.moe_packed_weights_bytes_ex(cfg, kind)
    got = moe.moe_layer_forward_packed_ex(inp["u"], inp["W_router"], inp["bias"], kind, packed, fb["b1"], fb["b2"],
                                          fb["b1s"], fb["b2s"], cfg=cfg)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b), (name, kind)
    log(f"[experts] packed {name} {kind} bitwise equal")
