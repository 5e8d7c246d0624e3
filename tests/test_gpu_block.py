"""GPU parity of the pre-norm residual block, y = h + MoE(RMSNorm(h))
("Lesson 2 -- From the Dense FFN to a Layer of Experts", section 2; "Sparse
MoE FFN" (DeepSeek-V3), eq. 12), against the oracle.

Unfused form: the GPU stores the normalised rows in the layer dtype before
routing on them.  moe_rmsnorm (the block's own kernel) is checked against
the oracle's fp64 RMSNorm to within one rounding of that dtype; the block is
then checked against the oracle evaluated on those same rows, so both sides
take the routing decisions on the same values.

Fused form (moe_block_forward_fused): the norm weight is folded into the
packed weights and each token's 1/rms is applied to its router logits and
gate/up accumulators.  The oracle routes on rs * (h . bf16(W_router * g)),
the precision the kernel decides in, and computes the outputs from the exact
fp64 RMSNorm."""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
import oracle
from oracle import block
from parity import (Y_TOL, host, mode_of, record, rel_l2, route_parity, sampled_outputs, tile_edge_tokens,
                    widen_gpu)
from synthetic import WORKLOADS, Workload, make_inputs, make_norm_weight

pytestmark = pytest.mark.gpu
EPS = 1e-6

SMALL = {
    "sigmoid_groups_shared_bf16": Workload("sigmoid_groups_shared_bf16", 333, 256, 16, 4, 192, 128,
                                           "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    # fp32 beyond the one-kernel small layer (1332 slots): the tiled kernels
    "sigmoid_groups_shared_fp32": Workload("sigmoid_groups_shared_fp32", 333, 256, 16, 4, 192, 128,
                                           "sigmoid", 4, 2, 2.5, "f32", "uniform"),
    "stream_sigmoid_groups_shared": Workload("stream_sigmoid_groups_shared", 1200, 512, 16, 4, 384, 256,
                                             "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
    "decode_sigmoid_groups_shared": Workload("decode_sigmoid_groups_shared", 40, 256, 16, 4, 256, 256,
                                             "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()
    return torch.device("cuda:0")


@pytest.mark.parametrize("dtype,d,T", [("bf16", 7168, 257), ("bf16", 64, 5), ("f32", 512, 130), ("f32", 8192, 3)])
def test_rmsnorm_matches_oracle(dev, dtype, d, T):
    gen = torch.Generator(device="cpu").manual_seed(d + T)
    scale = torch.exp(4 * torch.randn(T, 1, generator=gen))  # row scales over many decades
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    h = (torch.randn(T, d, generator=gen) * scale).to(tdt).to(dev)
    g = (1 + 0.1 * torch.randn(d, generator=gen)).to(tdt).to(dev)
    out = moe.moe_rmsnorm(h, g, EPS)
    again = moe.moe_rmsnorm(h.clone(), g, EPS, out=None)
    inplace = h.clone()
    moe.moe_rmsnorm(inplace, g, EPS, out=inplace)
    torch.cuda.synchronize()
    assert torch.equal(out, again) and torch.equal(out, inplace)
    ref = block.rmsnorm(host(h), host(g), EPS)
    got = widen_gpu(out)
    tol = 2.0 ** -8 if dtype == "bf16" else 4e-6  # one bf16 rounding / fp32 arithmetic
    err = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30)
    assert err.max() <= tol, f"max relative error {err.max():.3e}"


def block_both(w, inp, g, packed=None):
    cfg = moe.MoeConfig.from_workload(w)
    h = inp["u"]
    if packed is None:
        out = moe.moe_block_forward(h, g, EPS, inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                    inp["shared"], cfg=cfg)
    else:
        out = moe.moe_block_forward_packed(h, g, EPS, inp["W_router"], inp["bias"], packed, cfg=cfg)
    un = moe.moe_rmsnorm(h, g, EPS)
    torch.cuda.synchronize()
    return out, un


@pytest.mark.parametrize("name", list(SMALL))
def test_block_every_token(dev, name):
    w = SMALL[name]
    inp = make_inputs(w, seed=11, device=dev)
    g = make_norm_weight(w, seed=11, device=dev)
    (y, idx, gates), un = block_both(w, inp, g)
    # the block routes and computes exactly as the layer on its normalised rows
    cfg = moe.MoeConfig.from_workload(w)
    yl, il, gl = moe.moe_layer_forward(un, inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                       inp["shared"], cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(idx, il) and torch.equal(gates, gl)
    # against the oracle on those rows, with the residual
    shared = None if inp["shared"] is None else tuple(host(s) for s in inp["shared"])
    bias = None if inp["bias"] is None else inp["bias"].double().cpu().numpy()
    kw = dict(bias=bias, shared=shared, score_fn=mode_of(w), n_groups=w.n_groups, topk_groups=w.topk_groups,
              route_scale=w.route_scale)
    yr, ir, gr, ge, gg = block.block_forward(host(inp["u"]), host(g), EPS, host(inp["W_router"]), host(inp["W1"]),
                                             host(inp["W3"]), host(inp["W2"]), w.k, un=host(un), **kw)
    lg = oracle.router_logits(host(un), host(inp["W_router"]))
    gi = idx.cpu().numpy()
    st = route_parity(w, gi, gates.cpu().numpy(), ir, gr, ge, gg, lg, bias)
    diff = ~(np.sort(gi, 1) == np.sort(ir, 1)).all(1)
    if diff.any():
        t = np.nonzero(diff)[0]
        sub = oracle.forward(oracle.widen(host(un))[t], host(inp["W_router"]), host(inp["W1"]), host(inp["W3"]),
                             host(inp["W2"]), w.k, forced_idx=gi[t], **kw)
        yr[t] = sub[0] + oracle.widen(host(inp["u"]))[t]
    err = rel_l2(widen_gpu(y), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e}"
    st["rel_l2_max"] = float(err.max())
    log(f"[block] {name} {st}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_with_zero_down_projections_returns_its_input(dev, dtype):
    w = SMALL["sigmoid_groups_shared_bf16"].with_(dtype=dtype)
    inp = make_inputs(w, seed=3, device=dev)
    inp["W2"].zero_()
    inp["shared"][2].zero_()
    g = make_norm_weight(w, seed=3, device=dev)
    (y, _, _), _ = block_both(w, inp, g)
    assert torch.equal(y, inp["u"])


def test_block_packed_is_bitwise_the_plain_block(dev):
    w = Workload("prefill_sigmoid_groups_shared", 900, 512, 16, 4, 256, 512, "sigmoid", 4, 2, 2.5, "bf16",
                 "uniform")
    inp = make_inputs(w, seed=5, device=dev)
    g = make_norm_weight(w, seed=5, device=dev)
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    a, _ = block_both(w, inp, g)
    b, _ = block_both(w, inp, g, packed=packed)
    for x, z in zip(a, b):
        assert torch.equal(x, z)


def test_block_full_size_dsv3_prefill_packed(dev):
    """The DeepSeek-V3-shaped prefill block (T = 8192) with packed weights, as
    the benchmark runs it: routing of every token, outputs of sampled tokens."""
    w = WORKLOADS["dsv3_prefill"]
    inp = make_inputs(w, seed=0, device=dev)
    g = make_norm_weight(w, seed=0, device=dev)
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    (y, idx, gates), un = block_both(w, inp, g, packed=packed)
    del packed
    bias = inp["bias"].double().cpu().numpy()
    ir, gr, ge, gg, lg = oracle.route(host(un), host(inp["W_router"]), w.k, mode_of(w), w.n_groups,
                                      w.topk_groups, w.route_scale, bias=bias)
    gi = idx.cpu().numpy()
    st = route_parity(w, gi, gates.cpu().numpy(), ir, gr, ge, gg, lg, bias)
    tok = np.random.default_rng(0).choice(w.T, size=12, replace=False)
    near = (ge < 1e-5) | (gg < 1e-5)
    sel = np.where(near[tok, None], gi[tok], ir[tok])
    yr, _, _ = sampled_outputs(w, dict(inp, u=un), tok, sel)
    yr = yr + oracle.widen(host(inp["u"]))[tok]
    err = rel_l2(widen_gpu(y[torch.from_numpy(tok).to(dev)]), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e}"
    st["rel_l2_max"] = float(err.max())
    log(f"[block] dsv3_prefill {st}")


FUSED = {
    "stream_sigmoid_groups_shared": SMALL["stream_sigmoid_groups_shared"].with_(F=512),
    "decode_sigmoid_groups_shared": SMALL["decode_sigmoid_groups_shared"],
    "stream_softmax_no_shared": Workload("stream_softmax_no_shared", 700, 256, 8, 2, 256, 0, "softmax", 1, 1, 1.0,
                                         "bf16", "zero"),
    "decode_one_token": Workload("decode_one_token", 1, 512, 16, 4, 256, 256, "sigmoid", 4, 2, 2.5, "bf16",
                                 "uniform"),
}


def fused_run(w, inp, g):
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_block_weights(g, inp["W_router"], inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    assert packed.numel() == moe.moe_block_packed_bytes(cfg)
    out = moe.moe_block_forward_fused(inp["u"], EPS, inp["bias"], packed, cfg=cfg)
    torch.cuda.synchronize()
    return out, packed


def fused_check(w, inp, g, y, idx, gates, tokens=None):
    """Routing of every token and outputs of `tokens` (None: all) of the fused
    block against the oracle's fused block."""
    shared = None if inp["shared"] is None else tuple(host(s) for s in inp["shared"])
    bias = inp["bias"].double().cpu().numpy()
    h, gw, Wr = host(inp["u"]), host(g), host(inp["W_router"])
    rk = dict(bias=bias, score_fn=mode_of(w), n_groups=w.n_groups, topk_groups=w.topk_groups,
              route_scale=w.route_scale)
    ir, gr, ge, gg, lg = block.fused_route(h, gw, EPS, Wr, w.k, **rk)
    gi = idx.cpu().numpy()
    st = route_parity(w, gi, gates.cpu().numpy(), ir, gr, ge, gg, lg, bias)
    tok = np.arange(w.T) if tokens is None else np.asarray(tokens)
    near = (ge < 1e-5) | (gg < 1e-5)
    sel = np.where(near[tok, None], gi[tok], ir[tok]).astype(np.int32)
    gsel = block.gates_of(lg[tok], sel, mode_of(w), w.route_scale)
    un = block.rmsnorm(h[tok], gw, EPS)
    yr = oracle.widen(h[tok]) + block.expert_sum(un, host(inp["W1"]), host(inp["W3"]), host(inp["W2"]), sel, gsel,
                                                 shared)
    err = rel_l2(widen_gpu(y[torch.from_numpy(tok).to(y.device)]), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e} at token {tok[err.argmax()]}"
    st["rel_l2_max"] = float(err.max())
    st["outputs_checked"] = int(tok.size)
    return st


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_block_every_token(dev, name):
    w = FUSED[name]
    cfg = moe.MoeConfig.from_workload(w)
    log(f"[fused] {name} path={moe.moe_plan_describe(cfg)[0]}")
    inp = make_inputs(w, seed=21, device=dev)
    g = make_norm_weight(w, seed=21, device=dev)
    (y, idx, gates), _ = fused_run(w, inp, g)
    st = fused_check(w, inp, g, y, idx, gates)
    log(f"[fused] {name} {st}")
    record(f"fused_block_{name}", st)
    # deterministic: a second call gives the same bits
    (y2, idx2, g2), _ = fused_run(w, inp, g)
    assert torch.equal(y, y2) and torch.equal(idx, idx2) and torch.equal(gates, g2)


def test_fused_block_with_zero_down_projections_returns_its_input(dev):
    w = FUSED["stream_sigmoid_groups_shared"]
    inp = make_inputs(w, seed=22, device=dev)
    inp["W2"].zero_()
    inp["shared"][2].zero_()
    g = make_norm_weight(w, seed=22, device=dev)
    (y, _, _), _ = fused_run(w, inp, g)
    assert torch.equal(y, inp["u"])


def test_fused_block_argument_errors(dev):
    w = FUSED["stream_softmax_no_shared"]
    inp = make_inputs(w, seed=23, device=dev)
    g = make_norm_weight(w, seed=23, device=dev)
    _, packed = fused_run(w, inp, g)
    cfg = moe.MoeConfig.from_workload(w)
    with pytest.raises(moe.MoeError):
        moe.moe_block_forward_fused(inp["u"], -1.0, inp["bias"], packed, cfg=cfg)
    tiled = moe.MoeConfig.from_workload(w.with_(d=192))
    assert moe.moe_block_packed_bytes(tiled) == 0


def test_fused_block_full_size_dsv3_prefill_and_decode(dev):
    """The DeepSeek-V3-shaped block, prefill (T = 8192) and decode (T = 64)
    on the same weights: routing of every token against the oracle's fused
    block; outputs of 256 random tokens plus the first and last row of every
    routed and shared GEMM tile (prefill) and of all 64 tokens (decode)."""
    w = WORKLOADS["dsv3_prefill"]
    inp = make_inputs(w, seed=0, device=dev)
    g = make_norm_weight(w, seed=0, device=dev)
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_block_weights(g, inp["W_router"], inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    y, idx, gates = moe.moe_block_forward_fused(inp["u"], EPS, inp["bias"], packed, cfg=cfg)
    torch.cuda.synchronize()
    path, tile_m = moe.moe_plan_describe(cfg)
    # the tiles follow the fused router's own selection (its stable expert order is unique)
    c_f, _, p_f, _ = oracle.permutation(idx.cpu().numpy(), w.E)
    edge, ntiles = tile_edge_tokens(w, path, tile_m, c_f, p_f, w.T)
    tok = np.unique(np.concatenate([np.random.default_rng(0).choice(w.T, 256, replace=False), edge]))
    log(f"[fused] dsv3_prefill: oracle on {tok.size} tokens ({ntiles} tiles)")
    st = fused_check(w, inp, g, y, idx, gates, tokens=tok)
    st.update(tiles=int(ntiles), tile_edge_tokens=int(edge.size))
    log(f"[fused] dsv3_prefill {st}")
    record("fused_block_dsv3_prefill", st)
    wd = WORKLOADS["dsv3_decode"]
    from synthetic import make_u
    ind = dict(inp, u=make_u(wd, seed=0, device=dev))
    cfgd = moe.MoeConfig.from_workload(wd)
    y, idx, gates = moe.moe_block_forward_fused(ind["u"], EPS, ind["bias"], packed, cfg=cfgd)
    torch.cuda.synchronize()
    st = fused_check(wd, ind, g, y, idx, gates)
    log(f"[fused] dsv3_decode {st}")
    record("fused_block_dsv3_decode", st)
    del packed, inp, ind
