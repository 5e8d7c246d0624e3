"""GPU parity of the HIP layer against the CPU oracle (through the C ABI).

Small layers are checked on every token; the full-size workloads are checked
on every token's routing and on a sample of tokens' outputs, in the same
launch configuration the benchmark times.
"""
import math
import os
import sys

import numpy as np
import pytest
import torch

import mixture_experts_ffn_biased_amd as moe
import oracle
from oracle import balance, skew
from parity import (Y_TOL, host, mode_of, oracle_inputs, record, rel_l2, route_parity, sampled_outputs,
                    tile_edge_tokens, widen_gpu)
from synthetic import WORKLOADS, Workload, make_inputs, make_u

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.lib()  # fails loudly when libmoe.so is missing
    return torch.device("cuda:0")


def run(w, inp, bias="given", **kw):
    cfg = moe.MoeConfig.from_workload(w)
    b = inp["bias"] if bias == "given" else bias
    y, idx, g = moe.moe_layer_forward(inp["u"], inp["W_router"], b, inp["W1"], inp["W3"],
                                      inp["W2"], inp["shared"], cfg=cfg, **kw)
    torch.cuda.synchronize()
    return y, idx, g


def to_dev(inp, dev):
    out = {}
    for k_, v in inp.items():
        if v is None:
            out[k_] = None
        elif isinstance(v, tuple):
            out[k_] = tuple(t.to(dev) for t in v)
        else:
            out[k_] = v.to(dev)
    return out


def full_oracle(w, inp, forced=None):
    u, Wr, bias = oracle_inputs(inp)
    shared = None if inp["shared"] is None else tuple(host(t) for t in inp["shared"])
    return oracle.forward(u, Wr, host(inp["W1"]), host(inp["W3"]), host(inp["W2"]), w.k,
                          bias=bias, shared=shared, score_fn=mode_of(w), n_groups=w.n_groups,
                          topk_groups=w.topk_groups, route_scale=w.route_scale,
                          forced_idx=forced)


def check_full(w, inp, y, idx, g):
    """Every token: routing and output against the oracle."""
    yr, ir, gr, ge, gg = full_oracle(w, inp)
    u, Wr, bias = oracle_inputs(inp)
    lg = oracle.router_logits(u, Wr)
    gi = idx.cpu().numpy()
    st = route_parity(w, gi, g.cpu().numpy(), ir, gr, ge, gg, lg, bias)
    diff = ~(np.sort(gi, 1) == np.sort(ir, 1)).all(1)
    if diff.any():  # near-ties the GPU broke the other way: oracle with its choice
        t = np.nonzero(diff)[0]
        shared = None if inp["shared"] is None else tuple(host(s) for s in inp["shared"])
        sub = oracle.forward(u[t], Wr, host(inp["W1"]), host(inp["W3"]), host(inp["W2"]), w.k,
                             shared=shared, score_fn=mode_of(w), route_scale=w.route_scale,
                             n_groups=w.n_groups, topk_groups=w.topk_groups, forced_idx=gi[t])
        yr[t] = sub[0]
    err = rel_l2(widen_gpu(y), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e} at token {err.argmax()}"
    st["rel_l2_max"] = float(err.max())
    st["outputs_checked"] = int(w.T)
    record(w.name, st)
    return st


SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "sigmoid_groups_shared_bf16": Workload("sigmoid_groups_shared_bf16", 333, 256, 16, 4, 192, 128,
                                           "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
    "softmax_bias_bf16": Workload("softmax_bias_bf16", 517, 192, 32, 6, 320, 0, "softmax", 1, 1,
                                  1.0, "bf16", "uniform"),
    "sigmoid_groups_fp32": Workload("sigmoid_groups_fp32", 200, 128, 16, 3, 128, 64, "sigmoid", 4,
                                    2, 2.5, "f32", "uniform"),
    "k_equals_E_bf16": Workload("k_equals_E_bf16", 70, 128, 8, 8, 128, 64, "softmax", 1, 1, 1.0,
                                "bf16", "zero"),
    "single_token_k1_bf16": Workload("single_token_k1_bf16", 1, 128, 4, 1, 64, 0, "softmax", 1, 1,
                                     1.0, "bf16", "uniform"),
    "e256_groups_bf16": Workload("e256_groups_bf16", 150, 128, 256, 8, 64, 64, "sigmoid", 8, 4, 2.5,
                                 "bf16", "uniform"),
    # the largest top-k the library takes (32)
    "max_k32_bf16": Workload("max_k32_bf16", 90, 128, 64, 32, 64, 0, "softmax", 1, 1, 1.0, "bf16", "uniform"),
    # the largest group count (64 groups of 4, keep 8)
    "groups64_sigmoid_bf16": Workload("groups64_sigmoid_bf16", 120, 128, 256, 16, 64, 64, "sigmoid", 64, 8,
                                      2.5, "bf16", "uniform"),
    # the one-kernel small fp32 layer: groups and a shared expert (510 slots),
    # its size limits (512 slots, d = F = F_shared = 1024), every expert chosen
    "small_fp32_groups_shared": Workload("small_fp32_groups_shared", 170, 256, 16, 3, 192, 128, "sigmoid", 4,
                                         2, 2.5, "f32", "uniform"),
    "small_fp32_limits": Workload("small_fp32_limits", 256, 1024, 8, 2, 1024, 1024, "softmax", 1, 1, 1.0,
                                  "f32", "uniform"),
    "small_fp32_k_equals_E": Workload("small_fp32_k_equals_E", 50, 64, 8, 8, 64, 0, "softmax", 1, 1, 1.0,
                                      "f32", "zero"),
}


STREAM = {
    "stream_softmax": Workload("stream_softmax", 700, 256, 8, 2, 256, 0, "softmax", 1, 1, 1.0,
                               "bf16", "zero"),
    "stream_sigmoid_groups_shared": Workload("stream_sigmoid_groups_shared", 1200, 512, 16, 4, 384,
                                             256, "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
    "stream_many_tiles": Workload("stream_many_tiles", 2100, 256, 8, 3, 128, 128, "softmax", 1, 1,
                                  1.0, "bf16", "uniform"),
    # d = 768: the first product's K loop is two whole 12-stage turns with no
    # partial turn (d = 256 and 512 above end inside a turn).
    "stream_d768_shared": Workload("stream_d768_shared", 900, 768, 8, 2, 256, 256, "sigmoid", 2, 1,
                                   2.5, "bf16", "uniform"),
}


DECODE = {
    "decode_sigmoid_groups_shared": Workload("decode_sigmoid_groups_shared", 40, 256, 16, 4, 256, 256,
                                             "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
    "decode_softmax_e64": Workload("decode_softmax_e64", 37, 512, 64, 6, 512, 0, "softmax", 1, 1,
                                   1.0, "bf16", "uniform"),
    # one token: every tile (four routed, the shared expert's) holds a single row
    "decode_one_token": Workload("decode_one_token", 1, 256, 16, 4, 256, 256, "sigmoid", 4, 2, 2.5,
                                 "bf16", "uniform"),
    "decode_two_tokens_k8": Workload("decode_two_tokens_k8", 2, 512, 64, 8, 256, 256, "softmax", 1, 1,
                                     1.0, "bf16", "uniform"),
}


# The prefill streaming kernels across K: the first product's K loop (turns
# of 12 stages) with no whole turn, a partial turn of 4 or 8 stages, or whole
# turns only (d = 256 .. 2048), and the second product's stage ring with K
# from 4 to 20 stages (F, F_shared from 128 to 640), with and without a
# shared expert, softmax and grouped sigmoid routing.
SWEEP = {
    "sweep_d256_f640": Workload("sweep_d256_f640", 500, 256, 8, 2, 640, 0, "softmax", 1, 1, 1.0,
                                "bf16", "uniform"),
    "sweep_d512_f384_shared": Workload("sweep_d512_f384_shared", 700, 512, 16, 2, 384, 128, "sigmoid",
                                       4, 2, 2.5, "bf16", "uniform"),
    "sweep_d768_k1_shared": Workload("sweep_d768_k1_shared", 800, 768, 8, 1, 256, 256, "softmax", 1, 1,
                                     1.0, "bf16", "uniform"),
    "sweep_d1024_f128": Workload("sweep_d1024_f128", 600, 1024, 8, 2, 128, 0, "softmax", 1, 1, 1.0,
                                 "bf16", "uniform"),
    "sweep_d1536_e64_k6": Workload("sweep_d1536_e64_k6", 800, 1536, 64, 6, 256, 0, "sigmoid", 8, 4, 2.5,
                                   "bf16", "uniform"),
    "sweep_d2048_f512_shared": Workload("sweep_d2048_f512_shared", 520, 2048, 8, 2, 512, 384, "sigmoid",
                                        2, 1, 2.5, "bf16", "uniform"),
}


@pytest.mark.parametrize("name", list(SWEEP))
def test_stream_shapes_across_k_every_token(dev, name):
    w = SWEEP[name]
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == "stream"
    log(f"[sweep] {name}")
    inp = to_dev(make_inputs(w, seed=11, device="cpu"), dev)
    y, idx, g = run(w, inp)
    st = check_full(w, inp, y, idx, g)
    log(f"[sweep] {name} {st}")


@pytest.mark.parametrize("name", list(STREAM) + list(DECODE))
def test_stream_path_every_token(dev, name):
    w = STREAM.get(name) or DECODE[name]
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == (
        "stream" if name in STREAM else "stream_decode")
    log(f"[stream] {name}")
    inp = to_dev(make_inputs(w, seed=7, device="cpu"), dev)
    y, idx, g = run(w, inp)
    st = check_full(w, inp, y, idx, g)
    log(f"[stream] {name} {st}")


def test_stream_path_one_expert_takes_every_token(dev):
    """Expert 0 in every token's set: 2100 rows = 9 tiles of 256 (ragged)
    spread over several chunks and XCD lists."""
    w = STREAM["stream_many_tiles"]
    b = torch.zeros(w.E)
    b[0] = 100.0
    inp = to_dev(make_inputs(w, seed=8, device="cpu", bias=b), dev)
    y, idx, g = run(w, inp)
    assert (idx[:, 0] == 0).all()
    check_full(w, inp, y, idx, g)


def test_decode_path_one_expert_takes_every_token(dev):
    """Decode kernels (32-row tiles) with expert 0 in every token's set: its
    100 rows are 4 tiles (32, 32, 32, 4) in two chunks, each tile streaming
    the expert's weight slabs again; the shared expert has 4 tiles too."""
    w = Workload("decode_one_expert", 100, 256, 16, 2, 256, 256, "softmax", 1, 1, 1.0, "bf16", "uniform")
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == "stream_decode"
    b = torch.zeros(w.E)
    b[0] = 100.0
    inp = to_dev(make_inputs(w, seed=12, device="cpu", bias=b), dev)
    y, idx, g = run(w, inp)
    assert (idx[:, 0] == 0).all()
    check_full(w, inp, y, idx, g)


PACKABLE = {
    "stream_softmax": STREAM["stream_softmax"],
    "decode_sigmoid_groups_shared": DECODE["decode_sigmoid_groups_shared"],
    "prefill_sigmoid_groups_shared": Workload("prefill_sigmoid_groups_shared", 900, 512, 16, 4, 256, 512,
                                              "sigmoid", 4, 2, 2.5, "bf16", "uniform"),
}


def run_packed(w, inp, packed):
    cfg = moe.MoeConfig.from_workload(w)
    out = moe.moe_layer_forward_packed(inp["u"], inp["W_router"], inp["bias"], packed, cfg=cfg)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(PACKABLE))
def test_packed_weights_give_bitwise_identical_layer(dev, name):
    """The packed layout changes where weights live, not the arithmetic."""
    w = PACKABLE[name]
    inp = to_dev(make_inputs(w, seed=9, device="cpu"), dev)
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    ref = run(w, inp)
    got = run_packed(w, inp, packed)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    check_full(w, inp, *got)


SMALL_PATH = {"tiny_fp32", "small_fp32_groups_shared", "small_fp32_limits", "small_fp32_k_equals_E"}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_every_token(dev, name):
    w = SMALL[name]
    assert (moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == "small") == (name in SMALL_PATH)
    log(f"[small] {name}")
    inp = to_dev(make_inputs(w, seed=1, device="cpu"), dev)
    y, idx, g = run(w, inp)
    st = check_full(w, inp, y, idx, g)
    log(f"[small] {name} {st}")


def test_one_expert_takes_every_token(dev):
    """A large bias on expert 3 puts it in every token's set: one expert with
    all T rows over several tiles, while the gate still uses the raw score."""
    w = Workload("forced_e3", 300, 128, 8, 2, 128, 64, "softmax", 1, 1, 1.0, "bf16", "zero")
    b = torch.zeros(8)
    b[3] = 100.0
    inp = to_dev(make_inputs(w, seed=2, device="cpu", bias=b), dev)
    y, idx, g = run(w, inp)
    assert (idx[:, 0] == 3).all()
    check_full(w, inp, y, idx, g)


def test_null_bias_is_bitwise_zero_bias_and_runs_are_deterministic(dev):
    w = SMALL["sigmoid_groups_shared_bf16"].with_(bias="zero")
    inp = to_dev(make_inputs(w, seed=3, device="cpu"), dev)
    ref = run(w, inp)
    none = run(w, inp, bias=None)
    for a, b in zip(ref, none):
        assert torch.equal(a, b)
    for _ in range(3):
        again = run(w, inp)
        for a, b in zip(ref, again):
            assert torch.equal(a, b)


def test_nan_row_gives_valid_distinct_indices(dev):
    w = SMALL["sigmoid_groups_shared_bf16"]
    inp = make_inputs(w, seed=4, device="cpu")
    inp["u"][7] = float("nan")
    inp = to_dev(inp, dev)
    y, idx, g = run(w, inp)
    u, Wr, bias = oracle_inputs(inp)
    ir, _, _, _, _ = oracle.route(u, Wr, w.k, mode_of(w), w.n_groups, w.topk_groups,
                                  w.route_scale, bias=bias)
    gi = idx.cpu().numpy()
    assert ((gi >= 0) & (gi < w.E)).all()
    assert len(set(gi[7].tolist())) == w.k
    assert gi[7].tolist() == ir[7].tolist()


# Routed row counts at and around the tile edges.  Prefill (256-row tiles,
# rows spread evenly over ceil(c / 256) tiles): 255/256/257 (one tile, one,
# two), 511/512/513 (two, two, three), 767/768/769 (three, three, four), and
# counts of 1-2, 31-33, 128-129.  Decode (32-row tiles, ragged last tile):
# 31/32/33 .. 127/128, counts of 1-3 and 16-17, and 48 experts with no rows.
TILE_EDGES = {
    "prefill": (Workload("tile_edges_prefill", 2482, 256, 16, 2, 256, 256, "softmax", 1, 1, 1.0, "bf16",
                         "zero"),
                [255, 256, 257, 511, 512, 513, 767, 768, 769, 1, 2, 31, 32, 33, 128, 129], "stream"),
    "decode": (Workload("tile_edges_decode", 435, 512, 64, 2, 256, 256, "softmax", 1, 1, 1.0, "bf16", "zero"),
               [31, 32, 33, 63, 64, 65, 95, 96, 97, 1, 2, 3, 16, 17, 127, 128], "stream_decode"),
}


def routed_to_counts(w, counts, seed, dev):
    """Inputs whose routing gives expert e exactly counts[e] rows: the router
    reads u's first E columns (W_router is the identity there), and token t's
    two experts get 8 and 7 in those columns, the others |x| < 0.5, so every
    selection has a gap of more than 6 at the k-th expert.  Experts come from
    the sorted slot list: token t takes its t-th and (T + t)-th entries, which
    differ because no count exceeds T."""
    assert w.k == 2 and sum(counts) == w.T * w.k and max(counts) < w.T
    inp = make_inputs(w, seed=seed, device="cpu")
    slots = np.repeat(np.arange(len(counts)), counts)
    first, second = slots[:w.T], slots[w.T:]
    assert (first != second).all()
    rng = np.random.default_rng(seed)
    u = inp["u"].float().numpy().copy()
    u[:, :w.E] = rng.uniform(-0.5, 0.5, size=(w.T, w.E))
    u[np.arange(w.T), first] = 8.0
    u[np.arange(w.T), second] = 7.0
    inp["u"] = torch.from_numpy(u).to(torch.bfloat16)
    Wr = torch.zeros(w.E, w.d)
    Wr[torch.arange(w.E), torch.arange(w.E)] = 1.0
    inp["W_router"] = Wr.to(torch.bfloat16)
    inp["bias"] = torch.zeros(w.E)
    return to_dev(inp, dev)


@pytest.mark.parametrize("name", list(TILE_EDGES))
def test_tile_edge_row_counts_every_token(dev, name):
    w, counts, path = TILE_EDGES[name]
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == path
    log(f"[tile-edges] {name}")
    inp = routed_to_counts(w, counts, 21, dev)
    y, idx, g = run(w, inp)
    got = np.bincount(idx.cpu().numpy().ravel(), minlength=w.E)
    want = np.zeros(w.E, dtype=np.int64)
    want[:len(counts)] = counts
    assert (got == want).all(), f"rows per expert {got.tolist()}"
    st = check_full(w, inp, y, idx, g)
    log(f"[tile-edges] {name} {st}")


def test_side_stream_call_matches_the_default_stream(dev):
    """stream= runs the layer on another stream: its outputs and workspace
    are allocated on that stream, so default-stream allocations made while
    the kernels run cannot take their memory; results are bitwise those of
    the default-stream call."""
    w = STREAM["stream_sigmoid_groups_shared"]
    inp = to_dev(make_inputs(w, seed=17, device="cpu"), dev)
    ref = run(w, inp)
    cfg = moe.MoeConfig.from_workload(w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(3):
        outs.append(moe.moe_layer_forward(inp["u"], inp["W_router"], inp["bias"], inp["W1"], inp["W3"],
                                          inp["W2"], inp["shared"], cfg=cfg, stream=side))
        junk = torch.full((w.T * w.k, w.d), 7.0, dtype=inp["u"].dtype, device=dev)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for out in outs:
        for a, b in zip(ref, out):
            assert torch.equal(a, b)


def test_zero_tokens_is_a_noop(dev):
    w = SMALL["softmax_bias_bf16"]
    inp = to_dev(make_inputs(w.with_(T=4), seed=5, device="cpu"), dev)
    cfg = moe.MoeConfig.from_workload(w, T=0)
    u0 = inp["u"][:0]
    y, idx, g = moe.moe_layer_forward(u0, inp["W_router"], inp["bias"], inp["W1"], inp["W3"],
                                      inp["W2"], None, cfg=cfg)
    assert y.shape == (0, w.d) and idx.shape == (0, w.k)


@pytest.mark.parametrize("name", ["sigmoid_groups_shared_bf16", "e256_groups_bf16"])
def test_route_debug_permutation_is_exact(dev, name):
    w = SMALL[name].with_(T=3001)
    inp = to_dev(make_inputs(w, seed=6, device="cpu"), dev)
    cfg = moe.MoeConfig.from_workload(w)
    idx, g, counts, offsets, perm, inv = moe.moe_route_debug(inp["u"], inp["W_router"],
                                                             inp["bias"], cfg=cfg)
    torch.cuda.synchronize()
    c, o, p, iv = oracle.permutation(idx.cpu().numpy(), w.E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(perm.cpu().numpy(), p)
    assert np.array_equal(inv.cpu().numpy(), iv)
    # routing of the debug entry point is the forward's routing
    y2, idx2, g2 = run(w, inp)
    assert torch.equal(idx, idx2) and torch.equal(g, g2)


# ------------------------------------------------------------------ full-size workloads

def check_large(w, inp, n_sample, seed=0, must_include=None, tile_edges=True, tag=None):
    """Routing of every token against the oracle, and the outputs of n_sample
    seeded random tokens plus (tile_edges) the tokens in the first and last
    row of every routed and shared tile the GEMMs ran, from the permutation
    the library built on the same inputs."""
    u, Wr, bias = oracle_inputs(inp)
    bias_arg = bias if inp["bias"] is not None else None
    log(f"[{w.name}] gpu forward")
    y, idx, g = run(w, inp)
    log(f"[{w.name}] oracle routing on {w.T} tokens")
    ir, gr, ge, gg, lg = oracle.route(u, Wr, w.k, mode_of(w), w.n_groups, w.topk_groups,
                                      w.route_scale, bias=bias_arg)
    gi = idx.cpu().numpy()
    st = route_parity(w, gi, g.cpu().numpy(), ir, gr, ge, gg, lg, bias)
    rng = np.random.default_rng(seed)
    tok = rng.choice(w.T, size=min(n_sample, w.T), replace=False)
    n_tiles = 0
    if tile_edges:
        cfg = moe.MoeConfig.from_workload(w)
        path, tile_m = moe.moe_plan_describe(cfg)
        idx2, _, counts, _, perm, _ = moe.moe_route_debug(inp["u"], inp["W_router"], inp["bias"], cfg=cfg)
        torch.cuda.synchronize()
        assert torch.equal(idx2, idx), "the debug entry point routes as the forward does"
        edge, n_tiles = tile_edge_tokens(w, path, tile_m, counts.cpu().numpy(), perm.cpu().numpy(), w.T)
        tok = np.concatenate([tok, edge])
        st["gemm_path"] = path
        st["tiles"] = int(n_tiles)
        st["tile_edge_tokens"] = int(edge.size)
    if must_include is not None:
        tok = np.concatenate([tok, must_include])
    tok = np.unique(tok)
    near = (ge < 1e-5) | (gg < 1e-5)
    sel = np.where(near[tok, None], gi[tok], ir[tok])
    log(f"[{w.name}] oracle outputs on {tok.size} tokens ({n_tiles} tiles)")
    yr, _, _ = sampled_outputs(w, inp, tok, sel)
    err = rel_l2(widen_gpu(y[torch.from_numpy(tok).to(y.device)]), yr)
    assert err.max() <= Y_TOL[w.dtype], f"max rel-L2 {err.max():.3e} at token {tok[err.argmax()]}"
    st["rel_l2_max"] = float(err.max())
    st["outputs_checked"] = int(tok.size)
    log(f"[{w.name}] {st}")
    record(tag or w.name, st)
    return y, idx, g, st


@pytest.fixture(autouse=True)
def _release_memory():
    yield
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def test_mixtral_full_size(dev):
    w = WORKLOADS["mixtral_e8_top2"]
    inp = make_inputs(w, seed=0, device=dev)
    check_large(w, inp, n_sample=256)
    del inp


def test_dsv3_prefill_and_decode_full_size_packed(dev):
    """Packed-weight forward at the DSv3 prefill and decode shapes (the
    benchmark's launch configuration) is bitwise the plain forward, which
    the two tests below check against the oracle."""
    w = WORKLOADS["dsv3_prefill"]
    inp = make_inputs(w, seed=0, device=dev)
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    for wl in (w, WORKLOADS["dsv3_decode"]):
        u = inp["u"] if wl.T == w.T else make_u(wl, seed=0, device=dev)
        x = dict(inp, u=u)
        ref = run(wl, x)
        got = run_packed(wl, x, packed)
        for a, b in zip(ref, got):
            assert torch.equal(a, b), wl.name
        log(f"[packed] {wl.name} bitwise equal to the plain-weight forward")
    del inp, packed


def test_dsv3_prefill_full_size(dev):
    """Every token's routing, and the outputs of 256 random tokens plus the
    first and last row of each of the ~420 routed and 32 shared tiles."""
    w = WORKLOADS["dsv3_prefill"]
    inp = make_inputs(w, seed=0, device=dev)
    check_large(w, inp, n_sample=256)
    del inp


def test_dsv3_decode_full_size(dev):
    """All 64 tokens: routing and outputs."""
    w = WORKLOADS["dsv3_decode"]
    inp = make_inputs(w, seed=0, device=dev)
    _, _, _, st = check_large(w, inp, n_sample=w.T)
    assert st["outputs_checked"] == w.T
    del inp


@pytest.mark.parametrize("name,seed", [("dsv3_prefill", 1), ("dsv3_decode", 2)])
def test_dsv3_full_size_other_seed_plain_and_packed(dev, name, seed):
    """Another draw of every input at full size: routing of all tokens and
    sampled outputs against the oracle, and the packed-weight layer bitwise
    equal to the plain one."""
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=seed, device=dev)
    y, idx, g, _ = check_large(w, inp, n_sample=64, seed=seed, tag=f"{name}_seed{seed}")
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    yp, ip, gp = moe.moe_layer_forward_packed(inp["u"], inp["W_router"], inp["bias"], packed, cfg=cfg)
    torch.cuda.synchronize()
    assert torch.equal(ip, idx) and torch.equal(gp, g) and torch.equal(yp, y)
    del inp, packed


def test_streaming_schedule_overflow_falls_back_to_the_tiled_kernels(dev):
    """720,000 tokens: more expert chunks than the streaming schedule holds, so
    the layer runs on the tiled kernels (11,258 tiles); routing of every token
    and sampled outputs against the oracle."""
    w = Workload("huge_t", 720_000, 256, 8, 2, 128, 0, "softmax", 1, 1, 1.0, "bf16", "zero")
    assert moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == "tiled"
    inp = make_inputs(w, seed=4, device=dev)
    check_large(w, inp, n_sample=16, must_include=np.array([0, w.T - 1]), tile_edges=False)
    del inp


def test_skewed_load_bias_off_and_on(dev):
    w = WORKLOADS["skewed_e128_top8"]
    base = make_inputs(w, seed=0, device=dev)
    u = host(base["u"])
    Wr = host(base["W_router"])
    lg = oracle.router_logits(u, Wr)
    a = oracle.widen(u) @ base["skew_dir"].double().cpu().numpy()
    alpha = skew.calibrate_expert0_scale(lg[:, 1:], a, w.k, target=0.90)
    del base
    inp = make_inputs(w, seed=0, device=dev, expert0_scale=alpha)
    u, Wr, _ = oracle_inputs(inp)
    lg = oracle.router_logits(u, Wr)
    idx0, _, _, _ = oracle.select(lg, w.k, oracle.SOFTMAX)
    share = float((idx0 == 0).any(1).mean())
    log(f"[skewed] alpha={alpha:.4f} expert-0 share at zero bias={share:.4f}")
    assert abs(share - 0.90) <= 0.005
    # bias off
    _, idx, _, st0 = check_large(w, inp, n_sample=256, tag="skewed_e128_top8_bias_off",
                                 must_include=np.nonzero((idx0 == 0).any(1))[0][:8])
    cnt0 = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.E)
    # bias on: the aux-loss-free loop's correction vector
    b, hist = balance.balance_bias(lg, w.k)
    inp["bias"] = torch.from_numpy(b.astype(np.float32)).to(dev)
    _, idx, _, st1 = check_large(w, inp, n_sample=256, tag="skewed_e128_top8_bias_on",
                                 must_include=np.nonzero((idx0 == 0).any(1))[0][:8])
    cnt1 = np.bincount(idx.cpu().numpy().reshape(-1), minlength=w.E)
    e0, e1 = balance.entropy(cnt0), balance.entropy(cnt1)
    log(f"[skewed] expert-0 rows {cnt0[0]} -> {cnt1[0]}, entropy {e0:.4f} -> {e1:.4f} "
        f"(ln E = {math.log(w.E):.4f})")
    assert cnt1[0] < cnt0[0] and e1 > e0
    del inp


def _divisors(n):
    return [g for g in range(1, n + 1) if n % g == 0]


def random_shapes(n=25, seed=2024):
    """Seeded random layers over every kernel path (five of each): the
    one-kernel small fp32 layer, the tiled kernels in fp32 and bf16, and the
    prefill and decode streaming kernels, with random E, k, d, F, F_shared,
    score function, groups and bias."""
    rng = np.random.default_rng(seed)
    # kind of shape drawn -> the path name the library reports for it
    kinds = {"small": "small", "tiled_f32": "tiled", "tiled_bf16": "tiled", "stream": "stream",
             "stream_decode": "stream_decode"}
    order = list(kinds)
    out = {}
    i = 0
    while len(out) < n:
        kind = order[len(out) % len(order)]
        i += 1
        assert i <= 20 * n, f"random shapes: no {kind} layer drawn in {i} tries"
        sigmoid = bool(rng.integers(0, 2))
        if kind == "small":
            E = int(rng.choice([4, 8, 16, 32])); dtype = "f32"
            d = 64 * int(rng.integers(1, 9)); F = 64 * int(rng.integers(1, 9)); Fs = 64 * int(rng.integers(0, 4))
        elif kind == "tiled_f32":
            E = int(rng.choice([4, 8, 16])); dtype = "f32"
            d = 64 * int(rng.integers(1, 5)); F = 64 * int(rng.integers(1, 5)); Fs = 64 * int(rng.integers(0, 3))
        elif kind == "tiled_bf16":
            E = int(rng.choice([8, 16, 32])); dtype = "bf16"
            d = 64 * int(rng.choice([1, 3, 5, 7])); F = 64 * int(rng.integers(1, 6)); Fs = 64 * int(rng.integers(0, 3))
        elif kind == "stream":
            E = int(rng.choice([8, 16])); dtype = "bf16"
            d = 256 * int(rng.integers(1, 3)); F = 128 * int(rng.integers(1, 5)); Fs = 128 * int(rng.integers(0, 3))
        else:
            E = int(rng.choice([16, 32, 64])); dtype = "bf16"
            d = 256 * int(rng.integers(1, 3)); F = 256 * int(rng.integers(1, 3)); Fs = 256 * int(rng.integers(0, 2))
        G = int(rng.choice([g for g in _divisors(E) if E // g >= 2])) if sigmoid else 1
        M = int(rng.integers(1, G + 1))
        k = int(rng.integers(1, min(M * (E // G), 8) + 1))
        if kind == "small":
            T = int(rng.integers(1, 512 // k + 1))
        elif kind == "tiled_f32":
            T = int(rng.integers(513 // k + 1, 600 // k + 200))
        elif kind == "tiled_bf16":
            T = int(rng.integers(1, 400))
        elif kind == "stream":
            T = int(rng.integers(-(-64 * E // k), -(-64 * E // k) + 300))
        else:
            T = int(rng.integers(1, max(2, 64 * E // k)))
            T = min(T, 96)
        w = Workload(f"random_{kind}_{i}", T, d, E, k, F, Fs, "sigmoid" if sigmoid else "softmax", G, M,
                     2.5 if sigmoid else 1.0, dtype, "uniform" if rng.integers(0, 2) else "zero")
        if moe.moe_plan_describe(moe.MoeConfig.from_workload(w))[0] == kinds[kind]:
            out[w.name] = w
    return out


RANDOM = random_shapes()


@pytest.mark.parametrize("name", list(RANDOM))
def test_random_shapes_every_token(dev, name):
    w = RANDOM[name]
    log(f"[random] {w}")
    inp = to_dev(make_inputs(w, seed=17, device="cpu"), dev)
    y, idx, g = run(w, inp)
    st = check_full(w, inp, y, idx, g)
    log(f"[random] {name} {st}")
