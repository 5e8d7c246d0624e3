#!/usr/bin/env python3
"""Benchmark of the sparse MoE feed-forward layer forward on one MI355X.

One step = one call of moe_layer_forward over the DeepSeek-V3-shaped prefill
layer (T=8192 tokens, d=7168, 256 routed experts top-8 with sigmoid scores,
8 groups keep 4, selection-only bias, route_scale 2.5, 1 shared expert,
expert width 2048, bf16 with fp32 accumulation): router + top-k, permutation,
gate/up + SiLU*mul, down, combine.  Inputs are seeded synthetic tensors,
resident in HBM before the timed region starts.

The expert weights are packed once before timing (moe_pack_weights: a
one-time re-layout done at model load, identical results); the plain-layout
timing is reported beside it.

Printed: one JSON line with tokens/s, the layer's TFLOP/s and fraction of the
bf16 MFMA peak, the roofline of the dominant kernel (gate/up, from HIP events
recorded by the library on the launch stream during the timed steps), the
decode-shaped layer (T=64, same weights) with its HBM bandwidth, and the CPU
oracle timed on a bounded sample of the same workload.  Informational extras
(``other_configs``): the Mixtral-shaped layer, the skewed layer without and
with the balance-loop bias, and one expert-parallel shard's share of the
DeepSeek-V3 layer.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + % bf16 MFMA peak (DSv3 shape); decode HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0       # MI355X published HBM3E bandwidth
GATE_UP = 2                 # stage index of the gate/up grouped GEMM


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="dsv3_prefill")
    ap.add_argument("--decode-workload", default="dsv3_decode")
    ap.add_argument("--decode-steps", type=int, default=100)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="tokens whose expert outputs the CPU oracle computes")
    ap.add_argument("--plain-weights", action="store_true",
                    help="time the plain weight layout instead of the packed one")
    ap.add_argument("--no-plain", action="store_true",
                    help="skip the reference timing of the plain weight layout")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the informational timings of the other layer shapes")
    ap.add_argument("--no-bodies", action="store_true",
                    help="skip the informational timings of the GEGLU and GELU-MLP expert bodies")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the decode layer replayed from a captured HIP graph")
    ap.add_argument("--no-block", action="store_true",
                    help="skip the timings of the pre-norm residual block (fused and unfused)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, copy a buffer of this many MiB three times (a plain "
                         "copy kernel of known size, to scale hardware byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    """Hash of the sources of the streaming GEMM kernels (the dominant ones)."""
    h = hashlib.sha256()
    for f in ("gemm_stream.hip", "pipeline.hpp", "common.hpp", "plan.hpp"):
        h.update(open(os.path.join(ROOT, "mixture_experts_ffn_biased_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current source of the kernel; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def roofline(kernel, flops, nbytes, ms, traffic, bound=None):
    """Roofline of one kernel from its algorithmic FLOPs and bytes per launch
    and its average launch time.  `bound` names the peak the fraction is
    taken against ("mfma" for the prefill shapes, whose metric is MFMA
    utilisation; "hbm" for the weight-streaming decode shapes); None takes
    whichever peak gives the longer lower-bound time.  Both fractions, and
    the measured-to-algorithmic traffic ratio, are reported beside it."""
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if bound is None:
        bound = "hbm" if t_hbm >= t_mfma else "mfma"
    s = ms * 1e-3
    tflops = flops / s / 1e12
    gbs = nbytes / s / 1e9
    out = {"kernel": kernel}
    if bound == "hbm":
        out.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                   frac=round(gbs / PEAK_HBM_GBS, 4))
    else:
        out.update(bound="mfma", achieved=round(tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                   frac=round(tflops / PEAK_BF16_TFLOPS, 4))
    out.update(traffic=traffic, ms=round(ms, 4), alg_flops=flops, alg_bytes=int(nbytes),
               mfma_frac=round(tflops / PEAK_BF16_TFLOPS, 4), hbm_frac=round(gbs / PEAK_HBM_GBS, 4),
               ridge_flop_per_byte=round(PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9), 1),
               flop_per_byte=round(flops / nbytes, 1),
               traffic_over_alg=None if traffic is None else round(traffic / nbytes, 3))
    return out


def gate_up_flops(w):
    """FLOPs of one gate/up launch: 4 d F per routed slot (W1 and W3 rows) and
    4 d F_shared per token for the shared expert."""
    return 4.0 * w.d * (w.F * w.T * w.k + w.Fs * w.T)


def gate_up_bytes(w, hit, s=2):
    """Algorithmic HBM bytes of one gate/up launch: the W1 and W3 rows of every
    expert hit and of the shared expert once, the token matrix u read once
    (T d s: the gathered rows of the k slots of a token are the same row),
    and each routed slot's and each token's shared F-wide activation written
    once."""
    return ((hit * 2 * w.F * w.d + 2 * w.Fs * w.d) * s + w.T * w.d * s
            + (w.T * w.k * w.F + w.T * w.Fs) * s)


def layer_bytes(w, hit, s=2):
    """Algorithmic HBM bytes of one layer call: the router matrix and bias,
    the three matrices of every expert hit and of the shared expert, u read
    and y written once, and the k indices and gates of every token."""
    return (w.E * w.d * s + 4 * w.E + hit * 3 * w.d * w.F * s + 3 * w.d * w.Fs * s + 2 * w.T * w.d * s
            + 8 * w.T * w.k)


def timed_steps(step, steps, warmup, torch, stage_events=True):
    """Warm-up calls, then `steps` calls between two events.  With
    stage_events the library's per-stage events are recorded in the same
    timed region (the kernel durations the roofline uses); without, nothing
    but the layer calls is in it."""
    import mixture_experts_ffn_biased_amd as moe
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    moe.moe_timing_read(reset=True)
    moe.moe_timing_enable(stage_events)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    moe.moe_timing_enable(False)
    stage_ms, calls = moe.moe_timing_read(reset=True)
    ms = e0.elapsed_time(e1) / steps
    return ms, wall, [s / max(calls, 1) for s in stage_ms], calls


def run_layer(w, inp, u, steps, warmup, torch, packed=None, stage_events=True):
    """Time `steps` layer calls (plain weights, or the packed buffer if given)."""
    import mixture_experts_ffn_biased_amd as moe
    cfg = moe.MoeConfig.from_workload(w)
    dev = u.device
    y = torch.empty((w.T, w.d), dtype=u.dtype, device=dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(cfg, dev)

    def step():
        if packed is not None:
            moe.moe_layer_forward_packed(u, inp["W_router"], inp["bias"], packed, cfg=cfg, y=y,
                                         topk_idx=idx, gates=gates, workspace=ws)
        else:
            moe.moe_layer_forward(u, inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                  inp["shared"], cfg=cfg, y=y, topk_idx=idx, gates=gates,
                                  workspace=ws)

    ms, wall, stage_ms, calls = timed_steps(step, steps, warmup, torch, stage_events)
    return ms, wall, stage_ms, idx, (y, gates)


def graph_ms(w, inp, u, packed, steps, torch):
    """Average time of one layer call replayed from a captured HIP graph (the
    same kernels without the per-call launch work)."""
    import mixture_experts_ffn_biased_amd as moe
    cfg = moe.MoeConfig.from_workload(w)
    dev = u.device
    y = torch.empty((w.T, w.d), dtype=u.dtype, device=dev)
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    ws = moe.alloc_workspace(cfg, dev)

    def step():
        if packed is not None:
            moe.moe_layer_forward_packed(u, inp["W_router"], inp["bias"], packed, cfg=cfg, y=y, topk_idx=idx,
                                         gates=gates, workspace=ws)
        else:
            moe.moe_layer_forward(u, inp["W_router"], inp["bias"], inp["W1"], inp["W3"], inp["W2"],
                                  inp["shared"], cfg=cfg, y=y, topk_idx=idx, gates=gates, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def layer_record(w, ms, stage_ms, hit, path):
    """Throughput fields of one timed layer shape."""
    import mixture_experts_ffn_biased_amd as moe
    tf = w.flops / (ms * 1e-3) / 1e12
    nbytes = layer_bytes(w, hit, 2 if w.dtype == "bf16" else 4)
    return {"T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F, "F_shared": w.Fs, "score_fn": w.score_fn,
            "gemm_path": path, "ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
            "layer_tflops": round(tf, 2), "layer_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
            "experts_hit": hit, "layer_bytes": int(nbytes),
            "flop_per_byte": round(w.flops / nbytes, 1),
            "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, stage_ms)}}


def time_shape(w, inp, steps, warmup, torch, bias=None):
    """Pack the shape's weights, time the packed layer, free the weights' copy.
    Returns the record, the routing and the outputs (y, topk_idx, gates) of
    the last timed call."""
    import mixture_experts_ffn_biased_amd as moe
    cfg = moe.MoeConfig.from_workload(w)
    packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
    if bias is not None:
        inp = dict(inp, bias=bias)
    ms, _, stage_ms, idx, (y, gates) = run_layer(w, inp, inp["u"], steps, warmup, torch, packed)
    hit = int(torch.unique(idx).numel())
    del packed
    return layer_record(w, ms, stage_ms, hit, moe.moe_plan_describe(cfg)[0]), idx, (y, idx, gates)


def oracle_leg(w, inp, out, n_tokens, seed, bias=None):
    """The CPU oracle on a bounded sample of one extra shape (part of the CPU
    baseline leg): routing of every token and the outputs of n_tokens seeded
    tokens (all when T <= n_tokens), its rate on the host cores, and the
    parity of the GPU's outputs `out` (y, topk_idx, gates) on that sample."""
    import numpy as np

    import oracle
    from synthetic import to_numpy
    threads = oracle.default_threads()
    b = inp["bias"] if bias is None else bias
    tok = np.sort(np.random.default_rng(seed).choice(w.T, size=min(n_tokens, w.T), replace=False))
    W = (to_numpy(inp["W1"]), to_numpy(inp["W3"]), to_numpy(inp["W2"]),
         None if inp["shared"] is None else tuple(to_numpy(x) for x in inp["shared"]))
    par, t_route, t_ffn = oracle_check(w, to_numpy(inp["u"]), to_numpy(inp["W_router"]),
                                       b.double().cpu().numpy(), W, np.arange(w.E), to_numpy(out[0]),
                                       out[1].cpu().numpy().astype(np.int64), out[2].cpu().numpy(), tok, threads)
    n = tok.size
    rate = {"value": n / (t_ffn + t_route * n / w.T), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"routing of all {w.T} tokens ({t_route:.2f} s) + outputs of {n} seeded tokens ({t_ffn:.2f} s)"}
    return rate, par


def skew_inputs(w, seed, dev, torch, target=0.90):
    """The skewed layer's inputs with router row 0 = alpha * m, alpha bisected on
    the library's own routing (zero bias) so that `target` of the tokens pick
    expert 0."""
    import mixture_experts_ffn_biased_amd as moe
    from synthetic import make_inputs
    inp = make_inputs(w, seed=seed, device=dev, expert0_scale=1.0)
    cfg = moe.MoeConfig.from_workload(w)
    m = inp["skew_dir"]
    ws = moe.alloc_workspace(cfg, dev)

    def share(alpha):
        inp["W_router"][0] = (float(alpha) * m).to(inp["W_router"].dtype)
        idx = moe.moe_route_debug(inp["u"], inp["W_router"], None, cfg=cfg, workspace=ws)[0]
        return (idx == 0).any(dim=1).float().mean().item()
    lo, hi = 0.0, 1.0
    while share(hi) < target and hi < 1e3:
        hi *= 2
    for _ in range(30):
        mid = 0.5 * (lo + hi)
        lo, hi = (mid, hi) if share(mid) < target else (lo, mid)
    got = share(hi)
    return inp, hi, got


def expert_bodies(w, inp, args, torch):
    """The same layer with GEGLU experts and with biased GELU-MLP experts, on
    weights packed for each body (moe_pack_weights_ex, not timed)."""
    import mixture_experts_ffn_biased_amd as moe
    from synthetic import make_ffn_biases
    cfg = moe.MoeConfig.from_workload(w)
    dev = inp["u"].device
    fb = make_ffn_biases(w, seed=args.seed, device=dev)
    y = torch.empty_like(inp["u"])
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device=dev)
    gates = torch.empty((w.T, w.k), dtype=torch.float32, device=dev)
    W1s, W3s, W2s = inp["shared"]
    out = {}
    for kind in ("geglu", "gelu_mlp"):
        gated = kind == "geglu"
        packed = moe.moe_pack_weights_ex(kind, inp["W1"], inp["W3"] if gated else None, inp["W2"],
                                         (W1s, W3s if gated else None, W2s), cfg=cfg)
        ws = torch.empty(max(moe.moe_workspace_bytes_ex(cfg, kind), 256), dtype=torch.uint8, device=dev)
        b = (None,) * 4 if gated else (fb["b1"], fb["b2"], fb["b1s"], fb["b2s"])

        def step():
            moe.moe_layer_forward_packed_ex(inp["u"], inp["W_router"], inp["bias"], kind, packed, *b, cfg=cfg, y=y,
                                            topk_idx=idx, gates=gates, workspace=ws)
        ms, _, stage_ms, _ = timed_steps(step, args.steps, args.warmup, torch)
        # FLOPs: router + (6 or 4) d F per routed slot and per token for the shared expert
        per = 6.0 if gated else 4.0
        flops = w.T * (2.0 * w.d * w.E + per * w.d * w.F * w.k + per * w.d * w.Fs)
        tf = flops / (ms * 1e-3) / 1e12
        out[kind] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.T / (ms * 1e-3), 1),
                     "layer_tflops": round(tf, 2), "layer_mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "gemm_path": moe.moe_plan_describe_ex(cfg, kind)[0], "weights": "packed",
                     "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, stage_ms)}}
        del ws, packed
        torch.cuda.empty_cache()
    return out


def other_configs(args, torch, dev):
    """Informational timings of the other layer shapes (packed weights)."""
    import mixture_experts_ffn_biased_amd as moe
    from synthetic import EP_SHARD, WORKLOADS, make_inputs
    out = {}
    cpu = not args.no_cpu_baseline

    def cpu_leg(rec, w, inp, res, n, bias=None):
        # the oracle on a bounded sample, outside every timed region
        if cpu:
            rec["cpu_oracle"], rec["parity"] = oracle_leg(w, inp, res, n, args.seed, bias)

    # the tiny fp32 layer (tiled kernels, plain weights): a latency figure
    w = WORKLOADS["tiny_fp32"]
    log(f"[bench] {w.name}")
    inp = make_inputs(w, seed=args.seed, device=dev)
    # timed without the per-stage events in the timed region (at this size they would be most of it), the
    # stage split from a second run with them; and replayed from a captured graph (no per-call launch work)
    ms, _, stage_ms, idx, (y, gates) = run_layer(w, inp, inp["u"], 100, args.warmup, torch, None)
    ms_plain = run_layer(w, inp, inp["u"], 100, args.warmup, torch, None, stage_events=False)[0]
    rec = layer_record(w, ms_plain, stage_ms, int(torch.unique(idx).numel()), moe.moe_plan_describe(
        moe.MoeConfig.from_workload(w))[0])
    rec.update(weights="plain", latency_us=round(ms_plain * 1e3, 2),
               latency_us_with_stage_events=round(ms * 1e3, 2))
    if not args.no_graph:
        rec["graph_replay_latency_us"] = round(graph_ms(w, inp, inp["u"], None, 100, torch) * 1e3, 2)
    cpu_leg(rec, w, inp, (y, idx, gates), w.T)
    out[w.name] = rec
    del inp
    w = WORKLOADS["mixtral_e8_top2"]
    log(f"[bench] {w.name}")
    inp = make_inputs(w, seed=args.seed, device=dev)
    out[w.name], _, res = time_shape(w, inp, args.steps, args.warmup, torch)
    cpu_leg(out[w.name], w, inp, res, 64)
    del inp, res
    w = EP_SHARD
    log(f"[bench] {w.name}")
    inp = make_inputs(w, seed=args.seed, device=dev)
    out[w.name], _, _ = time_shape(w, inp, args.steps, args.warmup, torch)
    del inp
    w = WORKLOADS["skewed_e128_top8"]
    log(f"[bench] {w.name}: calibrating the skew on the library's routing")
    inp, alpha, got = skew_inputs(w, args.seed, dev, torch)
    rec_a, idx, res = time_shape(w, inp, args.steps, args.warmup, torch)
    rec_a.update(bias="zero", expert0_scale=round(alpha, 4), expert0_share=round(got, 4),
                 expert0_rows=int((idx == 0).sum().item()))
    cpu_leg(rec_a, w, inp, res, 256)
    del res
    # the aux-loss-free balance loop on the device: 10 steps of +-0.15 from zero
    cfg = moe.MoeConfig.from_workload(w)
    ws = moe.alloc_workspace(cfg, dev)
    b = torch.zeros(w.E, dtype=torch.float32, device=dev)
    for _ in range(10):
        idx = moe.moe_route_debug(inp["u"], inp["W_router"], b, cfg=cfg, workspace=ws)[0]
        moe.moe_balance_update(idx, b, E=w.E, gamma=0.15)
    rec_b, idx, res = time_shape(w, inp, args.steps, args.warmup, torch, bias=b)
    rec_b.update(bias="10 on-device balance steps, gamma 0.15",
                 expert0_rows=int((idx == 0).sum().item()))
    cpu_leg(rec_b, w, inp, res, 256, bias=b)
    del res
    out[w.name + "_a"] = rec_a
    out[w.name + "_b"] = rec_b
    del inp, ws
    torch.cuda.empty_cache()
    return out


def tile_edge_tokens(w, inp, u, torch):
    """Tokens in the first and last row of every routed and shared tile the
    grouped GEMMs run for this input (from the library's own permutation):
    where an error in a tile's row range would show."""
    import numpy as np

    import mixture_experts_ffn_biased_amd as moe
    cfg = moe.MoeConfig.from_workload(w)
    path, tile_m = moe.moe_plan_describe(cfg)
    _, _, counts, offsets, perm, _ = moe.moe_route_debug(u, inp["W_router"], inp["bias"], cfg=cfg)
    counts, offsets, perm = counts.cpu().numpy(), offsets.cpu().numpy(), perm.cpu().numpy()
    toks = set()

    def edges(base, c, is_shared):
        nt = -(-c // tile_m)
        for i in range(nt):
            if path == "stream":  # rows spread evenly over the expert's tiles
                q, r = divmod(c, nt)
                r0, n = i * q + min(i, r), q + (1 if i < r else 0)
            else:
                r0, n = i * tile_m, min(tile_m, c - i * tile_m)
            for row in (r0, r0 + n - 1):
                toks.add(int(row) if is_shared else int(perm[base + row]) // w.k)
    for e in range(w.E):
        edges(int(offsets[e]), int(counts[e]), False)
    if w.Fs:
        edges(0, w.T, True)
    return np.array(sorted(toks), dtype=np.int64)


def oracle_check(w, u_host, Wr, bias, W, used, gpu_y, gpu_idx, gpu_gates, tok, threads):
    """The oracle's routing of every token and its outputs for the tokens
    `tok`, compared with the GPU's: near-tie counts (k-th / (k+1)-th biased
    expert score or M-th / (M+1)-th group score within 1e-5 relative), tokens
    whose expert set differs without a near-tie, the largest gate error and
    the largest per-token relative L2 error of y.  A near-tie token the GPU
    broke the other way is compared with the oracle run on the GPU's choice."""
    import numpy as np

    import oracle
    mode = oracle.SIGMOID if w.score_fn == "sigmoid" else oracle.SOFTMAX
    t = time.perf_counter()
    ir, gr, ge, gg, _ = oracle.route(u_host, Wr, w.k, mode, w.n_groups, w.topk_groups, w.route_scale,
                                     bias=bias, nthreads=threads)
    t_route = time.perf_counter() - t
    near = (ge < 1e-5) | (gg < 1e-5)
    same = (np.sort(gpu_idx, 1) == np.sort(ir, 1)).all(1)
    ok = same & ~near
    g = np.take_along_axis(gpu_gates.astype(np.float64)[ok], np.argsort(gpu_idx[ok], 1), 1)
    r = np.take_along_axis(gr[ok], np.argsort(ir[ok], 1), 1)
    gate_err = float((np.abs(g - r) / np.maximum(1.0, np.abs(r))).max()) if g.size else 0.0
    sel = np.where(near[tok, None], gpu_idx[tok], ir[tok]).astype(np.int64)
    remap = np.full(w.E, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    assert (remap[sel] >= 0).all()
    W1, W3, W2, shared = W
    t = time.perf_counter()
    yr, _, _, _, _ = oracle.forward(u_host[tok], Wr[used], W1, W3, W2, w.k, shared=shared, score_fn=mode,
                                    route_scale=w.route_scale, forced_idx=remap[sel], nthreads=threads)
    t_ffn = time.perf_counter() - t
    yg = oracle.widen(gpu_y[tok])
    err = np.linalg.norm(yg - yr, axis=1) / np.maximum(np.linalg.norm(yr, axis=1), 1e-30)
    tol = 1e-2 if w.dtype == "bf16" else 1e-5
    rec = {"tokens_routed": int(w.T), "near_ties": int(near.sum()),
           "near_tie_diffs": int((~same & near).sum()),
           "set_mismatches_without_near_tie": int((~same & ~near).sum()),
           "gate_err_max": gate_err, "outputs_checked": int(tok.size),
           "rel_l2_max": float(err.max()), "rel_l2_tol": tol}
    rec["pass"] = rec["set_mismatches_without_near_tie"] == 0 and gate_err <= 1e-5 and rec["rel_l2_max"] <= tol
    return rec, t_route, t_ffn


def cpu_baseline(w, inp, n_tokens, seed, gpu_out, edge_tok, decode=None):
    """The oracle, as it stands, on the host cores: routing of every token and
    the expert outputs of a bounded sample of tokens -- the tokens in the
    first and last row of every GEMM tile, then seeded random ones up to
    n_tokens.  The same oracle results give the parity record of the timed
    run's outputs (gpu_out: y, topk_idx, gates), and of the decode-shaped
    layer's (decode: workload, u, y, topk_idx, gates; every token)."""
    import numpy as np
    import torch

    import oracle
    from synthetic import to_numpy

    u = to_numpy(inp["u"])
    Wr = to_numpy(inp["W_router"])
    bias = inp["bias"].double().cpu().numpy()
    threads = oracle.default_threads()
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(w.T), edge_tok)
    extra = max(0, min(n_tokens, w.T) - edge_tok.size)
    tok = np.sort(np.concatenate([edge_tok, rng.choice(rest, size=min(extra, rest.size), replace=False)]))
    gi = gpu_out[1].cpu().numpy().astype(np.int64)
    # every expert either layer's checked tokens may use: the GPU's and the oracle's choice
    used = np.arange(w.E)
    t = time.perf_counter()
    W1 = to_numpy(inp["W1"])
    W3 = to_numpy(inp["W3"])
    W2 = to_numpy(inp["W2"])
    shared = None if inp["shared"] is None else tuple(to_numpy(x) for x in inp["shared"])
    t_copy = time.perf_counter() - t
    W = (W1, W3, W2, shared)
    par, t_route, t_ffn = oracle_check(w, u, Wr, bias, W, used, to_numpy(gpu_out[0]), gi,
                                       gpu_out[2].cpu().numpy(), tok, threads)
    par["tile_edge_tokens"] = int(edge_tok.size)
    parity = {w.name: par}
    decode_rate = None
    n = tok.size
    value = n / (t_ffn + t_route * n / w.T)
    if decode is not None:
        wd, ud, yd, idd, gd = decode
        pd, td_route, td_ffn = oracle_check(wd, to_numpy(ud), Wr, bias, W, used, to_numpy(yd),
                                            idd.cpu().numpy().astype(np.int64), gd.cpu().numpy(),
                                            np.arange(wd.T), threads)
        parity[wd.name] = pd
        decode_rate = {"value": wd.T / (td_route + td_ffn), "unit": "tokens/s", "cores": threads,
                       "kind": "oracle",
                       "sample": (f"{wd.name}: routing ({td_route:.2f} s) and expert and shared outputs "
                                  f"({td_ffn:.2f} s) of all {wd.T} tokens")}
    base = {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"{w.name}: routing of all {w.T} tokens ({t_route:.2f} s) + expert and "
                       f"shared outputs of {n} tokens: the {edge_tok.size} in the first or last row of a "
                       f"GEMM tile and seeded random ones ({t_ffn:.2f} s); tokens/s = "
                       f"n / (t_ffn + t_route * n / T); device-to-host copy of the weights "
                       f"({t_copy:.2f} s) excluded")}
    return base, parity, decode_rate


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE "
              f"{world}); this layer build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_ffn_biased_amd as moe
    from synthetic import WORKLOADS, make_inputs, make_u

    moe.lib()
    dev = torch.device("cuda:0")
    w = WORKLOADS[args.workload]
    log(f"[bench] generating {w.name} inputs on {dev}")
    inp = make_inputs(w, seed=args.seed, device=dev)
    torch.cuda.synchronize()

    cfg = moe.MoeConfig.from_workload(w)
    packed = None
    if not args.plain_weights:
        log("[bench] packing the expert weights (one-time layout change, not timed)")
        packed = moe.moe_pack_weights(inp["W1"], inp["W3"], inp["W2"], inp["shared"], cfg=cfg)
        torch.cuda.synchronize()
    log(f"[bench] {w.name}: {args.warmup} warm-up + {args.steps} timed steps")
    ms, wall, stage_ms, idx, (y_out, g_out) = run_layer(w, inp, inp["u"], args.steps, args.warmup, torch,
                                                        packed)
    tokens_per_s = w.T / (ms * 1e-3)
    layer_tflops = w.flops / (ms * 1e-3) / 1e12
    hit_p = int(torch.unique(idx).numel())
    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; u ~ N(0,1), weights ~ N(0, 1/fan_in), bias ~ U(-0.05, 0.05))",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F,
                   "F_shared": w.Fs, "score_fn": w.score_fn, "n_groups": w.n_groups,
                   "topk_groups": w.topk_groups, "route_scale": w.route_scale,
                   "weights": "plain" if packed is None else "packed"},
        "layer_tflops": round(layer_tflops, 2),
        "layer_mfma_frac": round(layer_tflops / PEAK_BF16_TFLOPS, 4),
        "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, stage_ms)},
        "experts_hit": hit_p,
        # the prefill metric is MFMA utilisation: the fraction is taken against the bf16 MFMA peak
        "roofline": roofline("gemm_stream_prefill<gate_up>", gate_up_flops(w), gate_up_bytes(w, hit_p),
                             stage_ms[GATE_UP], stored_traffic(f"gate_up_{w.name}"), bound="mfma"),
    }

    # the layer inside its pre-norm residual block: y = u + MoE(RMSNorm(u)), with the
    # normalisation fused into the router and gate/up (norm weight folded into a
    # packed buffer once, not timed), and unfused (a separate RMSNorm pass)
    if packed is not None and not args.no_block:
        from synthetic import make_norm_weight
        g = make_norm_weight(w, seed=args.seed, device=dev)
        bws = moe.alloc_block_workspace(cfg, dev)
        yb = torch.empty_like(inp["u"])
        fpk = moe.moe_pack_block_weights(g, inp["W_router"], inp["W1"], inp["W3"], inp["W2"], inp["shared"],
                                         cfg=cfg)

        def fused_step():
            moe.moe_block_forward_fused(inp["u"], 1e-6, inp["bias"], fpk, cfg=cfg, y=yb, workspace=bws)
        fms, _, fstage, _ = timed_steps(fused_step, args.steps, args.warmup, torch)
        del fpk
        torch.cuda.empty_cache()

        def block_step():
            moe.moe_block_forward_packed(inp["u"], g, 1e-6, inp["W_router"], inp["bias"], packed, cfg=cfg, y=yb,
                                         workspace=bws)
        bms, _, _, _ = timed_steps(block_step, args.steps, args.warmup, torch)
        un = torch.empty_like(inp["u"])
        for _ in range(5):
            moe.moe_rmsnorm(inp["u"], g, 1e-6, out=un)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            moe.moe_rmsnorm(inp["u"], g, 1e-6, out=un)
        e1.record()
        torch.cuda.synchronize()
        nms = e0.elapsed_time(e1) / 50
        result["block"] = {"ms_per_step": round(fms, 4), "tokens_per_s": round(w.T / (fms * 1e-3), 1),
                           "form": "fused (norm weight folded into the packed weights, 1/rms in the router)",
                           "minus_layer_ms": round(fms - ms, 4),
                           "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, fstage)},
                           "unfused_ms_per_step": round(bms, 4),
                           "rmsnorm_us": round(nms * 1e3, 2),
                           "rmsnorm_GBps": round(2 * w.T * w.d * 2 / (nms * 1e-3) / 1e9, 1)}
        del bws, yb, un

    # one aux-loss-free balance step on this layer's routing (bias updated on a copy)
    bias_copy = inp["bias"].clone()
    for _ in range(5):
        moe.moe_balance_update(idx, bias_copy, E=w.E)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(100):
        moe.moe_balance_update(idx, bias_copy, E=w.E)
    e1.record()
    torch.cuda.synchronize()
    bu_ms = e0.elapsed_time(e1) / 100
    bu_bytes = 4 * w.T * w.k + 12 * w.E
    result["balance_update"] = {"us": round(bu_ms * 1e3, 2), "slots": w.T * w.k,
                                "GBps": round(bu_bytes / (bu_ms * 1e-3) / 1e9, 1)}

    if not args.no_decode:
        wd = WORKLOADS[args.decode_workload]
        ud = make_u(wd, seed=args.seed, device=dev)
        log(f"[bench] {wd.name}: {args.warmup} warm-up + {args.decode_steps} timed steps")
        dms, _, dstage, didx, (yd_out, gd_out) = run_layer(wd, inp, ud, args.decode_steps, args.warmup, torch,
                                                           packed)
        hit = int(torch.unique(didx).numel())
        dbytes = layer_bytes(wd, hit)
        gbs = dbytes / (dms * 1e-3) / 1e9
        result["decode"] = {
            "workload": wd.name, "T": wd.T, "ms_per_step": round(dms, 4),
            "tokens_per_s": round(wd.T / (dms * 1e-3), 1), "experts_hit": hit,
            "layer_bytes": dbytes, "layer_GBps": round(gbs, 1),
            "layer_hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, dstage)},
            # the decode metric is HBM bandwidth: the fraction is taken against the HBM peak
            "roofline": roofline("gemm_stream_decode<gate_up>", gate_up_flops(wd), gate_up_bytes(wd, hit),
                                 dstage[GATE_UP], stored_traffic(f"gate_up_{wd.name}"), bound="hbm"),
        }
        if packed is not None and not args.no_graph:
            gms = graph_ms(wd, inp, ud, packed, args.decode_steps, torch)
            result["decode"]["graph_replay"] = {
                "ms_per_step": round(gms, 4), "layer_GBps": round(dbytes / (gms * 1e-3) / 1e9, 1),
                "layer_hbm_frac": round(dbytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    if packed is not None and not args.no_plain:
        # the same layer with the weights in their plain layout, for reference
        pms, _, pstage, _, _ = run_layer(w, inp, inp["u"], max(3, args.steps // 2), 2, torch, None)
        result["plain_weights"] = {"ms_per_step": round(pms, 4),
                                   "tokens_per_s": round(w.T / (pms * 1e-3), 1),
                                   "stage_ms": {n: round(v, 4) for n, v in zip(moe.STAGES, pstage)}}

    if packed is not None and not args.no_bodies:
        result["expert_bodies"] = expert_bodies(w, inp, args, torch)

    if not args.no_others:
        result["other_configs"] = other_configs(args, torch, dev)

    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline on {args.cpu_tokens} tokens, parity of the timed outputs")
        edge = tile_edge_tokens(w, inp, inp["u"], torch)
        dec = None if args.no_decode else (wd, ud, yd_out, didx, gd_out)
        result["cpu_baseline"], result["parity"], decode_rate = cpu_baseline(
            w, inp, args.cpu_tokens, args.seed, (y_out, idx, g_out), edge, decode=dec)
        if decode_rate is not None:
            result["decode"]["cpu_oracle"] = decode_rate
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
