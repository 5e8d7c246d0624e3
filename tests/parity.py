"""Parity helpers: compare the HIP path with the CPU oracle on the same inputs.

Rules (the parity bar of the layer):
  * top-k: the GPU's expert set per token equals the oracle's, except tokens
    whose last-chosen and first-rejected biased scores (or group scores) are
    within 1e-5 relative (|a-b| / max(|a|,|b|,1)); those near-ties are counted
    and, where the GPU chose differently, its own choice is re-checked by the
    oracle with that selection forced;
  * order: descending biased score; adjacent picks whose scores are within
    the same 1e-5 may swap;
  * gates: |g - g_ref| <= 1e-5 * max(1, |g_ref|), matched by expert id;
  * outputs: per-token relative L2 error <= 1e-2 (bf16) or 1e-5 (fp32).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from synthetic import to_numpy

TIE_TOL = 1e-5
GATE_TOL = 1e-5
Y_TOL = {"bf16": 1e-2, "f32": 1e-5}

# Per-case parity statistics of this test session (near-tie counts, the
# largest rel-L2, tokens and tiles checked); conftest writes them to the
# JSON file named by MOE_PARITY_RECORD at the end of the session.
RECORD = {}


def record(name, stats):
    RECORD[name] = dict(stats)


def mode_of(w):
    return oracle.SIGMOID if w.score_fn == "sigmoid" else oracle.SOFTMAX


def biased_scores(w, logits, bias):
    s = 1.0 / (1.0 + np.exp(-logits)) if w.score_fn == "sigmoid" else logits
    return s + (0.0 if bias is None else np.asarray(bias, dtype=np.float64))


def route_parity(w, gpu_idx, gpu_gates, ref_idx, ref_gates, gap_e, gap_g, logits, bias):
    """Checks selection, order and gates; returns a stats dict."""
    gpu_idx = np.asarray(gpu_idx)
    T, k = ref_idx.shape
    assert gpu_idx.shape == (T, k)
    assert ((gpu_idx >= 0) & (gpu_idx < w.E)).all(), "expert index out of range"
    assert all(len(set(r)) == k for r in gpu_idx.tolist()), "repeated expert in a token"
    near = (gap_e < TIE_TOL) | (gap_g < TIE_TOL)
    same = (np.sort(gpu_idx, 1) == np.sort(ref_idx, 1)).all(1)
    bad = ~same & ~near
    assert not bad.any(), (f"{int(bad.sum())} tokens select different experts with no near-tie; "
                           f"first {np.nonzero(bad)[0][:8].tolist()}")
    ok = same & ~near
    og = np.argsort(gpu_idx[ok], 1)
    orf = np.argsort(ref_idx[ok], 1)
    g = np.take_along_axis(np.asarray(gpu_gates, dtype=np.float64)[ok], og, 1)
    r = np.take_along_axis(ref_gates[ok], orf, 1)
    gerr = np.abs(g - r) / np.maximum(1.0, np.abs(r))
    assert gerr.size == 0 or gerr.max() <= GATE_TOL, f"gate error {gerr.max():.3e}"
    # order: descending biased score, swaps allowed only within the tie margin
    sb = biased_scores(w, logits, bias)
    chosen = np.take_along_axis(sb, gpu_idx.astype(np.int64), 1)
    a, b = chosen[:, :-1], chosen[:, 1:]
    gap = np.abs(a - b) / np.maximum(1.0, np.maximum(np.abs(a), np.abs(b)))
    misorder = (b > a) & (gap >= TIE_TOL)
    assert not misorder.any(), f"{int(misorder.any(1).sum())} tokens out of order"
    return {"tokens": int(T), "near_ties": int(near.sum()),
            "near_tie_diffs": int((~same & near).sum()),
            "gate_err_max": float(gerr.max()) if gerr.size else 0.0}


def rel_l2(y, ref):
    y = np.asarray(y, dtype=np.float64)
    num = np.linalg.norm(y - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-30)
    return num / den


def host(t):
    return to_numpy(t)


def widen_gpu(t):
    return oracle.widen(to_numpy(t))


def oracle_inputs(inp):
    """Exact host copies of a workload's small tensors."""
    u = host(inp["u"])
    Wr = host(inp["W_router"])
    bias = inp["bias"].detach().cpu().numpy().astype(np.float64)
    return u, Wr, bias


def sampled_outputs(w, inp, tokens, sel, nthreads=None):
    """Oracle outputs for tokens with the given selections, fetching only the
    experts those tokens use (compact expert table, indices remapped)."""
    tokens = np.asarray(tokens, dtype=np.int64)
    sel = np.asarray(sel, dtype=np.int64)
    used = np.unique(sel)
    remap = np.full(w.E, -1, dtype=np.int64)
    remap[used] = np.arange(used.size)
    dev = inp["W1"].device
    ui = torch.from_numpy(used).to(dev)
    u = host(inp["u"].index_select(0, torch.from_numpy(tokens).to(dev)))
    Wr = host(inp["W_router"].index_select(0, ui))
    W1 = host(inp["W1"].index_select(0, ui))
    W3 = host(inp["W3"].index_select(0, ui))
    W2 = host(inp["W2"].index_select(0, ui))
    shared = None
    if inp["shared"] is not None:
        shared = tuple(host(t) for t in inp["shared"])
    y, idx, gates, _, _ = oracle.forward(
        u, Wr, W1, W3, W2, w.k, shared=shared, score_fn=mode_of(w), n_groups=1, topk_groups=1,
        route_scale=w.route_scale, forced_idx=remap[sel], nthreads=nthreads)
    return y, used[idx], gates


def tile_spans(path, tile_m, counts, n_tokens, has_shared):
    """Row spans (expert, first position, rows) of every tile the grouped GEMMs
    run: each expert's rows in tiles of at most tile_m, spread evenly over
    ceil(c / tile_m) tiles on the prefill streaming path and in full tiles with
    a ragged last one elsewhere, then the shared expert's T rows the same way.
    Positions index the expert-contiguous order (offsets[e] + row)."""
    balanced = path == "stream"
    spans = []

    def split(e, base, c):
        nt = -(-c // tile_m)
        for i in range(nt):
            if balanced:
                q, r = divmod(c, nt)
                r0, n = i * q + min(i, r), q + (1 if i < r else 0)
            else:
                r0, n = i * tile_m, min(tile_m, c - i * tile_m)
            spans.append((e, base + r0, n))

    off = 0
    for e, c in enumerate(np.asarray(counts).tolist()):
        split(e, off, int(c))
        off += int(c)
    if has_shared:
        split(len(counts), 0, int(n_tokens))
    return spans


def tile_edge_tokens(w, path, tile_m, counts, perm, n_tokens):
    """Tokens that sit in the first and last row of every routed and shared
    tile, and in the rows either side of the 128-row split of a 256-row tile
    (the two wave rows of the prefill kernels): the rows where a wrong tile
    offset, row count or row-group bound would show."""
    perm = np.asarray(perm, dtype=np.int64)
    E = len(counts)
    toks = set()
    spans = tile_spans(path, tile_m, counts, n_tokens, w.Fs > 0)
    for e, p0, n in spans:
        rows = {0, n - 1}
        if n > 128:
            rows |= {127, 128}
        for r in rows:
            toks.add(int(p0 + r) if e == E else int(perm[p0 + r] // w.k))
    return np.array(sorted(toks), dtype=np.int64), len(spans)
