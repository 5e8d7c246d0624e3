"""Pins of the CPU oracle against what the pages and mathematics fix.

Every test here runs on the CPU.  Each pins a part of the oracle to something
other than the oracle itself: hand-worked examples, brute-force enumeration,
closed forms, library routines (NumPy/PyTorch float64), invariants of the
method, and a second independent implementation.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import balance, expert_major

HERE = os.path.dirname(os.path.abspath(__file__))
MODE = {"softmax": oracle.SOFTMAX, "sigmoid": oracle.SIGMOID}


def _onehot_inputs(logits):
    """u = e_0 and W_router[e] = [logit_e, 0, ...], so the router returns logits."""
    E = len(logits)
    d = 4
    u = np.zeros((1, d))
    u[0, 0] = 1.0
    Wr = np.zeros((E, d))
    Wr[:, 0] = logits
    return u, Wr


# ---------------------------------------------------------------- worked examples

def test_worked_examples_from_fixture():
    spec = json.load(open(os.path.join(HERE, "golden", "route_worked_examples.json")))
    for ex in spec["examples"]:
        u, Wr = _onehot_inputs(ex["logits"])
        idx, gates, _, _, lg = oracle.route(
            u, Wr, ex["k"], MODE[ex["score_fn"]], ex["n_groups"], ex["topk_groups"],
            ex["route_scale"], bias=np.array(ex["bias"]))
        assert lg[0].tolist() == ex["logits"], ex["name"]
        assert idx[0].tolist() == ex["expected_idx"], ex["name"]
        np.testing.assert_allclose(gates[0], ex["expected_gates"], rtol=1e-12, atol=0,
                                   err_msg=ex["name"])


# ---------------------------------------------------------------- P-1 brute force

def _brute_force_select(sb, k, n_groups, topk_groups):
    """Max-sum k-subset (exact rational sums), ties -> lexicographically
    smallest index tuple; two-stage when grouped.  Scores must be finite."""
    E = len(sb)
    eligible = list(range(E))
    if n_groups > 1:
        per = E // n_groups
        gscore = []
        for g in range(n_groups):
            members = range(g * per, (g + 1) * per)
            # largest rounded pair sum == sum of the two largest (rounding is monotone)
            gscore.append(max(sb[a] + sb[b] for a, b in itertools.combinations(members, 2)))
        best = None
        for groups in itertools.combinations(range(n_groups), topk_groups):
            key = sum(Fraction(gscore[g]) for g in groups)
            if best is None or key > best[0]:
                best = (key, groups)
        eligible = [e for g in best[1] for e in range(g * per, (g + 1) * per)]
    best = None
    for subset in itertools.combinations(eligible, k):
        key = sum(Fraction(sb[e]) for e in subset)
        if best is None or key > best[0]:
            best = (key, subset)
    return set(best[1])


def _check_order(idx_row, sb):
    for a, b in zip(idx_row[:-1], idx_row[1:]):
        assert sb[a] > sb[b] or (sb[a] == sb[b] and a < b)


@pytest.mark.parametrize("E,k", [(8, 2), (10, 3), (6, 6), (5, 1)])
def test_brute_force_softmax_mode_with_forced_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T, d = 200, 6
    u = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    Wr = rng.integers(-2, 3, size=(E, d)).astype(np.float64)
    bias = rng.integers(-2, 3, size=E) * 0.5
    for b in (None, bias):
        idx, gates, _, _, lg = oracle.route(u, Wr, k, oracle.SOFTMAX, bias=b)
        assert np.array_equal(lg, u @ Wr.T)  # integer logits, exact
        sb_all = lg + (0 if b is None else b)
        for t in range(T):
            sb = sb_all[t].tolist()
            assert set(idx[t].tolist()) == _brute_force_select(sb, k, 1, 1)
            assert len(set(idx[t].tolist())) == k
            _check_order(idx[t].tolist(), sb)


@pytest.mark.parametrize("E,G,M,k,score", [(16, 4, 2, 4, "sigmoid"), (16, 4, 2, 4, "softmax"),
                                           (12, 3, 1, 2, "sigmoid"), (8, 4, 3, 5, "sigmoid")])
def test_brute_force_group_limited(E, G, M, k, score):
    rng = np.random.default_rng(E * 1000 + G * 10 + M + k)
    T, d = 150, 5
    u = rng.integers(-2, 3, size=(T, d)).astype(np.float64)
    Wr = rng.integers(-1, 2, size=(E, d)).astype(np.float64)
    bias = rng.integers(-2, 3, size=E) * 0.25
    idx, gates, _, _, lg = oracle.route(u, Wr, k, MODE[score], G, M, 2.5, bias=bias)
    for t in range(T):
        s = [1.0 / (1.0 + math.exp(-x)) if score == "sigmoid" else x for x in lg[t]]
        sb = [a + b for a, b in zip(s, bias)]
        assert set(idx[t].tolist()) == _brute_force_select(sb, k, G, M), t
        _check_order(idx[t].tolist(), sb)


def test_nan_scores_rank_last_and_indices_stay_valid():
    logits = np.array([[np.nan, 1.0, np.nan, 0.5, -3.0, np.nan]])
    idx, gates, _, _ = oracle.select(logits, 4, oracle.SOFTMAX)
    assert idx[0].tolist() == [1, 3, 4, 0]
    all_nan = np.full((1, 8), np.nan)
    for mode, G, M in ((oracle.SOFTMAX, 1, 1), (oracle.SIGMOID, 4, 2)):
        idx, gates, _, _ = oracle.select(all_nan, 3, mode, G, M)
        assert idx[0].tolist() == [0, 1, 2]


# ---------------------------------------------------------------- P-2 closed forms

def test_gate_closed_forms():
    rng = np.random.default_rng(1)
    T, d, E = 300, 16, 32
    u = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / 4
    bias = rng.uniform(-0.05, 0.05, E)
    idx, g, _, _, lg = oracle.route(u, Wr, 4, oracle.SOFTMAX, bias=bias)
    np.testing.assert_allclose(g.sum(1), 1.0, rtol=0, atol=1e-12)
    chosen = np.take_along_axis(lg, idx.astype(np.int64), 1)
    np.testing.assert_allclose(g[:, 1:] / g[:, :1], np.exp(chosen[:, 1:] - chosen[:, :1]),
                               rtol=1e-12)
    idx, g, _, _, lg = oracle.route(u, Wr, 8, oracle.SIGMOID, 8, 4, 2.5, bias=bias)
    np.testing.assert_allclose(g.sum(1), 2.5, rtol=0, atol=1e-12)
    s = 1 / (1 + np.exp(-np.take_along_axis(lg, idx.astype(np.int64), 1)))
    np.testing.assert_allclose(g[:, 1:] / g[:, :1], s[:, 1:] / s[:, :1], rtol=1e-12)


# ---------------------------------------------------------------- P-3 bias is selection-only

@pytest.mark.parametrize("mode,G,M,scale", [(oracle.SOFTMAX, 1, 1, 1.0), (oracle.SIGMOID, 8, 4, 2.5)])
def test_bias_changes_selection_never_gate_values(mode, G, M, scale):
    rng = np.random.default_rng(2)
    T, d, E, k = 200, 16, 64, 6
    u = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / 4
    bias = rng.uniform(-0.05, 0.05, E)
    lg = oracle.router_logits(u, Wr)
    idx0, g0, _, _ = oracle.select(lg, k, mode, G, M, scale, bias)
    # A perturbation that keeps every selected set keeps gates bit-identical.
    idx1, g1, _, _ = oracle.select(lg, k, mode, G, M, scale, bias * (1 + 1e-9))
    same = (np.sort(idx0, 1) == np.sort(idx1, 1)).all(1)
    assert same.mean() > 0.95
    for t in np.nonzero(same)[0]:
        a = dict(zip(idx0[t], g0[t]))
        b = dict(zip(idx1[t], g1[t]))
        assert all(a[e] == b[e] for e in a)
    # A huge bias forces expert 5 into every set; its gate still uses the raw score.
    big = bias.copy()
    big[5] = 1e6
    idx2, g2, _, _ = oracle.select(lg, k, mode, G, M, scale, big)
    assert (idx2[:, 0] == 5).all()
    s = lg if mode == oracle.SOFTMAX else 1 / (1 + np.exp(-lg))
    chosen = np.take_along_axis(s, idx2.astype(np.int64), 1)
    if mode == oracle.SOFTMAX:
        z = np.exp(chosen - chosen.max(1, keepdims=True))
        ref = scale * z / z.sum(1, keepdims=True)
    else:
        ref = scale * chosen / chosen.sum(1, keepdims=True)
    np.testing.assert_allclose(g2, ref, rtol=1e-13)


# ---------------------------------------------------------------- P-4 zero bias

def test_zero_bias_equals_no_bias_and_the_softmax_all_router():
    rng = np.random.default_rng(3)
    T, d, E, k = 300, 24, 16, 3
    u = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d)) / 4
    for mode, G, M in ((oracle.SOFTMAX, 1, 1), (oracle.SIGMOID, 4, 2)):
        a = oracle.route(u, Wr, k, mode, G, M, bias=None)
        b = oracle.route(u, Wr, k, mode, G, M, bias=np.zeros(E))
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    idx, g, _, _, _ = oracle.route(u, Wr, k, oracle.SOFTMAX)
    ridx, rw = expert_major.softmax_router(u, Wr, k)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(g, rw, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- P-5 library reductions

def _torch_swiglu(x, W1, W3, W2):
    x, W1, W3, W2 = (torch.from_numpy(oracle.widen(a)) for a in (x, W1, W3, W2))
    return ((torch.nn.functional.silu(x @ W1.T) * (x @ W3.T)) @ W2.T).numpy()


def _rand_layer(rng, T, d, E, F, Fs=0, dtype=np.float64):
    u = rng.standard_normal((T, d)).astype(dtype)
    Wr = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(dtype)
    W1 = (rng.standard_normal((E, F, d)) / math.sqrt(d)).astype(dtype)
    W3 = (rng.standard_normal((E, F, d)) / math.sqrt(d)).astype(dtype)
    W2 = (rng.standard_normal((E, d, F)) / math.sqrt(F)).astype(dtype)
    shared = None
    if Fs:
        shared = ((rng.standard_normal((Fs, d)) / math.sqrt(d)).astype(dtype),
                  (rng.standard_normal((Fs, d)) / math.sqrt(d)).astype(dtype),
                  (rng.standard_normal((d, Fs)) / math.sqrt(Fs)).astype(dtype))
    return u, Wr, W1, W3, W2, shared


def test_single_expert_is_dense_swiglu():
    rng = np.random.default_rng(4)
    u, Wr, W1, W3, W2, _ = _rand_layer(rng, 40, 32, 1, 48)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, W3, W2, 1)
    assert (idx == 0).all() and (g == 1.0).all()
    np.testing.assert_allclose(y, _torch_swiglu(u, W1[0], W3[0], W2[0]), rtol=1e-12, atol=1e-13)


def test_k_equals_E_is_softmax_weighted_dense_sum():
    rng = np.random.default_rng(5)
    T, d, E, F = 30, 16, 4, 24
    u, Wr, W1, W3, W2, _ = _rand_layer(rng, T, d, E, F)
    y, _, _, _, _ = oracle.forward(u, Wr, W1, W3, W2, E)
    p = torch.softmax(torch.from_numpy(u @ Wr.T), dim=1).numpy()
    ref = sum(p[:, e:e + 1] * _torch_swiglu(u, W1[e], W3[e], W2[e]) for e in range(E))
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


def test_zero_routed_down_projection_leaves_the_shared_expert():
    rng = np.random.default_rng(6)
    u, Wr, W1, W3, W2, shared = _rand_layer(rng, 25, 16, 8, 20, Fs=12)
    y, _, _, _, _ = oracle.forward(u, Wr, W1, W3, np.zeros_like(W2), 3, shared=shared,
                                   score_fn=oracle.SIGMOID, n_groups=4, topk_groups=2,
                                   route_scale=2.5)
    np.testing.assert_allclose(y, _torch_swiglu(u, *shared), rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P-6 identical experts

@pytest.mark.parametrize("mode,G,M,scale,k", [(oracle.SOFTMAX, 1, 1, 1.0, 2),
                                              (oracle.SIGMOID, 8, 4, 2.5, 8)])
def test_identical_experts_every_token_gets_k_outputs_and_the_shared_one(mode, G, M, scale, k):
    rng = np.random.default_rng(7)
    T, d, E, F, Fs = 64, 16, 32, 20, 12
    u, Wr, W1, W3, W2, shared = _rand_layer(rng, T, d, E, F, Fs)
    Wr[0] *= 8.0  # skew: many tokens pick expert 0
    W1[:] = W1[0]
    W3[:] = W3[0]
    W2[:] = W2[0]
    bias = rng.uniform(-0.05, 0.05, E)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, W3, W2, k, bias=bias, shared=shared,
                                     score_fn=mode, n_groups=G, topk_groups=M, route_scale=scale)
    ref = scale * _torch_swiglu(u, W1[0], W3[0], W2[0]) + _torch_swiglu(u, *shared)
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-12)
    assert all(len(set(r)) == k for r in idx.tolist())


# ---------------------------------------------------------------- P-7 second implementation

def test_token_major_matches_expert_major_softmax():
    rng = np.random.default_rng(8)
    u, Wr, W1, W3, W2, shared = _rand_layer(rng, 80, 32, 8, 40, Fs=24)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, W3, W2, 2, shared=shared)
    ref, ridx, rg = expert_major.layer(u, Wr, W1, W3, W2, 2, shared=shared)
    assert np.array_equal(idx, ridx)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_token_major_matches_expert_major_sigmoid_grouped_bf16_bits():
    rng = np.random.default_rng(9)
    arrs = _rand_layer(rng, 64, 32, 16, 24, Fs=16, dtype=np.float32)
    # bf16 bit patterns (truncated fp32): the oracle widens them exactly
    to_bf16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    u, Wr, W1, W3, W2 = (to_bf16(a) for a in arrs[:5])
    shared = tuple(to_bf16(a) for a in arrs[5])
    bias = rng.uniform(-0.05, 0.05, 16)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, W3, W2, 4, bias=bias, shared=shared,
                                     score_fn=oracle.SIGMOID, n_groups=4, topk_groups=2,
                                     route_scale=2.5)
    ref, _, _ = expert_major.layer(u, Wr, W1, W3, W2, 4, shared=shared, idx=idx, gates=g)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)
    # selection also checked from the widened values through an independent route
    lg = oracle.widen(u) @ oracle.widen(Wr).T
    s = 1 / (1 + np.exp(-lg)) + bias
    for t in range(len(idx)):
        assert set(idx[t].tolist()) == _brute_force_select(s[t].tolist(), 4, 4, 2)


def test_token_subset_and_forced_selection():
    rng = np.random.default_rng(10)
    u, Wr, W1, W3, W2, shared = _rand_layer(rng, 50, 16, 8, 16, Fs=8)
    full = oracle.forward(u, Wr, W1, W3, W2, 2, shared=shared)
    tok = np.array([49, 0, 17, 17])
    sub = oracle.forward(u, Wr, W1, W3, W2, 2, shared=shared, tokens=tok)
    np.testing.assert_array_equal(sub[0], full[0][tok])
    forced = oracle.forward(u, Wr, W1, W3, W2, 2, shared=shared, tokens=tok,
                            forced_idx=full[1][tok])
    np.testing.assert_array_equal(forced[0], full[0][tok])
    np.testing.assert_array_equal(forced[2], full[2][tok])


# ---------------------------------------------------------------- expert bodies

# Standard normal CDF at 1 and 2 from printed tables: GELU(x) = x Phi(x).
_PHI_1 = 0.8413447460685429
_PHI_2 = 0.9772498680518208


def test_gelu_mlp_closed_form_with_per_expert_biases():
    """Diagonal W1, identity W2, one forced expert per token: the layer is
    GELU(a_e x + b1_e) + b2_e elementwise, with the gate of a single chosen
    expert equal to 1 (softmax over the k chosen)."""
    from scipy.stats import norm
    E, d = 4, 6
    a = np.array([[1.0, 0.5, -1.0, 2.0, 0.0, 1.5],
                  [2.0, 1.0, 1.0, -0.5, 3.0, 0.25],
                  [-2.0, 1.0, 0.75, 1.0, -1.0, 1.0],
                  [1.0, 1.0, 1.0, 1.0, 1.0, 1.0]])
    b1 = np.arange(E * d, dtype=np.float64).reshape(E, d) * 0.05 - 0.4
    b2 = np.arange(E * d, dtype=np.float64).reshape(E, d)[:, ::-1] * 0.1 - 1.0
    W1 = np.stack([np.diag(r) for r in a])
    W2 = np.stack([np.eye(d)] * E)
    u = np.array([[1.0, -1.0, 0.5, 2.0, -0.3, 0.0],
                  [0.2, 0.4, -2.0, 1.0, 1.0, -1.5],
                  [1.0, 1.0, 1.0, 1.0, 1.0, 1.0],
                  [-0.7, 2.2, 0.1, -1.1, 0.9, 0.3],
                  [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]])
    Wr = np.zeros((E, d))
    forced = np.array([[2], [0], [3], [1], [2]], dtype=np.int32)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, None, W2, 1, kind=oracle.GELU_MLP, b1=b1,
                                     b2=b2, forced_idx=forced)
    assert (g == 1.0).all()
    e = forced[:, 0]
    z = a[e] * u + b1[e]
    np.testing.assert_allclose(y, z * norm.cdf(z) + b2[e], rtol=1e-14, atol=1e-15)
    # row 2 (expert 3: a = 1): the pre-activation is 1 + b1[3]; check the
    # printed table values where the argument lands on 1 or 2 exactly
    u1 = np.array([[1.0 - b1[3, 0], 2.0 - b1[3, 1], -1.0 - b1[3, 2], 0.0, 0.0, 0.0]])
    y1, _, _, _, _ = oracle.forward(u1, Wr, W1, None, W2, 1, kind=oracle.GELU_MLP, b1=b1,
                                    b2=np.zeros_like(b2), forced_idx=np.array([[3]], np.int32))
    np.testing.assert_allclose(y1[0, :3], [_PHI_1, 2 * _PHI_2, -(1 - _PHI_1)], rtol=1e-14)


def test_geglu_closed_form():
    from scipy.stats import norm
    E, d = 3, 5
    rng = np.random.default_rng(21)
    a = rng.uniform(-2, 2, (E, d))
    c = rng.uniform(-2, 2, (E, d))
    W1 = np.stack([np.diag(r) for r in a])
    W3 = np.stack([np.diag(r) for r in c])
    W2 = np.stack([np.eye(d)] * E)
    u = rng.standard_normal((7, d))
    forced = (np.arange(7, dtype=np.int32) % E)[:, None]
    y, _, g, _, _ = oracle.forward(u, np.zeros((E, d)), W1, W3, W2, 1, kind=oracle.GEGLU,
                                   forced_idx=forced)
    e = forced[:, 0]
    z = a[e] * u
    np.testing.assert_allclose(y, z * norm.cdf(z) * (c[e] * u), rtol=1e-13, atol=1e-15)


def _torch_gelu_mlp(x, W1, W2, b1, b2):
    x, W1, W2, b1, b2 = (torch.from_numpy(oracle.widen(t)) for t in (x, W1, W2, b1, b2))
    return (torch.nn.functional.gelu(x @ W1.T + b1) @ W2.T + b2).numpy()


def test_gelu_mlp_k_equals_E_weights_the_output_bias_by_the_gate():
    """k = E: y = sum_e p_e (W2_e GELU(W1_e x + b1_e) + b2_e), p the softmax of
    the logits (PyTorch's exact GELU)."""
    rng = np.random.default_rng(22)
    T, d, E, F = 20, 12, 4, 16
    u, Wr, W1, _, W2, _ = _rand_layer(rng, T, d, E, F)
    b1 = rng.standard_normal((E, F)) * 0.3
    b2 = rng.standard_normal((E, d)) * 0.3
    y, _, _, _, _ = oracle.forward(u, Wr, W1, None, W2, E, kind=oracle.GELU_MLP, b1=b1, b2=b2)
    p = torch.softmax(torch.from_numpy(u @ Wr.T), dim=1).numpy()
    ref = sum(p[:, e:e + 1] * _torch_gelu_mlp(u, W1[e], W2[e], b1[e], b2[e]) for e in range(E))
    np.testing.assert_allclose(y, ref, rtol=1e-11, atol=1e-13)


def test_gelu_mlp_shared_expert_with_biases_is_added_unweighted():
    rng = np.random.default_rng(23)
    T, d, E, F, Fs = 24, 16, 8, 12, 20
    u, Wr, W1, _, W2, _ = _rand_layer(rng, T, d, E, F)
    W1s = rng.standard_normal((Fs, d)) / 4
    W2s = rng.standard_normal((d, Fs)) / 4
    b1s = rng.standard_normal(Fs) * 0.2
    b2s = rng.standard_normal(d) * 0.2
    y, _, _, _, _ = oracle.forward(u, Wr, W1, None, np.zeros_like(W2), 3, kind=oracle.GELU_MLP,
                                   shared=(W1s, None, W2s, b1s, b2s), score_fn=oracle.SIGMOID,
                                   n_groups=4, topk_groups=2, route_scale=2.5)
    np.testing.assert_allclose(y, _torch_gelu_mlp(u, W1s, W2s, b1s, b2s), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kind", [oracle.GEGLU, oracle.GELU_MLP])
def test_token_major_matches_expert_major_other_bodies(kind):
    rng = np.random.default_rng(24 + kind)
    arrs = _rand_layer(rng, 64, 32, 16, 24, Fs=16, dtype=np.float32)
    to_bf16 = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)
    u, Wr, W1, W3, W2 = (to_bf16(a) for a in arrs[:5])
    W1s, W3s, W2s = (to_bf16(a) for a in arrs[5])
    b1 = b2 = b1s = b2s = None
    if kind == oracle.GELU_MLP:
        W3 = W3s = None
        b1 = to_bf16(rng.standard_normal((16, 24)).astype(np.float32) * 0.2)
        b2 = to_bf16(rng.standard_normal((16, 32)).astype(np.float32) * 0.2)
        b1s = to_bf16(rng.standard_normal(16).astype(np.float32) * 0.2)
        b2s = to_bf16(rng.standard_normal(32).astype(np.float32) * 0.2)
    shared = (W1s, W3s, W2s, b1s, b2s)
    bias = rng.uniform(-0.05, 0.05, 16)
    y, idx, g, _, _ = oracle.forward(u, Wr, W1, W3, W2, 4, bias=bias, shared=shared,
                                     score_fn=oracle.SIGMOID, n_groups=4, topk_groups=2,
                                     route_scale=2.5, kind=kind, b1=b1, b2=b2)
    ref, _, _ = expert_major.layer(u, Wr, W1, W3, W2, 4, shared=shared, idx=idx, gates=g,
                                   kind=kind, b1=b1, b2=b2)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-13)


def test_expert_kind_argument_checks():
    rng = np.random.default_rng(25)
    u, Wr, W1, W3, W2, _ = _rand_layer(rng, 4, 8, 2, 8)
    with pytest.raises(ValueError):
        oracle.forward(u, Wr, W1, W3, W2, 1, kind=7)
    with pytest.raises(ValueError):
        oracle.forward(u, Wr, W1, W3, W2, 1, b1=np.zeros((2, 8)))


# ---------------------------------------------------------------- permutation

def test_permutation_is_the_stable_expert_order():
    rng = np.random.default_rng(11)
    E = 13
    idx = rng.integers(0, E, size=(300, 4)).astype(np.int32)
    idx[:, 0] = 3  # a heavy expert; experts 11, 12 may be empty
    idx[idx == 12] = 11
    counts, offsets, perm, inv = oracle.permutation(idx, E)
    flat = idx.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(inv[perm], np.arange(flat.size))
    assert counts[12] == 0


# ---------------------------------------------------------------- P-8 balance loop

def test_balance_loop_raises_entropy_toward_ln_E():
    rng = np.random.default_rng(12)
    T, d, E, k = 4096, 32, 16, 2
    m = rng.standard_normal(d)
    m /= np.linalg.norm(m)
    u = rng.standard_normal((T, d)) + 2.0 * m
    Wr = rng.standard_normal((E, d)) / math.sqrt(d)
    Wr[0] = 2.0 * m
    lg = oracle.router_logits(u, Wr)
    b, hist = balance.balance_bias(lg, k)
    before, after = hist[0]["entropy"], hist[-1]["entropy"]
    assert hist[0]["counts"][0] > 0.6 * T  # skewed before balancing
    assert after > before
    assert after <= balance.max_entropy(E) + 1e-12
    assert hist[-1]["counts"][0] < hist[0]["counts"][0]
    # one update step: over target goes down by gamma, under goes up
    c = hist[0]["counts"]
    target = T * k / E
    step = balance.update_bias(np.zeros(E), c, target)
    assert np.all(step[c > target] == -0.15) and np.all(step[c < target] == 0.15)
    # the bias never moved a gate: gates at the final bias come from raw logits
    idx, g, _, _ = oracle.select(lg, k, oracle.SOFTMAX, bias=b)
    chosen = np.take_along_axis(lg, idx.astype(np.int64), 1)
    z = np.exp(chosen - chosen.max(1, keepdims=True))
    np.testing.assert_allclose(g, z / z.sum(1, keepdims=True), rtol=1e-13)


def test_invalid_configurations_are_rejected():
    lg = np.zeros((2, 8))
    for k, G, M in ((9, 1, 1), (2, 3, 1), (2, 8, 4), (5, 4, 2)):
        with pytest.raises(ValueError):
            oracle.select(lg, k, oracle.SIGMOID, G, M)


def test_balance_step_hand_worked():
    """One step of the balance update ("Mixture of Experts and Hybrid
    Architectures", "Aux-loss-free balance loop") on a routing small enough to
    follow by hand: 3 tokens, k = 2, E = 4, picks (0,1), (0,2), (0,1).
    counts = [3, 2, 1, 0], S = 6, target = 6/4 = 1.5: experts 0 and 1 are over
    (bias - gamma), 2 and 3 under (+ gamma); p = [1/2, 1/3, 1/6, 0], entropy =
    (1/2) ln 2 + (1/3) ln 3 + (1/6) ln 6."""
    g = np.float32(0.15)
    b, c, h = balance.update_step_fp32(np.array([[0, 1], [0, 2], [0, 1]]), 4,
                                       np.array([0.5, 0, 0, -1], np.float32), g)
    assert c.tolist() == [3, 2, 1, 0]
    assert b.tolist() == [np.float32(0.5) - g, -g, g, np.float32(-1) + g]
    assert h == pytest.approx(0.5 * math.log(2) + math.log(3) / 3 + math.log(6) / 6, rel=1e-15)
    # on target exactly: E = 2, one token picking both -> counts [1, 1] = target 1, bias kept
    b, c, h = balance.update_step_fp32(np.array([[1, 0]]), 2, np.array([0.25, -0.5], np.float32), g)
    assert b.tolist() == [0.25, -0.5] and c.tolist() == [1, 1] and h == pytest.approx(math.log(2))
    # entries outside [0, E) are not counted but stay in S; no tokens: nothing moves
    b, c, h = balance.update_step_fp32(np.array([[0, 7], [-1, 0]]), 2, np.zeros(2, np.float32), g)
    assert c.tolist() == [2, 0] and b.tolist() == [0.0, g]  # S = 4, target 2: expert 0 on target
    assert h == pytest.approx(-0.5 * math.log(0.5))
    b, c, h = balance.update_step_fp32(np.zeros((0, 2), np.int32), 3, np.ones(3, np.float32), g)
    assert b.tolist() == [1, 1, 1] and c.tolist() == [0, 0, 0] and h == 0.0
    # the fp32 step equals the fp64 loop's update rounded once
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 16, size=(500, 4))
    b0 = (rng.integers(-10, 10, 16) * 0.15).astype(np.float32)
    b, c, _ = balance.update_step_fp32(idx, 16, b0, g)
    ref = balance.update_bias(b0.astype(np.float64), balance.usage(idx, 16), 500 * 4 / 16, float(g))
    assert np.array_equal(b, ref.astype(np.float32))


def test_rmsnorm_closed_forms():
    """RMSNorm ("Mixture of experts and architecture families": normalisation
    without mean-centering; the pre-norm block of "Lesson 2 -- From the Dense
    FFN to a Layer of Experts", section 2): x / sqrt(mean x^2 + eps) * g."""
    from oracle import block
    rng = np.random.default_rng(9)
    g = rng.standard_normal(48)
    # a constant row c normalises to sign(c) * g (eps = 0)
    for c in (3.0, -0.25):
        np.testing.assert_allclose(block.rmsnorm(np.full((1, 48), c), g, 0.0)[0], np.sign(c) * g, rtol=1e-15)
    x = rng.standard_normal((5, 48))
    # scale invariance at eps = 0, and unit mean square with g = 1
    np.testing.assert_allclose(block.rmsnorm(7.5 * x, g, 0.0), block.rmsnorm(x, g, 0.0), rtol=1e-14)
    n = block.rmsnorm(x, np.ones(48), 0.0)
    np.testing.assert_allclose((n * n).mean(axis=1), 1.0, rtol=1e-14)
    # eps keeps a zero row at zero; eps shrinks small rows: mean square = m / (m + eps)
    assert np.array_equal(block.rmsnorm(np.zeros((1, 48)), g, 1e-6), np.zeros((1, 48)))
    m = (x[0] ** 2).mean()
    np.testing.assert_allclose((block.rmsnorm(x[:1], np.ones(48), 0.5) ** 2).mean(), m / (m + 0.5), rtol=1e-14)


def test_block_residual_passes_through_when_the_experts_output_zero():
    """y = h + MoE(RMSNorm(h)): with every down projection zero (routed and
    shared) the block returns its input exactly."""
    from oracle import block
    rng = np.random.default_rng(10)
    T, d, E, F = 12, 32, 4, 16
    h = rng.standard_normal((T, d))
    Wr = rng.standard_normal((E, d))
    W1, W3 = rng.standard_normal((E, F, d)), rng.standard_normal((E, F, d))
    shared = (rng.standard_normal((F, d)), rng.standard_normal((F, d)), np.zeros((d, F)))
    y, idx, g, _, _ = block.block_forward(h, np.ones(d), 1e-6, Wr, W1, W3, np.zeros((E, d, F)), 2,
                                          shared=shared)
    assert np.array_equal(y, h)
    # and the layer part is the layer on the normalised rows
    W2 = rng.standard_normal((E, d, F))
    y, idx, g, _, _ = block.block_forward(h, np.ones(d), 1e-6, Wr, W1, W3, W2, 2)
    y0, idx0, g0, _, _ = oracle.forward(block.rmsnorm(h, np.ones(d), 1e-6), Wr, W1, W3, W2, 2)
    assert np.array_equal(idx, idx0) and np.array_equal(y, y0 + h)


def _bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def test_bf16_rounding_is_torchs_nearest_even():
    """The fused block's fold of the norm weight into the router rows rounds
    products of two bf16 values to bf16, nearest even: checked against
    PyTorch's bf16 conversion on products, exact halfway cases and signs."""
    from oracle import block
    rng = np.random.default_rng(31)
    a = oracle.widen(_bf16_bits(rng.standard_normal(4000)))
    b = oracle.widen(_bf16_bits(1 + 0.1 * rng.standard_normal(4000)))
    p = a * b  # exact in fp64 and in fp32
    want = torch.from_numpy(p.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(block.bf16_round(p), want)
    ties = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2.0 ** -130 * 3])
    assert np.array_equal(block.bf16_round(ties),
                          torch.from_numpy(ties.astype(np.float32)).to(torch.bfloat16).double().numpy())
    assert block.bf16_round(np.array([1.0 + 2 ** -8]))[0] == 1.0          # tie to the even neighbour
    assert block.bf16_round(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6


def _fused_inputs(rng, T=40, d=64, E=16, F=32, Fs=32):
    h = _bf16_bits(rng.standard_normal((T, d)) * np.exp(rng.standard_normal((T, 1))))
    Wr = _bf16_bits(rng.standard_normal((E, d)) / math.sqrt(d))
    W1 = _bf16_bits(rng.standard_normal((E, F, d)) / math.sqrt(d))
    W3 = _bf16_bits(rng.standard_normal((E, F, d)) / math.sqrt(d))
    W2 = _bf16_bits(rng.standard_normal((E, d, F)) / math.sqrt(F))
    shared = (_bf16_bits(rng.standard_normal((Fs, d)) / math.sqrt(d)),
              _bf16_bits(rng.standard_normal((Fs, d)) / math.sqrt(d)),
              _bf16_bits(rng.standard_normal((d, Fs)) / math.sqrt(Fs)))
    return h, Wr, W1, W3, W2, shared


DSV3_SMALL = dict(score_fn=oracle.SIGMOID, n_groups=4, topk_groups=2, route_scale=2.5)


def test_expert_sum_is_the_layers_weighted_sum():
    """The fused block's output composition, shared + sum_j g_j FFN_j, equals
    the layer oracle's output for the layer's own selection and gates."""
    from oracle import block
    rng = np.random.default_rng(32)
    h, Wr, W1, W3, W2, shared = _fused_inputs(rng)
    bias = rng.uniform(-0.05, 0.05, 16)
    y, idx, g, _, _ = oracle.forward(h, Wr, W1, W3, W2, 4, bias=bias, shared=shared, **DSV3_SMALL)
    ys = block.expert_sum(h, W1, W3, W2, idx, g, shared)
    np.testing.assert_allclose(ys, y, rtol=1e-12, atol=1e-13)
    lg = oracle.router_logits(h, Wr)
    np.testing.assert_allclose(block.gates_of(lg, idx, oracle.SIGMOID, 2.5), g, rtol=1e-14)
    ys2, idx2, g2, _, _ = oracle.forward(h, Wr, W1, W3, W2, 3)
    np.testing.assert_allclose(block.gates_of(oracle.router_logits(h, Wr), idx2, oracle.SOFTMAX, 1.0), g2,
                               rtol=1e-14)


def test_fused_block_with_unit_norm_weight_is_the_block():
    """g = 1: folding changes nothing (the router rows are already bf16), so
    the fused block routes as the block on its exact fp64 normalised rows and
    returns the same output."""
    from oracle import block
    rng = np.random.default_rng(33)
    h, Wr, W1, W3, W2, shared = _fused_inputs(rng)
    g = _bf16_bits(np.ones(h.shape[1]))
    bias = rng.uniform(-0.05, 0.05, 16)
    kw = dict(bias=bias, shared=shared, **DSV3_SMALL)
    y, idx, gt, ge, gg = block.fused_block_forward(h, g, 1e-6, Wr, W1, W3, W2, 4, **kw)
    y0, idx0, g0, ge0, gg0 = block.block_forward(h, g, 1e-6, Wr, W1, W3, W2, 4, **kw)
    assert np.array_equal(idx, idx0)
    np.testing.assert_allclose(gt, g0, rtol=1e-13)
    np.testing.assert_allclose(y, y0, rtol=1e-12, atol=1e-12)


def test_fused_block_with_a_power_of_two_norm_weight_routes_as_the_block():
    """g = 2 everywhere: W_router * g is exact in bf16, so the fused routing
    equals the block's on RMSNorm(h) = 2 h / rms, and so does the output."""
    from oracle import block
    rng = np.random.default_rng(34)
    h, Wr, W1, W3, W2, shared = _fused_inputs(rng)
    g = _bf16_bits(np.full(h.shape[1], 2.0))
    kw = dict(shared=shared, score_fn=oracle.SOFTMAX)
    y, idx, gt, _, _ = block.fused_block_forward(h, g, 1e-6, Wr, W1, W3, W2, 3, **kw)
    y0, idx0, g0, _, _ = block.block_forward(h, g, 1e-6, Wr, W1, W3, W2, 3, **kw)
    assert np.array_equal(idx, idx0)
    np.testing.assert_allclose(gt, g0, rtol=1e-12)
    np.testing.assert_allclose(y, y0, rtol=1e-12, atol=1e-12)


def test_fused_block_is_invariant_to_the_scale_of_its_input():
    """RMSNorm(c h) = RMSNorm(h) (eps = 0): with c a power of two, routing is
    unchanged and the output moves by exactly the residual's change."""
    from oracle import block
    rng = np.random.default_rng(35)
    h, Wr, W1, W3, W2, shared = _fused_inputs(rng)
    g = _bf16_bits(1 + 0.1 * rng.standard_normal(h.shape[1]))
    kw = dict(shared=shared, **DSV3_SMALL)
    y, idx, gt, _, _ = block.fused_block_forward(h, g, 0.0, Wr, W1, W3, W2, 4, **kw)
    h4 = _bf16_bits(4.0 * oracle.widen(h))
    y4, idx4, g4, _, _ = block.fused_block_forward(h4, g, 0.0, Wr, W1, W3, W2, 4, **kw)
    assert np.array_equal(idx, idx4)
    np.testing.assert_allclose(g4, gt, rtol=1e-13)
    np.testing.assert_allclose(y4 - oracle.widen(h4), y - oracle.widen(h), rtol=1e-11, atol=1e-12)


def test_fused_routing_decides_on_the_bf16_folded_router():
    """The fused routing's logits are rs * (h . bf16(W_router * g)): against a
    brute-force sum over the folded rows in exact rational arithmetic for a
    few tokens."""
    from oracle import block
    rng = np.random.default_rng(36)
    h, Wr, _, _, _, _ = _fused_inputs(rng, T=3, d=16, E=4)
    g = _bf16_bits(1 + 0.1 * rng.standard_normal(16))
    _, _, _, _, lg = block.fused_route(h, g, 1e-6, Wr, 2)
    hw, Ww, gw = oracle.widen(h), oracle.widen(Wr), oracle.widen(g)
    Wg = block.bf16_round(Ww * gw)
    for t in range(3):
        rs = 1.0 / math.sqrt(float(np.mean(hw[t] ** 2)) + 1e-6)
        for e in range(4):
            dot = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(hw[t], Wg[e]))
            assert lg[t, e] == pytest.approx(rs * float(dot), rel=1e-13, abs=1e-15)
