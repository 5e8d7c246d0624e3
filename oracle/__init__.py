"""CPU oracle for the forward pass of one sparse MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; the product path never imports it,
and it imports nothing from the product package.

Three parts, all fp64:

* ``moe_oracle.c`` (wrapped here through ctypes): the token-major layer as the
  pages define it -- router logits, scores, selection-only bias, group limit,
  stable top-k, gates from raw scores, experts (SwiGLU, GEGLU, or the GELU
  MLP with biases), unweighted shared expert, gate-weighted sum -- plus the
  expert-contiguous permutation.
* ``expert_major.py``: an independent second implementation, expert-major in
  the dispatch / combine form (flattened (token, slot) pairs grouped by
  expert, one batched product per expert, scatter-add of the weighted rows),
  with the softmax router of "Mixture of experts and architecture families",
  "The router and load balancing" (NumPy float64).
* ``balance.py``: the auxiliary-loss-free bias loop and the routing entropy of
  "Mixture of Experts and Hybrid Architectures", "Aux-loss-free balance loop".

Arrays are NumPy.  Floating inputs may be float64, float32 or uint16 holding
bfloat16 bit patterns (read exactly, widened to fp64).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")

SOFTMAX = 0
SIGMOID = 1

SWIGLU = 0
GEGLU = 1
GELU_MLP = 2

_F32, _BF16, _F64 = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (plain -O2, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_router_logits.argtypes = [I64, P, I, I, P, I, P, I, P, I]
        lib.oracle_router_logits.restype = I
        lib.oracle_select.argtypes = [I64, I, I, I, I, I, D, P, P, P, P, P, P, I]
        lib.oracle_select.restype = I
        lib.oracle_forward.argtypes = [I64, P, I, I, I, I, I, I, I, I, D,
                                       P, I, P, P, P, P, P, P, P, P, I,
                                       P, P, P, P, P, P, I]
        lib.oracle_forward.restype = I
        lib.oracle_forward_ex.argtypes = [I64, P, I, I, I, I, I, I, I, I, D,
                                          P, I, P, P, I, P, P, P, P, P, P, P, P, P, P, I,
                                          P, P, P, P, P, P, I]
        lib.oracle_forward_ex.restype = I
        lib.oracle_permutation.argtypes = [I64, I, P, P, P, P, P]
        lib.oracle_permutation.restype = I
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return _F64
    if a.dtype == np.float32:
        return _F32
    if a.dtype == np.uint16:
        return _BF16
    raise TypeError(f"oracle input dtype {a.dtype} (want float64, float32 or uint16 bf16 bits)")


def _c(a):
    return None if a is None else np.ascontiguousarray(a)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 copy of a float32/float64 array or of uint16 bf16 bits."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _check_weights(*arrs):
    codes = {_code(a) for a in arrs if a is not None}
    if len(codes) != 1:
        raise TypeError("router, expert and shared weights must share one dtype")
    return codes.pop()


def router_logits(u, W_router, tokens=None, nthreads=None):
    """l[i][e] = u[tokens[i]] . W_router[e] in fp64 (tokens None: all rows)."""
    u, Wr = _c(u), _c(W_router)
    T, d = u.shape
    E = Wr.shape[0]
    assert Wr.shape[1] == d
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = T if tok is None else tok.shape[0]
    out = np.empty((n, E), dtype=np.float64)
    rc = _load().oracle_router_logits(n, _p(tok), d, E, _p(u), _code(u), _p(Wr),
                                      _code(Wr), _p(out), nthreads or default_threads())
    if rc:
        raise ValueError("oracle_router_logits: invalid arguments")
    return out


def select(logits, k, score_fn=SOFTMAX, n_groups=1, topk_groups=1, route_scale=1.0,
           bias=None, nthreads=None):
    """Scores, biased (group-limited) stable top-k and gates from logits [n][E].

    Returns (idx int32 [n][k], gates [n][k], gap_expert [n], gap_group [n]).
    gap_* is the relative gap |a-b|/max(|a|,|b|,1) between the last chosen and
    the first rejected biased expert score (group score); inf when none."""
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    n, E = logits.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    idx = np.empty((n, k), dtype=np.int32)
    gates = np.empty((n, k), dtype=np.float64)
    ge = np.empty(n, dtype=np.float64)
    gg = np.empty(n, dtype=np.float64)
    rc = _load().oracle_select(n, E, k, score_fn, n_groups, topk_groups, float(route_scale),
                               _p(b), _p(logits), _p(idx), _p(gates), _p(ge), _p(gg),
                               nthreads or default_threads())
    if rc:
        raise ValueError("oracle_select: invalid configuration")
    return idx, gates, ge, gg


def route(u, W_router, k, score_fn=SOFTMAX, n_groups=1, topk_groups=1, route_scale=1.0,
          bias=None, tokens=None, nthreads=None):
    """Router logits then selection: (idx, gates, gap_expert, gap_group, logits)."""
    lg = router_logits(u, W_router, tokens=tokens, nthreads=nthreads)
    idx, gates, ge, gg = select(lg, k, score_fn, n_groups, topk_groups, route_scale, bias,
                                nthreads=nthreads)
    return idx, gates, ge, gg, lg


def forward(u, W_router, W1, W3, W2, k, *, bias=None, shared=None, score_fn=SOFTMAX,
            n_groups=1, topk_groups=1, route_scale=1.0, tokens=None, forced_idx=None,
            kind=SWIGLU, b1=None, b2=None, nthreads=None):
    """Whole-layer output for the listed tokens (None: all).

    kind: SWIGLU (W2 (SiLU(W1 x) * W3 x)), GEGLU (GELU in place of SiLU) or
    GELU_MLP (W2 GELU(W1 x + b1) + b2; W3 is None, b1 [E][F] / b2 [E][d] or
    None for zero).
    shared is None or (W1s [Fs][d], W3s [Fs][d] or None, W2s [d][Fs]
    [, b1s [Fs], b2s [d]]).
    forced_idx [n][k] replaces selection (gates still come from raw scores).
    Returns (y fp64 [n][d], idx [n][k], gates [n][k], gap_expert [n], gap_group [n])."""
    if kind not in (SWIGLU, GEGLU, GELU_MLP):
        raise ValueError(f"unknown expert kind {kind}")
    gated = kind != GELU_MLP
    u, Wr, W1, W3, W2 = _c(u), _c(W_router), _c(W1), _c(W3), _c(W2)
    T, d = u.shape
    E, F, d1 = W1.shape
    assert d1 == d and W2.shape == (E, d, F) and Wr.shape == (E, d)
    assert (W3 is not None and W3.shape == W1.shape) if gated else W3 is None
    if not gated:
        b1, b2 = _c(b1), _c(b2)
        assert b1 is None or b1.shape == (E, F)
        assert b2 is None or b2.shape == (E, d)
    elif b1 is not None or b2 is not None:
        raise ValueError("biases belong to the GELU MLP expert only")
    b1s = b2s = None
    if shared is not None:
        sh = tuple(_c(a) for a in shared)
        W1s, W3s, W2s = sh[:3]
        if len(sh) == 5:
            b1s, b2s = sh[3:]
            if gated and (b1s is not None or b2s is not None):
                raise ValueError("biases belong to the GELU MLP expert only")
        Fs = W1s.shape[0]
        assert W1s.shape == (Fs, d) and W2s.shape == (d, Fs)
        assert (W3s is not None and W3s.shape == (Fs, d)) if gated else W3s is None
        assert b1s is None or b1s.shape == (Fs,)
        assert b2s is None or b2s.shape == (d,)
    else:
        W1s = W3s = W2s = None
        Fs = 0
    wcode = _check_weights(Wr, W1, W3, W2, W1s, W3s, W2s, b1, b2, b1s, b2s)
    tok = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
    n = T if tok is None else tok.shape[0]
    if tok is not None and n and (tok.min() < 0 or tok.max() >= T):
        raise ValueError("token index out of range")
    fi = None if forced_idx is None else np.ascontiguousarray(forced_idx, dtype=np.int32)
    if fi is not None:
        assert fi.shape == (n, k)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float64)
    y = np.empty((n, d), dtype=np.float64)
    idx = np.empty((n, k), dtype=np.int32)
    gates = np.empty((n, k), dtype=np.float64)
    ge = np.empty(n, dtype=np.float64)
    gg = np.empty(n, dtype=np.float64)
    rc = _load().oracle_forward_ex(n, _p(tok), d, E, k, F, Fs, score_fn, n_groups, topk_groups,
                                   float(route_scale), _p(u), _code(u), _p(Wr), _p(b), kind,
                                   _p(W1), _p(W3), _p(W2), _p(b1), _p(b2), _p(W1s), _p(W3s),
                                   _p(W2s), _p(b1s), _p(b2s), wcode, _p(fi), _p(y), _p(idx),
                                   _p(gates), _p(ge), _p(gg), nthreads or default_threads())
    if rc:
        raise ValueError("oracle_forward: invalid arguments")
    return y, idx, gates, ge, gg


def permutation(idx, E):
    """Expert-contiguous stable order of the T*k slots of idx [T][k].

    Returns (counts [E], offsets [E+1], perm [T*k], inv [T*k]), int32."""
    flat = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(-1))
    n = flat.shape[0]
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(n, dtype=np.int32)
    inv = np.empty(n, dtype=np.int32)
    rc = _load().oracle_permutation(n, E, _p(flat), _p(counts), _p(offsets), _p(perm), _p(inv))
    if rc:
        raise ValueError("oracle_permutation: expert index out of range")
    return counts, offsets, perm, inv
