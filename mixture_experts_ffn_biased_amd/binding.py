"""ctypes binding of libmoe (include/moe.h), with the same entry-point names.

Argument marshalling only: checks that tensors have the shapes, dtypes and
device the ABI expects, allocates outputs and workspace with torch, and passes
raw device pointers plus torch's current HIP stream.  Every step of the layer
runs in the library's HIP kernels; if ``libmoe.so`` is missing this module
raises instead of computing anything another way.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_EXPERT_SWIGLU, MOE_EXPERT_GEGLU, MOE_EXPERT_GELU_MLP = 0, 1, 2
EXPERT_KINDS = {"swiglu": MOE_EXPERT_SWIGLU, "geglu": MOE_EXPERT_GEGLU, "gelu_mlp": MOE_EXPERT_GELU_MLP}
MOE_N_STAGES = 5
STAGES = ("router_topk", "permute", "gate_up", "down", "combine")

STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_CFG",
          -4: "MOE_ERR_DTYPE", -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP", -7: "MOE_ERR_ALIGN"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({moe_status_str(status)})")


class moe_cfg(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("F", ctypes.c_int32), ("F_shared", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("score_fn", ctypes.c_int32),
                ("n_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32),
                ("route_scale", ctypes.c_float)]


class moe_shared(ctypes.Structure):
    _fields_ = [("W1", ctypes.c_void_p), ("W3", ctypes.c_void_p), ("W2", ctypes.c_void_p)]


class moe_experts(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32)] + [
        (n, ctypes.c_void_p) for n in ("W1", "W3", "W2", "b1", "b2", "W1s", "W3s", "W2s", "b1s", "b2s")]


@dataclass(frozen=True)
class MoeConfig:
    """Python mirror of moe_cfg."""
    T: int
    d: int
    E: int
    k: int
    F: int
    F_shared: int = 0
    dtype: str = "bf16"          # "bf16" | "f32"
    score_fn: str = "softmax"    # "softmax" | "sigmoid"
    n_groups: int = 1
    topk_groups: int = 1
    route_scale: float = 1.0

    def to_c(self) -> moe_cfg:
        return moe_cfg(self.T, self.d, self.E, self.k, self.F, self.F_shared,
                       MOE_BF16 if self.dtype == "bf16" else
                       (MOE_F32 if self.dtype == "f32" else 99),
                       MOE_SCORE_SIGMOID if self.score_fn == "sigmoid" else
                       (MOE_SCORE_SOFTMAX if self.score_fn == "softmax" else 99),
                       self.n_groups, self.topk_groups, self.route_scale)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @classmethod
    def from_workload(cls, w, T: Optional[int] = None) -> "MoeConfig":
        return cls(T=w.T if T is None else T, d=w.d, E=w.E, k=w.k, F=w.F, F_shared=w.Fs,
                   dtype=w.dtype, score_fn=w.score_fn, n_groups=w.n_groups,
                   topk_groups=w.topk_groups, route_scale=w.route_scale)


_lib = None


def lib():
    """The loaded libmoe.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_ffn_biased_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        CP = ctypes.POINTER(moe_cfg)
        L.moe_workspace_bytes.argtypes = [CP]
        L.moe_workspace_bytes.restype = SZ
        L.moe_check_cfg.argtypes = [CP]
        L.moe_check_cfg.restype = I32
        L.moe_layer_forward.argtypes = [P, P, P, P, P, P, ctypes.POINTER(moe_shared), CP, P, P, P,
                                        P, SZ, P]
        L.moe_layer_forward.restype = I32
        L.moe_layer_forward_noalloc.argtypes = [P, P, P, P, P, P, ctypes.POINTER(moe_shared), CP, P, P, P, P]
        L.moe_layer_forward_noalloc.restype = I32
        L.moe_route_debug.argtypes = [P, P, P, CP, P, P, P, P, P, P, P, SZ, P]
        L.moe_route_debug.restype = I32
        L.moe_balance_update.argtypes = [P, I64, I32, I32, ctypes.c_float, P, P, P, P]
        L.moe_balance_update.restype = I32
        F32 = ctypes.c_float
        L.moe_rmsnorm.argtypes = [P, P, F32, I64, I32, I32, P, P]
        L.moe_rmsnorm.restype = I32
        L.moe_block_workspace_bytes.argtypes = [CP]
        L.moe_block_workspace_bytes.restype = SZ
        L.moe_block_forward.argtypes = [P, P, F32, P, P, P, P, P, ctypes.POINTER(moe_shared), CP, P, P, P,
                                        P, SZ, P]
        L.moe_block_forward.restype = I32
        L.moe_block_forward_packed.argtypes = [P, P, F32, P, P, P, CP, P, P, P, P, SZ, P]
        L.moe_block_forward_packed.restype = I32
        L.moe_block_packed_bytes.argtypes = [CP]
        L.moe_block_packed_bytes.restype = SZ
        L.moe_pack_block_weights.argtypes = [CP, P, P, P, P, P, ctypes.POINTER(moe_shared), P, SZ, P]
        L.moe_pack_block_weights.restype = I32
        L.moe_block_forward_fused.argtypes = [P, F32, P, P, CP, P, P, P, P, SZ, P]
        L.moe_block_forward_fused.restype = I32
        L.moe_packed_weights_bytes.argtypes = [CP]
        L.moe_packed_weights_bytes.restype = SZ
        L.moe_pack_weights.argtypes = [CP, P, P, P, ctypes.POINTER(moe_shared), P, SZ, P]
        L.moe_pack_weights.restype = I32
        L.moe_layer_forward_packed.argtypes = [P, P, P, P, CP, P, P, P, P, SZ, P]
        L.moe_layer_forward_packed.restype = I32
        L.moe_plan_describe.argtypes = [CP, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32)]
        L.moe_plan_describe.restype = I32
        L.moe_workspace_bytes_ex.argtypes = [CP, I32]
        L.moe_workspace_bytes_ex.restype = SZ
        L.moe_plan_describe_ex.argtypes = [CP, I32, ctypes.POINTER(ctypes.c_int32),
                                           ctypes.POINTER(ctypes.c_int32)]
        L.moe_plan_describe_ex.restype = I32
        L.moe_layer_forward_ex.argtypes = [P, P, P, ctypes.POINTER(moe_experts), CP, P, P, P, P, SZ, P]
        L.moe_layer_forward_ex.restype = I32
        L.moe_packed_weights_bytes_ex.argtypes = [CP, I32]
        L.moe_packed_weights_bytes_ex.restype = SZ
        L.moe_pack_weights_ex.argtypes = [CP, ctypes.POINTER(moe_experts), P, SZ, P]
        L.moe_pack_weights_ex.restype = I32
        L.moe_layer_forward_packed_ex.argtypes = [P, P, P, ctypes.POINTER(moe_experts), P, CP, P, P, P, P,
                                                  SZ, P]
        L.moe_layer_forward_packed_ex.restype = I32
        L.moe_status_str.argtypes = [I32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_timing_enable.argtypes = [I32]
        L.moe_timing_enable.restype = I32
        L.moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), I32]
        L.moe_timing_read.restype = I32
        _lib = L
    return _lib


def moe_status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def moe_check_cfg(cfg: MoeConfig) -> int:
    c = cfg.to_c()
    return int(lib().moe_check_cfg(ctypes.byref(c)))


GEMM_PATHS = {0: "tiled", 1: "stream", 2: "stream_decode", 3: "small"}


def moe_plan_describe(cfg: MoeConfig):
    """(gemm path name, rows per GEMM tile) the library uses for cfg."""
    c = cfg.to_c()
    path, rows = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib().moe_plan_describe(ctypes.byref(c), ctypes.byref(path), ctypes.byref(rows))
    if st != 0:
        raise MoeError(st, "moe_plan_describe")
    return GEMM_PATHS[path.value], rows.value


def moe_workspace_bytes(cfg: MoeConfig) -> int:
    c = cfg.to_c()
    return int(lib().moe_workspace_bytes(ctypes.byref(c)))


def _kind(kind) -> int:
    return EXPERT_KINDS[kind] if isinstance(kind, str) else int(kind)


def moe_workspace_bytes_ex(cfg: MoeConfig, kind) -> int:
    c = cfg.to_c()
    return int(lib().moe_workspace_bytes_ex(ctypes.byref(c), _kind(kind)))


def moe_plan_describe_ex(cfg: MoeConfig, kind):
    """moe_plan_describe for experts of the given kind ("swiglu", "geglu", "gelu_mlp")."""
    c = cfg.to_c()
    path, rows = ctypes.c_int32(-1), ctypes.c_int32(-1)
    st = lib().moe_plan_describe_ex(ctypes.byref(c), _kind(kind), ctypes.byref(path), ctypes.byref(rows))
    if st != 0:
        raise MoeError(st, "moe_plan_describe_ex")
    return GEMM_PATHS[path.value], rows.value


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, shape, dtype, name, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype}, got {tuple(t.shape)} {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, is on {t.device}")


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _on_stream(fn):
    """Runs an entry-point wrapper with the caller's `stream` current, so that
    the outputs and the workspace it allocates belong to the stream the
    kernels run on (torch's caching allocator then never hands their memory
    to other work while those kernels may still use it)."""
    @functools.wraps(fn)
    def wrapped(*args, stream=None, **kw):
        ctx = contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)
        with ctx:
            return fn(*args, stream=stream, **kw)
    return wrapped


def alloc_workspace(cfg: MoeConfig, device) -> torch.Tensor:
    n = moe_workspace_bytes(cfg)
    if n == 0 and cfg.T > 0:
        raise MoeError(moe_check_cfg(cfg), "moe_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


@_on_stream
def moe_layer_forward(u, W_router, bias, W1, W3, W2, shared: Optional[Sequence] = None, *,
                      cfg: MoeConfig, y=None, topk_idx=None, gates=None, workspace=None,
                      stream=None):
    """y, topk_idx, gates = moe_layer_forward(u, W_router, bias, W1, W3, W2, shared, cfg=cfg).

    shared: None or (W1s [Fs][d], W3s [Fs][d], W2s [d][Fs]).  bias: fp32 [E] or None."""
    dev = u.device
    dt = cfg.torch_dtype
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared
    _need(u, (T, d), dt, "u", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    _need(W1, (E, F, d), dt, "W1", dev)
    _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    sh = None
    if shared is not None:
        W1s, W3s, W2s = shared
        _need(W1s, (Fs, d), dt, "W1s", dev)
        _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        sh = moe_shared(W1s.data_ptr(), W3s.data_ptr(), W2s.data_ptr())
    if y is None:
        y = torch.empty((T, d), dtype=dt, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(y, (T, d), dt, "y", dev)
    _need(topk_idx, (T, k), torch.int32, "topk_idx", dev)
    _need(gates, (T, k), torch.float32, "gates", dev)
    if workspace is None:
        workspace = alloc_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_layer_forward(_ptr(u), _ptr(W_router), _ptr(bias), _ptr(W1), _ptr(W3), _ptr(W2),
                                 ctypes.byref(sh) if sh is not None else None, ctypes.byref(c),
                                 _ptr(y), _ptr(topk_idx), _ptr(gates), _ptr(workspace),
                                 workspace.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_layer_forward")
    return y, topk_idx, gates


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


@_on_stream
def moe_layer_forward_noalloc(u, W_router, bias, W1, W3, W2, shared: Optional[Sequence] = None, *,
                              cfg: MoeConfig, y, topk_idx, gates, stream=None):
    """moe_layer_forward without a workspace: the library's fixed per-GPU
    scratch array serves as one.  The outputs y, topk_idx and gates are the
    caller's (nothing is allocated here either)."""
    dev = u.device
    dt = cfg.torch_dtype
    T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared
    _need(u, (T, d), dt, "u", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    _need(W1, (E, F, d), dt, "W1", dev)
    _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    sh = None
    if shared is not None:
        W1s, W3s, W2s = shared
        _need(W1s, (Fs, d), dt, "W1s", dev)
        _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        sh = moe_shared(W1s.data_ptr(), W3s.data_ptr(), W2s.data_ptr())
    _need(y, (T, d), dt, "y", dev)
    _need(topk_idx, (T, k), torch.int32, "topk_idx", dev)
    _need(gates, (T, k), torch.float32, "gates", dev)
    c = cfg.to_c()
    st = lib().moe_layer_forward_noalloc(_ptr(u), _ptr(W_router), _ptr(bias), _ptr(W1), _ptr(W3), _ptr(W2),
                                         ctypes.byref(sh) if sh is not None else None, ctypes.byref(c),
                                         _ptr(y), _ptr(topk_idx), _ptr(gates), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_layer_forward_noalloc")
    return y, topk_idx, gates


def _experts(cfg, kind, W1, W3, W2, b1, b2, shared, dev):
    """Checks the expert tensors and builds the moe_experts struct."""
    dt = cfg.torch_dtype
    E, d, F, Fs = cfg.E, cfg.d, cfg.F, cfg.F_shared
    _need(W1, (E, F, d), dt, "W1", dev)
    if W3 is not None:
        _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    if b1 is not None:
        _need(b1, (E, F), dt, "b1", dev)
    if b2 is not None:
        _need(b2, (E, d), dt, "b2", dev)
    ex = moe_experts(_kind(kind), *(None if t is None else t.data_ptr() for t in (W1, W3, W2, b1, b2)))
    if shared is not None:
        sh = list(shared) + [None] * (5 - len(shared))
        W1s, W3s, W2s, b1s, b2s = sh
        _need(W1s, (Fs, d), dt, "W1s", dev)
        if W3s is not None:
            _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        if b1s is not None:
            _need(b1s, (Fs,), dt, "b1s", dev)
        if b2s is not None:
            _need(b2s, (d,), dt, "b2s", dev)
        for name, t in zip(("W1s", "W3s", "W2s", "b1s", "b2s"), sh):
            setattr(ex, name, None if t is None else t.data_ptr())
    return ex


def _bias_struct(cfg, kind, b1, b2, b1s, b2s, dev):
    """moe_experts with only the kind and the biases (for the packed forward)."""
    dt = cfg.torch_dtype
    for t, shape, name in ((b1, (cfg.E, cfg.F), "b1"), (b2, (cfg.E, cfg.d), "b2"),
                           (b1s, (cfg.F_shared,), "b1s"), (b2s, (cfg.d,), "b2s")):
        if t is not None:
            _need(t, shape, dt, name, dev)
    ex = moe_experts(_kind(kind))
    for name, t in (("b1", b1), ("b2", b2), ("b1s", b1s), ("b2s", b2s)):
        setattr(ex, name, None if t is None else t.data_ptr())
    return ex


def _layer_outputs(cfg, dev, y, topk_idx, gates):
    dt = cfg.torch_dtype
    T, d, k = cfg.T, cfg.d, cfg.k
    if y is None:
        y = torch.empty((T, d), dtype=dt, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(y, (T, d), dt, "y", dev)
    _need(topk_idx, (T, k), torch.int32, "topk_idx", dev)
    _need(gates, (T, k), torch.float32, "gates", dev)
    return y, topk_idx, gates


def _workspace_ex(cfg, kind, dev, workspace):
    if workspace is None:
        n = moe_workspace_bytes_ex(cfg, kind)
        if n == 0 and cfg.T > 0:
            raise MoeError(moe_check_cfg(cfg) or -4, "moe_workspace_bytes_ex")
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    return workspace


@_on_stream
def moe_layer_forward_ex(u, W_router, bias, kind, W1, W3, W2, b1=None, b2=None, shared=None, *,
                         cfg: MoeConfig, y=None, topk_idx=None, gates=None, workspace=None, stream=None):
    """moe_layer_forward with experts of the given kind ("swiglu", "geglu", "gelu_mlp").

    W3 is None for the GELU MLP; b1 [E][F] and b2 [E][d] (GELU MLP only) may be None.
    shared: None or (W1s, W3s, W2s[, b1s, b2s])."""
    dev = u.device
    _need(u, (cfg.T, cfg.d), cfg.torch_dtype, "u", dev)
    _need(W_router, (cfg.E, cfg.d), cfg.torch_dtype, "W_router", dev)
    if bias is not None:
        _need(bias, (cfg.E,), torch.float32, "bias", dev)
    ex = _experts(cfg, kind, W1, W3, W2, b1, b2, shared, dev)
    y, topk_idx, gates = _layer_outputs(cfg, dev, y, topk_idx, gates)
    workspace = _workspace_ex(cfg, kind, dev, workspace)
    c = cfg.to_c()
    st = lib().moe_layer_forward_ex(_ptr(u), _ptr(W_router), _ptr(bias), ctypes.byref(ex), ctypes.byref(c),
                                    _ptr(y), _ptr(topk_idx), _ptr(gates), _ptr(workspace), workspace.numel(),
                                    _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_layer_forward_ex")
    return y, topk_idx, gates


def moe_packed_weights_bytes_ex(cfg: MoeConfig, kind) -> int:
    c = cfg.to_c()
    return int(lib().moe_packed_weights_bytes_ex(ctypes.byref(c), _kind(kind)))


@_on_stream
def moe_pack_weights_ex(kind, W1, W3, W2, shared=None, *, cfg: MoeConfig, packed=None, stream=None):
    """One-time re-layout of the weights of experts of the given kind; returns
    the packed uint8 buffer (biases are not packed).  shared: None or
    (W1s, W3s, W2s); W3 / W3s None for the GELU MLP."""
    dev = W1.device
    ex = _experts(cfg, kind, W1, W3, W2, None, None, None if shared is None else tuple(shared)[:3], dev)
    n = moe_packed_weights_bytes_ex(cfg, kind)
    if n == 0:
        raise MoeError(-2, "moe_packed_weights_bytes_ex")
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=dev)
    c = cfg.to_c()
    st = lib().moe_pack_weights_ex(ctypes.byref(c), ctypes.byref(ex), _ptr(packed), packed.numel(),
                                   _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_pack_weights_ex")
    return packed


@_on_stream
def moe_layer_forward_packed_ex(u, W_router, bias, kind, packed, b1=None, b2=None, b1s=None, b2s=None, *,
                                cfg: MoeConfig, y=None, topk_idx=None, gates=None, workspace=None,
                                stream=None):
    """moe_layer_forward_ex on weights packed by moe_pack_weights_ex for the same kind."""
    dev = u.device
    _need(u, (cfg.T, cfg.d), cfg.torch_dtype, "u", dev)
    _need(W_router, (cfg.E, cfg.d), cfg.torch_dtype, "W_router", dev)
    if bias is not None:
        _need(bias, (cfg.E,), torch.float32, "bias", dev)
    _need(packed, (moe_packed_weights_bytes_ex(cfg, kind),), torch.uint8, "packed", dev)
    ex = _bias_struct(cfg, kind, b1, b2, b1s, b2s, dev)
    y, topk_idx, gates = _layer_outputs(cfg, dev, y, topk_idx, gates)
    workspace = _workspace_ex(cfg, kind, dev, workspace)
    c = cfg.to_c()
    st = lib().moe_layer_forward_packed_ex(_ptr(u), _ptr(W_router), _ptr(bias), ctypes.byref(ex), _ptr(packed),
                                           ctypes.byref(c), _ptr(y), _ptr(topk_idx), _ptr(gates),
                                           _ptr(workspace), workspace.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_layer_forward_packed_ex")
    return y, topk_idx, gates


def moe_packed_weights_bytes(cfg: MoeConfig) -> int:
    c = cfg.to_c()
    return int(lib().moe_packed_weights_bytes(ctypes.byref(c)))


@_on_stream
def moe_pack_weights(W1, W3, W2, shared: Optional[Sequence] = None, *, cfg: MoeConfig,
                     packed=None, stream=None):
    """One-time re-layout of the expert weights; returns the packed uint8 buffer."""
    dev = W1.device
    dt = cfg.torch_dtype
    E, d, F, Fs = cfg.E, cfg.d, cfg.F, cfg.F_shared
    _need(W1, (E, F, d), dt, "W1", dev)
    _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    sh = None
    if shared is not None:
        W1s, W3s, W2s = shared
        _need(W1s, (Fs, d), dt, "W1s", dev)
        _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        sh = moe_shared(W1s.data_ptr(), W3s.data_ptr(), W2s.data_ptr())
    n = moe_packed_weights_bytes(cfg)
    if n == 0:
        raise MoeError(-2, "moe_packed_weights_bytes")
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=dev)
    c = cfg.to_c()
    st = lib().moe_pack_weights(ctypes.byref(c), _ptr(W1), _ptr(W3), _ptr(W2),
                                ctypes.byref(sh) if sh is not None else None, _ptr(packed),
                                packed.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_pack_weights")
    return packed


@_on_stream
def moe_layer_forward_packed(u, W_router, bias, packed, *, cfg: MoeConfig, y=None, topk_idx=None,
                             gates=None, workspace=None, stream=None):
    """moe_layer_forward with weights from moe_pack_weights."""
    dev = u.device
    dt = cfg.torch_dtype
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    _need(u, (T, d), dt, "u", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    _need(packed, (moe_packed_weights_bytes(cfg),), torch.uint8, "packed", dev)
    if y is None:
        y = torch.empty((T, d), dtype=dt, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(y, (T, d), dt, "y", dev)
    _need(topk_idx, (T, k), torch.int32, "topk_idx", dev)
    _need(gates, (T, k), torch.float32, "gates", dev)
    if workspace is None:
        workspace = alloc_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_layer_forward_packed(_ptr(u), _ptr(W_router), _ptr(bias), _ptr(packed),
                                        ctypes.byref(c), _ptr(y), _ptr(topk_idx), _ptr(gates),
                                        _ptr(workspace), workspace.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_layer_forward_packed")
    return y, topk_idx, gates


@_on_stream
def moe_rmsnorm(h, norm_weight, eps: float, *, out=None, stream=None):
    """out = h / sqrt(mean(h^2, -1) + eps) * norm_weight, rows of h [T][d] (bf16 or fp32)."""
    dev = h.device
    if h.dim() != 2 or h.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("h must be a [T][d] bf16 or fp32 tensor")
    T, d = h.shape
    _need(h, (T, d), h.dtype, "h", dev)
    _need(norm_weight, (d,), h.dtype, "norm_weight", dev)
    if out is None:
        out = torch.empty_like(h)
    _need(out, (T, d), h.dtype, "out", dev)
    dtype = MOE_BF16 if h.dtype == torch.bfloat16 else MOE_F32
    st = lib().moe_rmsnorm(_ptr(h), _ptr(norm_weight), float(eps), T, d, dtype, _ptr(out), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_rmsnorm")
    return out


def moe_block_workspace_bytes(cfg: MoeConfig) -> int:
    c = cfg.to_c()
    return int(lib().moe_block_workspace_bytes(ctypes.byref(c)))


def alloc_block_workspace(cfg: MoeConfig, device) -> torch.Tensor:
    n = moe_block_workspace_bytes(cfg)
    if n == 0 and cfg.T > 0:
        raise MoeError(moe_check_cfg(cfg) or -2, "moe_block_workspace_bytes")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _block_outputs(cfg, dev, y, topk_idx, gates):
    dt = cfg.torch_dtype
    T, d, k = cfg.T, cfg.d, cfg.k
    if y is None:
        y = torch.empty((T, d), dtype=dt, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if gates is None:
        gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(y, (T, d), dt, "y", dev)
    _need(topk_idx, (T, k), torch.int32, "topk_idx", dev)
    _need(gates, (T, k), torch.float32, "gates", dev)
    return y, topk_idx, gates


@_on_stream
def moe_block_forward(h, norm_weight, norm_eps, W_router, bias, W1, W3, W2, shared=None, *, cfg: MoeConfig,
                      y=None, topk_idx=None, gates=None, workspace=None, stream=None):
    """y = h + MoE(RMSNorm(h)); returns (y, topk_idx, gates)."""
    dev = h.device
    dt = cfg.torch_dtype
    T, d, E, F, Fs = cfg.T, cfg.d, cfg.E, cfg.F, cfg.F_shared
    _need(h, (T, d), dt, "h", dev)
    _need(norm_weight, (d,), dt, "norm_weight", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    _need(W1, (E, F, d), dt, "W1", dev)
    _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    sh = None
    if shared is not None:
        W1s, W3s, W2s = shared
        _need(W1s, (Fs, d), dt, "W1s", dev)
        _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        sh = moe_shared(W1s.data_ptr(), W3s.data_ptr(), W2s.data_ptr())
    y, topk_idx, gates = _block_outputs(cfg, dev, y, topk_idx, gates)
    if workspace is None:
        workspace = alloc_block_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_block_forward(_ptr(h), _ptr(norm_weight), float(norm_eps), _ptr(W_router), _ptr(bias),
                                 _ptr(W1), _ptr(W3), _ptr(W2), ctypes.byref(sh) if sh is not None else None,
                                 ctypes.byref(c), _ptr(y), _ptr(topk_idx), _ptr(gates), _ptr(workspace),
                                 workspace.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_block_forward")
    return y, topk_idx, gates


@_on_stream
def moe_block_forward_packed(h, norm_weight, norm_eps, W_router, bias, packed, *, cfg: MoeConfig, y=None,
                             topk_idx=None, gates=None, workspace=None, stream=None):
    """moe_block_forward with weights from moe_pack_weights."""
    dev = h.device
    dt = cfg.torch_dtype
    T, d, E = cfg.T, cfg.d, cfg.E
    _need(h, (T, d), dt, "h", dev)
    _need(norm_weight, (d,), dt, "norm_weight", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    _need(packed, (moe_packed_weights_bytes(cfg),), torch.uint8, "packed", dev)
    y, topk_idx, gates = _block_outputs(cfg, dev, y, topk_idx, gates)
    if workspace is None:
        workspace = alloc_block_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_block_forward_packed(_ptr(h), _ptr(norm_weight), float(norm_eps), _ptr(W_router),
                                        _ptr(bias), _ptr(packed), ctypes.byref(c), _ptr(y), _ptr(topk_idx),
                                        _ptr(gates), _ptr(workspace), workspace.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_block_forward_packed")
    return y, topk_idx, gates


def moe_block_packed_bytes(cfg: MoeConfig) -> int:
    """Bytes of the fused block's packed buffer (0: cfg cannot be packed)."""
    c = cfg.to_c()
    return int(lib().moe_block_packed_bytes(ctypes.byref(c)))


@_on_stream
def moe_pack_block_weights(norm_weight, W_router, W1, W3, W2, shared: Optional[Sequence] = None, *,
                           cfg: MoeConfig, packed=None, stream=None):
    """One-time packing for moe_block_forward_fused: the expert weights in the
    streaming kernels' order with the RMSNorm weight folded into W1, W3 (and
    the shared W1s, W3s), then the router rows folded the same way."""
    dev = W1.device
    dt = cfg.torch_dtype
    E, d, F, Fs = cfg.E, cfg.d, cfg.F, cfg.F_shared
    _need(norm_weight, (d,), dt, "norm_weight", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    _need(W1, (E, F, d), dt, "W1", dev)
    _need(W3, (E, F, d), dt, "W3", dev)
    _need(W2, (E, d, F), dt, "W2", dev)
    sh = None
    if shared is not None:
        W1s, W3s, W2s = shared
        _need(W1s, (Fs, d), dt, "W1s", dev)
        _need(W3s, (Fs, d), dt, "W3s", dev)
        _need(W2s, (d, Fs), dt, "W2s", dev)
        sh = moe_shared(W1s.data_ptr(), W3s.data_ptr(), W2s.data_ptr())
    n = moe_block_packed_bytes(cfg)
    if n == 0:
        raise MoeError(-2, "moe_block_packed_bytes")
    if packed is None:
        packed = torch.empty(n, dtype=torch.uint8, device=dev)
    c = cfg.to_c()
    st = lib().moe_pack_block_weights(ctypes.byref(c), _ptr(norm_weight), _ptr(W_router), _ptr(W1), _ptr(W3),
                                      _ptr(W2), ctypes.byref(sh) if sh is not None else None, _ptr(packed),
                                      packed.numel(), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_pack_block_weights")
    return packed


@_on_stream
def moe_block_forward_fused(h, norm_eps, bias, packed, *, cfg: MoeConfig, y=None, topk_idx=None, gates=None,
                            workspace=None, stream=None):
    """y = h + MoE(RMSNorm(h)) with the normalisation fused (packed buffer from
    moe_pack_block_weights, which holds the norm weight and the router)."""
    dev = h.device
    dt = cfg.torch_dtype
    T, d, E = cfg.T, cfg.d, cfg.E
    _need(h, (T, d), dt, "h", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    _need(packed, (moe_block_packed_bytes(cfg),), torch.uint8, "packed", dev)
    y, topk_idx, gates = _block_outputs(cfg, dev, y, topk_idx, gates)
    if workspace is None:
        workspace = alloc_block_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_block_forward_fused(_ptr(h), float(norm_eps), _ptr(bias), _ptr(packed), ctypes.byref(c),
                                       _ptr(y), _ptr(topk_idx), _ptr(gates), _ptr(workspace), workspace.numel(),
                                       _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_block_forward_fused")
    return y, topk_idx, gates


@_on_stream
def moe_route_debug(u, W_router, bias, *, cfg: MoeConfig, workspace=None, stream=None):
    """Routing + permutation only: (topk_idx, gates, counts, offsets, perm, inv)."""
    dev = u.device
    dt = cfg.torch_dtype
    T, d, E, k = cfg.T, cfg.d, cfg.E, cfg.k
    _need(u, (T, d), dt, "u", dev)
    _need(W_router, (E, d), dt, "W_router", dev)
    if bias is not None:
        _need(bias, (E,), torch.float32, "bias", dev)
    i32 = dict(dtype=torch.int32, device=dev)
    topk_idx = torch.empty((T, k), **i32)
    gates = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, **i32)
    offsets = torch.empty(E + 1, **i32)
    perm = torch.empty(T * k, **i32)
    inv = torch.empty(T * k, **i32)
    if workspace is None:
        workspace = alloc_workspace(cfg, dev)
    c = cfg.to_c()
    st = lib().moe_route_debug(_ptr(u), _ptr(W_router), _ptr(bias), ctypes.byref(c),
                               _ptr(topk_idx), _ptr(gates), _ptr(counts), _ptr(offsets),
                               _ptr(perm), _ptr(inv), _ptr(workspace), workspace.numel(),
                               _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_route_debug")
    return topk_idx, gates, counts, offsets, perm, inv


@_on_stream
def moe_balance_update(topk_idx, bias, *, E: int, gamma: float = 0.15, counts=None, entropy=None,
                       stream=None):
    """One aux-loss-free balance step on the routing topk_idx [T][k] (int32):
    updates bias [E] (fp32) in place; returns (counts [E] int32, entropy [1] fp32)."""
    dev = bias.device
    _need(bias, (E,), torch.float32, "bias", dev)
    if topk_idx.dim() != 2 or topk_idx.dtype != torch.int32 or topk_idx.device != dev:
        raise ValueError("topk_idx must be an int32 [T][k] tensor on the bias device")
    if not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous")
    T, k = topk_idx.shape
    if counts is None:
        counts = torch.empty(E, dtype=torch.int32, device=dev)
    if entropy is None:
        entropy = torch.empty(1, dtype=torch.float32, device=dev)
    st = lib().moe_balance_update(_ptr(topk_idx) if T > 0 else None, T, k, E, float(gamma), _ptr(bias),
                                  _ptr(counts), _ptr(entropy), _stream(dev, stream))
    if st != 0:
        raise MoeError(st, "moe_balance_update")
    return counts, entropy


def moe_timing_enable(on: bool) -> None:
    lib().moe_timing_enable(1 if on else 0)


def moe_timing_read(reset: bool = True):
    """(milliseconds per stage summed over the recorded calls, number of calls)."""
    ms = (ctypes.c_double * MOE_N_STAGES)()
    calls = ctypes.c_int64(0)
    st = lib().moe_timing_read(ms, ctypes.byref(calls), 1 if reset else 0)
    if st != 0:
        raise MoeError(st, "moe_timing_read")
    return list(ms), int(calls.value)
