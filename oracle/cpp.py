"""ctypes binding of the C++ float64 oracle (moe_oracle.cpp).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import this module; the GPU library never does.

The functions have the names, arguments and results of the NumPy oracle
(oracle.moe_oracle), so the same pins check both implementations.  Arrays may be
NumPy arrays (float64 or float32) or torch CPU tensors (float32 or bfloat16,
read in place: the C++ code converts one element at a time, exactly, to
float64).  Layouts are the x W orientation: x [T, d]; w_router [d, N];
w_gate, w_up [N, d, d_ff] (one expert: [d, d_ff]); w_down [N, d_ff, d].

The library is built by oracle/build.py (called from __graft_entry__.build());
if it is missing it is built here on first use.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Dict, Optional, Sequence

import numpy as np

from .moe_oracle import RELU2, SOFTMAX_TOPK, SWIGLU, TOPK_SOFTMAX

_DT_F32, _DT_BF16, _DT_F64 = 0, 1, 2
_FFN = {RELU2: 0, SWIGLU: 1}
_GATING = {TOPK_SOFTMAX: 0, SOFTMAX_TOPK: 1}
_lib = None

_vp, _i32, _dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double


class _Layer(ctypes.Structure):
    _fields_ = [(n, _i32) for n in ("T", "d", "N", "k", "d_ff", "ffn", "gating", "has_shared")] + [
        ("capacity_factor", _dbl), ("x", _vp), ("x_dt", _i32), ("w_router", _vp), ("wr_dt", _i32),
        ("logit_bias", _vp), ("w_gate", _vp), ("w_up", _vp), ("w_down", _vp), ("sh_gate", _vp),
        ("sh_up", _vp), ("sh_down", _vp), ("w_dt", _i32), ("z_in", _vp)]


class _Out(ctypes.Structure):
    _fields_ = [(n, _vp) for n in ("z", "idx", "w", "counts", "offsets", "perm", "inv", "C", "y")]


def load():
    """The loaded library (built with g++ first if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    from .build import LIB, build
    if not os.path.exists(LIB):
        build(verbose=False)
    lib = ctypes.CDLL(LIB)
    lib.orc_max_threads.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_router_logits.argtypes = [_i32, _i32, _i32, _vp, _i32, _vp, _i32, _vp, _vp]
    lib.orc_rank_experts.argtypes = [_i32, _i32, _vp, _vp]
    lib.orc_gate_weights.argtypes = [_i32, _i32, _i32, _vp, _vp, _i32, _vp]
    lib.orc_topk_route.argtypes = [_i32, _i32, _i32, _vp, _i32, _vp, _vp]
    lib.orc_capacity_route.argtypes = [_i32, _i32, _i32, ctypes.c_int64, _vp, _i32, _vp, _vp, _vp]
    lib.orc_group_by_expert.argtypes = [_i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.orc_expert_ffn.argtypes = [_i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp, _vp, _i32, _vp]
    lib.orc_forward.argtypes = [ctypes.POINTER(_Layer), _i32, _vp, ctypes.POINTER(_Out)]
    lib.orc_forward.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(load().orc_max_threads())


def set_threads(n: int) -> None:
    """Threads of the OpenMP loops (over tokens or rows; results do not depend on it)."""
    load().orc_set_threads(int(n))


class _In:
    """An input array as (pointer, dtype code), kept alive while the call runs."""

    def __init__(self, a):
        if a is None:
            self.keep, self.ptr, self.dt, self.shape = None, None, _DT_F64, ()
            return
        if type(a).__module__.startswith("torch"):
            import torch
            t = a.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                dt = _DT_BF16
            elif t.dtype == torch.float32:
                dt = _DT_F32
            else:
                t, dt = t.to(torch.float64), _DT_F64
            self.keep, self.ptr, self.dt, self.shape = t, t.data_ptr(), dt, tuple(t.shape)
            return
        arr = np.asarray(a)
        if arr.dtype == np.float32:
            arr, dt = np.ascontiguousarray(arr), _DT_F32
        else:
            arr, dt = np.ascontiguousarray(arr, dtype=np.float64), _DT_F64
        self.keep, self.ptr, self.dt, self.shape = arr, arr.ctypes.data, dt, arr.shape


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32a(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """z[t, e] = sum_i x[t, i] w_router[i, e] (+ b[e]); w_router [d, N]."""
    X, Wr = _In(x), _In(w_router)
    T, d = X.shape
    N = Wr.shape[1]
    assert Wr.shape[0] == d
    b = None if logit_bias is None else np.ascontiguousarray(np.asarray(logit_bias, dtype=np.float32))
    z = np.empty((T, N), dtype=np.float64)
    load().orc_router_logits(T, d, N, X.ptr, X.dt, Wr.ptr, Wr.dt, None if b is None else b.ctypes.data,
                             z.ctypes.data)
    return z


def rank_experts(z) -> np.ndarray:
    z = _f64(z)
    T, N = z.shape
    o = np.empty((T, N), dtype=np.int32)
    load().orc_rank_experts(T, N, z.ctypes.data, o.ctypes.data)
    return o.astype(np.int64)


def gate_weights(z, idx, gating: str) -> np.ndarray:
    z, idx = _f64(z), _i32a(idx)
    T, N = z.shape
    k = idx.shape[1]
    w = np.empty((T, k), dtype=np.float64)
    load().orc_gate_weights(T, N, k, z.ctypes.data, idx.ctypes.data, _GATING[gating], w.ctypes.data)
    return w


def topk_route(z, k: int, gating: str):
    z = _f64(z)
    T, N = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    load().orc_topk_route(T, N, k, z.ctypes.data, _GATING[gating], idx.ctypes.data, w.ctypes.data)
    return idx.astype(np.int64), w


def capacity_route(z, k: int, C: int, gating: str = TOPK_SOFTMAX):
    z = _f64(z)
    T, N = z.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    fill = np.empty(N, dtype=np.int64)
    load().orc_capacity_route(T, N, k, int(C), z.ctypes.data, _GATING[gating], idx.ctypes.data, w.ctypes.data,
                              fill.ctypes.data)
    return idx.astype(np.int64), w, fill


def expert_capacity(capacity_factor: float, T: int, k: int, N: int) -> int:
    return int(math.ceil(capacity_factor * T * k / N))


def route_from_logits(z, k: int, gating: str, C: Optional[int] = None):
    if C is None or C <= 0:
        return topk_route(z, k, gating)
    idx, w, _ = capacity_route(z, k, C, gating)
    return idx, w


def group_by_expert(idx, N: int):
    idx = _i32a(idx)
    T, k = idx.shape
    counts = np.empty(N, dtype=np.int32)
    offsets = np.empty(N + 1, dtype=np.int32)
    perm = np.empty(max(T * k, 1), dtype=np.int32)
    inv = np.empty(max(T * k, 1), dtype=np.int32)
    load().orc_group_by_expert(T, k, N, idx.ctypes.data, counts.ctypes.data, offsets.ctypes.data,
                               perm.ctypes.data, inv.ctypes.data)
    n = int(offsets[N])
    return (counts.astype(np.int64), offsets.astype(np.int64), perm[:n].astype(np.int64),
            inv[:T * k].astype(np.int64))


def expert_ffn(xr, w_up, w_down, ffn: str, w_gate=None) -> np.ndarray:
    """One expert on rows xr [M, d]; w_gate, w_up [d, d_ff], w_down [d_ff, d]."""
    X, U, D, G = _In(xr), _In(w_up), _In(w_down), _In(w_gate)
    M, d = X.shape
    d_ff = U.shape[1]
    assert U.shape[0] == d and D.shape == (d_ff, d)
    if ffn == SWIGLU:
        assert G.shape == (d, d_ff) and G.dt == U.dt
    assert U.dt == D.dt
    y = np.empty((M, d), dtype=np.float64)
    load().orc_expert_ffn(M, d, d_ff, _FFN[ffn], X.ptr, X.dt, G.ptr, U.ptr, D.ptr, U.dt, y.ctypes.data)
    return y


def forward(x, w_router, w_up, w_down, k: int, ffn: str, gating: str, w_gate=None,
            logit_bias=None, capacity_factor: float = 0.0, shared: Optional[Sequence] = None,
            tokens: Optional[Sequence[int]] = None, z=None) -> Dict[str, np.ndarray]:
    """The whole layer, steps 1-7, as oracle.moe_oracle.forward: expert weights are whole stacks
    (w_gate, w_up [N, d, d_ff], w_down [N, d_ff, d]) in one dtype; shared = (sh_gate, sh_up,
    sh_down) or None; tokens: evaluate the FFNs and the combine for these tokens only; z: use
    these logits instead of step 1."""
    X, Wr = _In(x), _In(w_router)
    U, D, G = _In(w_up), _In(w_down), _In(w_gate)
    T, d = X.shape
    N, _, d_ff = U.shape
    assert U.shape == (N, d, d_ff) and D.shape == (N, d_ff, d)
    assert U.dt == D.dt and (ffn != SWIGLU or (G.shape == U.shape and G.dt == U.dt))
    S = [_In(None)] * 3
    if shared is not None:
        S = [_In(a) for a in shared]
        assert S[1].shape == (d, d_ff) and S[2].shape == (d_ff, d) and S[1].dt == U.dt
    zin = None if z is None else _f64(z)
    b = None if logit_bias is None else np.ascontiguousarray(np.asarray(logit_bias, dtype=np.float32))
    L = _Layer(T=T, d=d, N=N, k=k, d_ff=d_ff, ffn=_FFN[ffn], gating=_GATING[gating],
               has_shared=1 if shared is not None else 0, capacity_factor=float(capacity_factor),
               x=X.ptr, x_dt=X.dt, w_router=Wr.ptr, wr_dt=Wr.dt,
               logit_bias=None if b is None else b.ctypes.data, w_gate=G.ptr, w_up=U.ptr, w_down=D.ptr,
               sh_gate=S[0].ptr, sh_up=S[1].ptr, sh_down=S[2].ptr, w_dt=U.dt,
               z_in=None if zin is None else zin.ctypes.data)
    tok = None if tokens is None else _i32a(tokens)
    n = T if tok is None else tok.size
    zo = np.empty((T, N), dtype=np.float64)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    counts = np.empty(N, dtype=np.int32)
    offsets = np.empty(N + 1, dtype=np.int32)
    perm = np.empty(max(T * k, 1), dtype=np.int32)
    inv = np.empty(max(T * k, 1), dtype=np.int32)
    C = np.zeros(1, dtype=np.int64)
    y = np.empty((n, d), dtype=np.float64)
    out = _Out(zo.ctypes.data, idx.ctypes.data, w.ctypes.data, counts.ctypes.data, offsets.ctypes.data,
               perm.ctypes.data, inv.ctypes.data, C.ctypes.data, y.ctypes.data)
    rc = load().orc_forward(ctypes.byref(L), n, None if tok is None else tok.ctypes.data, ctypes.byref(out))
    if rc != 0:
        raise ValueError("orc_forward: invalid layer shape")
    nk = int(offsets[N])
    return dict(z=zo, idx=idx.astype(np.int64), w=w, counts=counts.astype(np.int64),
                offsets=offsets.astype(np.int64), perm=perm[:nk].astype(np.int64),
                inv=inv[:T * k].astype(np.int64), C=int(C[0]), y=y)
