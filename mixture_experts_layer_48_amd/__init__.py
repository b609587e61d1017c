"""Python binding of libmoe.so, the MI355X (gfx950) sparse MoE layer forward.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory and the current HIP stream.  The
functions keep the C ABI's names (include/moe.h) and raise MoeError on any
status other than MOE_OK.  If libmoe.so has not been built this module still
imports, but every call raises (there is no other code path).
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_GATE_TOPK_SOFTMAX, MOE_GATE_SOFTMAX_TOPK = 0, 1
MOE_FFN_RELU2, MOE_FFN_SWIGLU = 0, 1
MOE_NUM_STAGES = 6
STAGE_NAMES = ("route", "capacity", "permute", "ffn_in", "ffn_out", "combine")
MOE_NUM_STATS = 8
MOE_EP_MAX_RANKS = 64
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
STAT_NAMES = ("entropy_bits", "entropy_ideal_bits", "top3_share", "max_share", "cv", "balance_loss",
              "reroute_rate", "experts_touched")

_DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16}
_FFNS = {"relu2": MOE_FFN_RELU2, "swiglu": MOE_FFN_SWIGLU}
_GATINGS = {"topk_softmax": MOE_GATE_TOPK_SOFTMAX, "softmax_topk": MOE_GATE_SOFTMAX_TOPK}


class MoeError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {_status_name(status)}: {detail}")


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("gating", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("has_shared", ctypes.c_int32)]


class moe_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "logit_bias", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")]


class moe_q4_matrix(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class moe_weights_q4(ctypes.Structure):
    _fields_ = [("w_router", ctypes.c_void_p), ("logit_bias", ctypes.c_void_p)] + \
               [(n, moe_q4_matrix) for n in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")]


class moe_routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("logits", "idx", "w", "counts", "offsets", "perm", "inv")]


_lib: Optional[ctypes.CDLL] = None


def _status_name(s: int) -> str:
    names = ["MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]
    return names[s] if 0 <= s < len(names) else f"status {s}"


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m mixture_experts_layer_48_amd.build`")
    # torch first: its HIP runtime (same soname) is then the one libmoe.so binds to, so streams
    # and device pointers from torch are valid in the library
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    pdesc = ctypes.POINTER(moe_layer_desc)
    lib.moe_workspace_size.argtypes = [pdesc]
    lib.moe_workspace_size.restype = sz
    lib.moe_route.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute.argtypes = [pdesc, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_expert_ffn.argtypes = [pdesc, ctypes.POINTER(moe_weights), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_combine.argtypes = [pdesc, vp, vp, vp, vp, vp]
    lib.moe_layer_forward.argtypes = [pdesc, ctypes.POINTER(moe_weights), vp, vp,
                                      ctypes.POINTER(moe_routing), vp, sz, vp]
    lib.moe_layer_forward_timed.argtypes = [pdesc, ctypes.POINTER(moe_weights), vp, vp,
                                            ctypes.POINTER(moe_routing), vp, sz, vp, ctypes.POINTER(vp)]
    lib.moe_layer_forward_noalloc.argtypes = [pdesc, ctypes.POINTER(moe_weights), vp, vp,
                                              ctypes.POINTER(moe_routing), vp]
    lib.moe_routing_stats.argtypes = [pdesc, vp, vp, vp, ctypes.c_double, vp, vp, vp, vp, sz, vp]
    pi32 = ctypes.POINTER(ctypes.c_int32)
    pq4 = ctypes.POINTER(moe_weights_q4)
    lib.moe_quantize_q4.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.moe_expert_ffn_q4.argtypes = [pdesc, pq4, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_layer_forward_q4.argtypes = [pdesc, pq4, vp, vp, ctypes.POINTER(moe_routing), vp, sz, vp,
                                         ctypes.POINTER(vp)]
    lib.moe_ep_dispatch.argtypes = [pdesc, vp, pi32, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.moe_ep_receive_layout.argtypes = [ctypes.c_int32, ctypes.c_int32, pi32, ctypes.c_int32, vp,
                                          ctypes.c_int32, vp, vp, vp, vp, vp]
    lib.moe_ep_unpack.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp, vp]
    for f in ("moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
              "moe_layer_forward_timed", "moe_layer_forward_noalloc", "moe_routing_stats", "moe_ep_dispatch", "moe_ep_receive_layout",
              "moe_ep_unpack", "moe_quantize_q4", "moe_expert_ffn_q4", "moe_layer_forward_q4"):
        getattr(lib, f).restype = i32
    lib.moe_status_str.argtypes = [i32]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_version.argtypes = []
    lib.moe_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != MOE_OK:
        raise MoeError(status, func, load_library().moe_last_error().decode())


def make_desc(T: int, d: int, N: int, k: int, d_ff: int, dtype: str = "bf16", ffn: str = "swiglu",
              gating: str = "topk_softmax", capacity_factor: float = 0.0, has_shared: bool = False) -> moe_layer_desc:
    return moe_layer_desc(T, d, N, k, d_ff, _DTYPES.get(dtype, dtype), _FFNS.get(ffn, ffn),
                          _GATINGS.get(gating, gating), float(capacity_factor), int(bool(has_shared)))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _weights(w: Dict) -> moe_weights:
    return moe_weights(*(_ptr(w.get(n)) for n in
                         ("w_router", "logit_bias", "w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")))


# ---------------------------------------------------------------- the C ABI, one to one
def moe_workspace_size(desc: moe_layer_desc) -> int:
    return int(load_library().moe_workspace_size(ctypes.byref(desc)))


def moe_route(desc, x, w_router, logit_bias, logits, idx, w, ws, stream=None) -> None:
    _check(load_library().moe_route(ctypes.byref(desc), _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(logits),
                                    _ptr(idx), _ptr(w), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream)), "moe_route")


def moe_permute(desc, idx, counts, offsets, perm, inv, x=None, x_perm=None, stream=None) -> None:
    _check(load_library().moe_permute(ctypes.byref(desc), _ptr(idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                                      _ptr(inv), _ptr(x), _ptr(x_perm), _stream(stream)), "moe_permute")


def moe_expert_ffn(desc, weights: Dict, x, perm, offsets, row_scale, y_perm, ws, stream=None) -> None:
    wt = _weights(weights)
    _check(load_library().moe_expert_ffn(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(perm), _ptr(offsets),
                                         _ptr(row_scale), _ptr(y_perm), _ptr(ws),
                                         0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn")


def moe_combine(desc, y_perm, inv, w, y, stream=None) -> None:
    _check(load_library().moe_combine(ctypes.byref(desc), _ptr(y_perm), _ptr(inv), _ptr(w), _ptr(y),
                                      _stream(stream)), "moe_combine")


def moe_layer_forward(desc, weights: Dict, x, y, routing: Optional[Dict] = None, ws=None, stream=None,
                      events: Optional[Sequence[int]] = None) -> None:
    """The whole layer; `events` (MOE_NUM_STAGES + 1 hipEvent_t handles, None = no event at that
    stage boundary) selects the timed entry point."""
    lib = load_library()
    wt = _weights(weights)
    r = moe_routing(*(_ptr((routing or {}).get(n)) for n in
                      ("logits", "idx", "w", "counts", "offsets", "perm", "inv")))
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    if events is None:
        st = lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(y), ctypes.byref(r),
                                   _ptr(ws), ws_bytes, _stream(stream))
        _check(st, "moe_layer_forward")
    else:
        arr = (ctypes.c_void_p * len(events))(*events)
        st = lib.moe_layer_forward_timed(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(y), ctypes.byref(r),
                                         _ptr(ws), ws_bytes, _stream(stream), arr)
        _check(st, "moe_layer_forward_timed")


def moe_layer_forward_noalloc(desc, weights: Dict, x, y, routing: Optional[Dict] = None, stream=None) -> None:
    """The whole layer on the library's built-in per-GPU workspace (MOE_NOALLOC_SCRATCH_BYTES):
    no workspace argument and no allocation."""
    wt = _weights(weights)
    r = moe_routing(*(_ptr((routing or {}).get(n)) for n in
                      ("logits", "idx", "w", "counts", "offsets", "perm", "inv")))
    _check(load_library().moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(y),
                                                    ctypes.byref(r), _stream(stream)), "moe_layer_forward_noalloc")


def moe_routing_stats(desc, logits, idx, counts, stats, top3, ws, alpha: float = 0.01, prob_mean=None,
                      stream=None) -> None:
    _check(load_library().moe_routing_stats(ctypes.byref(desc), _ptr(logits), _ptr(idx), _ptr(counts),
                                            float(alpha), _ptr(stats), _ptr(top3), _ptr(prob_mean), _ptr(ws),
                                            0 if ws is None else ws.numel() * ws.element_size(),
                                            _stream(stream)), "moe_routing_stats")


def _owner_arr(owner: Sequence[int]):
    return (ctypes.c_int32 * len(owner))(*[int(v) for v in owner])


def moe_ep_dispatch(desc, idx, owner: Sequence[int], G: int, counts, expert_offsets, send_counts, send_offsets,
                    perm, inv, x=None, send_buf=None, stream=None) -> None:
    """owner: host sequence [N] of ranks; the other tensors on the device."""
    _check(load_library().moe_ep_dispatch(ctypes.byref(desc), _ptr(idx), _owner_arr(owner), int(G), _ptr(counts),
                                          _ptr(expert_offsets), _ptr(send_counts), _ptr(send_offsets), _ptr(perm),
                                          _ptr(inv), _ptr(x), _ptr(send_buf), _stream(stream)), "moe_ep_dispatch")


def moe_ep_receive_layout(N: int, G: int, owner: Sequence[int], rank: int, recv_counts, max_rows: int,
                          recv_offsets, local_offsets, recv_perm, recv_inv, stream=None) -> None:
    _check(load_library().moe_ep_receive_layout(int(N), int(G), _owner_arr(owner), int(rank), _ptr(recv_counts),
                                                int(max_rows), _ptr(recv_offsets), _ptr(local_offsets),
                                                _ptr(recv_perm), _ptr(recv_inv), _stream(stream)),
           "moe_ep_receive_layout")


def moe_ep_unpack(G: int, max_rows: int, row_bytes: int, recv_offsets, recv_inv, y_grouped, ret,
                  stream=None) -> None:
    _check(load_library().moe_ep_unpack(int(G), int(max_rows), int(row_bytes), _ptr(recv_offsets), _ptr(recv_inv),
                                        _ptr(y_grouped), _ptr(ret), _stream(stream)), "moe_ep_unpack")


def moe_quantize_q4(w, codes, scales, stream=None) -> None:
    """w: bf16 device tensor [n_mats, K, rows] (or [K, rows]; the x W orientation); codes
    uint32-sized [.., rows, K/8] (int32 storage is fine); scales fp32 [n_mats, K/128, rows]."""
    shape = tuple(w.shape)
    n_mats, K, rows = (1,) + shape if len(shape) == 2 else shape
    _check(load_library().moe_quantize_q4(_ptr(w), n_mats, rows, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_q4")


def _weights_q4(q: Dict) -> moe_weights_q4:
    def m(name):
        return moe_q4_matrix(_ptr(q.get(name + "_codes")), _ptr(q.get(name + "_scales")))
    return moe_weights_q4(_ptr(q.get("w_router")), _ptr(q.get("logit_bias")),
                          *(m(n) for n in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down")))


def moe_expert_ffn_q4(desc, qweights: Dict, x, perm, offsets, row_scale, y_perm, ws, stream=None) -> None:
    wt = _weights_q4(qweights)
    _check(load_library().moe_expert_ffn_q4(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(perm),
                                            _ptr(offsets), _ptr(row_scale), _ptr(y_perm), _ptr(ws),
                                            0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "moe_expert_ffn_q4")


def moe_layer_forward_q4(desc, qweights: Dict, x, y, routing: Optional[Dict] = None, ws=None, stream=None,
                         events: Optional[Sequence[int]] = None) -> None:
    lib = load_library()
    wt = _weights_q4(qweights)
    r = moe_routing(*(_ptr((routing or {}).get(n)) for n in
                      ("logits", "idx", "w", "counts", "offsets", "perm", "inv")))
    arr = None if events is None else (ctypes.c_void_p * len(events))(*events)
    _check(lib.moe_layer_forward_q4(ctypes.byref(desc), ctypes.byref(wt), _ptr(x), _ptr(y), ctypes.byref(r),
                                    _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                    _stream(stream), arr), "moe_layer_forward_q4")


def quantize_weights_q4(weights: Dict, stream=None) -> Dict:
    """Int4 copies of a layer's expert weights (bf16 device tensors in the ABI layouts):
    returns {name + "_codes", name + "_scales"} for every expert matrix present, plus the
    router and bias as they are."""
    import torch
    out = {"w_router": weights.get("w_router"), "logit_bias": weights.get("logit_bias")}
    for name in ("w_gate", "w_up", "w_down", "sh_gate", "sh_up", "sh_down"):
        w = weights.get(name)
        if w is None:
            continue
        shape = tuple(w.shape)
        n_mats, K, rows = (1,) + shape if len(shape) == 2 else shape
        codes = torch.empty((n_mats, rows, K // 8), dtype=torch.int32, device=w.device)
        scales = torch.empty((n_mats, K // 128, rows), dtype=torch.float32, device=w.device)
        moe_quantize_q4(w, codes, scales, stream=stream)
        out[name + "_codes"], out[name + "_scales"] = codes, scales
    return out


# ---------------------------------------------------------------- convenience
class MoELayer:
    """One layer's descriptor, weights (device tensors in the ABI layouts) and workspace.

    forward(x) enqueues moe_layer_forward on the current stream and returns
    y plus, if routing=True, the routing tensors (logits, idx, w, counts,
    offsets, perm, inv)."""

    def __init__(self, desc: moe_layer_desc, weights: Dict, device=None, qweights: Optional[Dict] = None):
        """qweights: int4 expert weights (quantize_weights_q4); forward then runs
        moe_layer_forward_q4."""
        import torch
        self.desc = desc
        self.weights = weights
        self.qweights = qweights
        ref = weights["w_up"] if weights.get("w_up") is not None else weights["w_router"]
        self.device = device or ref.device
        self.dtype = ref.dtype
        nbytes = moe_workspace_size(desc)
        if nbytes == 0:
            _check(MOE_ERR_INVALID_ARG, "moe_workspace_size")
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)

    def routing_buffers(self) -> Dict:
        import torch
        T, N, k = self.desc.T, self.desc.N, self.desc.k
        dev = self.device
        return dict(logits=torch.empty((T, N), dtype=torch.float32, device=dev),
                    idx=torch.empty((T, k), dtype=torch.int32, device=dev),
                    w=torch.empty((T, k), dtype=torch.float32, device=dev),
                    counts=torch.empty(N, dtype=torch.int32, device=dev),
                    offsets=torch.empty(N + 1, dtype=torch.int32, device=dev),
                    perm=torch.empty(T * k, dtype=torch.int32, device=dev),
                    inv=torch.empty(T * k, dtype=torch.int32, device=dev))

    def routing_stats(self, r: Dict, alpha: float = 0.01, with_prob_mean: bool = False) -> Dict:
        """Enqueue moe_routing_stats on the routing tensors `r` of a forward(routing=True) call;
        returns device tensors stats [MOE_NUM_STATS] fp64, top3 [3] int32 (and prob_mean [N])."""
        import torch
        out = dict(stats=torch.empty(MOE_NUM_STATS, dtype=torch.float64, device=self.device),
                   top3=torch.empty(3, dtype=torch.int32, device=self.device))
        if with_prob_mean:
            out["prob_mean"] = torch.empty(self.desc.N, dtype=torch.float64, device=self.device)
        moe_routing_stats(self.desc, r["logits"], r["idx"], r["counts"], out["stats"], out["top3"], self.ws,
                          alpha=alpha, prob_mean=out.get("prob_mean"))
        return out

    def forward(self, x, routing: bool = False, y=None, out_routing: Optional[Dict] = None, events=None):
        import torch
        if y is None:
            y = torch.empty((self.desc.T, self.desc.d), dtype=self.dtype, device=self.device)
        r = out_routing if out_routing is not None else (self.routing_buffers() if routing else None)
        if self.qweights is not None:
            moe_layer_forward_q4(self.desc, self.qweights, x, y, r, self.ws, events=events)
        else:
            moe_layer_forward(self.desc, self.weights, x, y, r, self.ws, events=events)
        return (y, r) if r is not None else y
