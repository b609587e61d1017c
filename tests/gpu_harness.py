"""Shared helpers of the GPU parity tests: build a layer on the GPU from a
seeded workload, run it through the C ABI, and hand the same input values to
the CPU oracle (one expert at a time, converted to float64 on demand)."""
from __future__ import annotations

import math
import sys
from typing import Dict

import numpy as np
import torch

import mixture_experts_layer_48_amd as M
import oracle as O
import workloads as W


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def desc_of(cfg: W.LayerConfig) -> M.moe_layer_desc:
    return M.make_desc(cfg.T, cfg.d, cfg.N, cfg.k, cfg.d_ff, cfg.dtype, cfg.ffn, cfg.gating,
                       cfg.capacity_factor, cfg.has_shared)


def check_shapes(cfg: W.LayerConfig, inp: Dict) -> None:
    """Host-side check that every operand matches what the kernels assume."""
    T, d, N, dff = cfg.T, cfg.d, cfg.N, cfg.d_ff
    assert inp["x"].shape == (T, d) and inp["x"].is_contiguous()
    assert inp["w_router"].shape == (N, d)
    assert inp["w_up"].shape == (N, dff, d) and inp["w_down"].shape == (N, d, dff)
    if cfg.ffn == W.FFN_SWIGLU:
        assert inp["w_gate"].shape == (N, dff, d)
    if cfg.has_shared:
        assert inp["sh_up"].shape == (dff, d) and inp["sh_down"].shape == (d, dff)
    for key, t in inp.items():
        if t is not None and key != "logit_bias":
            assert t.dtype == cfg.torch_dtype and t.is_contiguous(), key
    if cfg.dtype == "bf16":
        assert d % 64 == 0 and dff % 64 == 0


class ExpertView:
    """Index -> one expert's weights as a float64 numpy array (copied from the device lazily)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.cache: Dict[int, np.ndarray] = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].float().cpu().numpy().astype(np.float64)
        return self.cache[e]


def f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def run_layer(cfg: W.LayerConfig, inp: Dict, events=None):
    check_shapes(cfg, inp)
    layer = M.MoELayer(desc_of(cfg), inp)
    y, r = layer.forward(inp["x"], routing=True, events=events)
    torch.cuda.synchronize()
    return layer, y, r


def oracle_forward(cfg: W.LayerConfig, inp: Dict, tokens=None, z=None):
    shared = None
    if cfg.has_shared:
        shared = (None if inp["sh_gate"] is None else f64(inp["sh_gate"]), f64(inp["sh_up"]), f64(inp["sh_down"]))
    return O.forward(f64(inp["x"]), f64(inp["w_router"]), ExpertView(inp["w_up"]), ExpertView(inp["w_down"]),
                     cfg.k, O.SWIGLU if cfg.ffn == W.FFN_SWIGLU else O.RELU2,
                     O.TOPK_SOFTMAX if cfg.gating == W.GATE_TOPK_SOFTMAX else O.SOFTMAX_TOPK,
                     w_gate=ExpertView(inp["w_gate"]) if inp["w_gate"] is not None else None,
                     logit_bias=None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy(),
                     capacity_factor=cfg.capacity_factor, shared=shared, tokens=tokens, z=z)


def tolerance(cfg: W.LayerConfig) -> float:
    """Bar on |y_gpu - y_oracle| relative to RMS(y_oracle): 1e-4 for fp32 layers, 2e-2 for bf16."""
    return 1e-4 if cfg.dtype == "f32" else 2e-2


def rel_rms_err(y_gpu: np.ndarray, y_ref: np.ndarray) -> float:
    """max |y_gpu - y_ref| / RMS(y_ref) (the literal metric, always logged)."""
    rms = math.sqrt(float(np.mean(y_ref ** 2)))
    return float(np.max(np.abs(y_gpu - y_ref))) / max(rms, 1e-30)


def half_ulp(v: np.ndarray, mant_bits: int) -> np.ndarray:
    """Half a unit in the last place of |v| in a binary format with `mant_bits` fraction bits
    (7 for bf16, 23 for fp32): the most that rounding to that format can move v."""
    a = np.maximum(np.abs(v), np.finfo(np.float64).tiny)
    return np.exp2(np.floor(np.log2(a)) - mant_bits - 1)


def check_y(cfg: W.LayerConfig, y_gpu: np.ndarray, y_ref: np.ndarray, label: str = "") -> float:
    """|y_gpu - y_ref| <= tol * RMS(y_ref) + half an ulp of the output format, elementwise.

    The half ulp is the rounding of y to the layer's output dtype, which an exactly computed y
    also incurs; in bf16 it alone reaches 2^-8 |y|, i.e. above 2e-2 * RMS wherever
    |y| > 5.12 RMS, which these layers' outputs reach."""
    tol = tolerance(cfg)
    rms = math.sqrt(float(np.mean(y_ref ** 2)))
    mant = 23 if cfg.dtype == "f32" else 7
    allow = tol * rms + np.maximum(half_ulp(y_ref, mant), half_ulp(y_gpu, mant))
    excess = float(np.max(np.abs(y_gpu - y_ref) - allow))
    err = rel_rms_err(y_gpu, y_ref)
    log(f"[{cfg.name}]{label} max|y - y_oracle|/RMS = {err:.3e}; max|y|/RMS = "
        f"{float(np.max(np.abs(y_ref))) / rms:.2f}; worst margin to the bar = {-excess / rms:.3e} RMS")
    assert excess <= 0.0, f"{cfg.name}: error exceeds tol*RMS + half ulp by {excess / rms:.3e} RMS"
    return err


def routing_to_np(r: Dict) -> Dict[str, np.ndarray]:
    return {k: v.cpu().numpy() for k, v in r.items()}


def check_routing_exact_on_gpu_logits(cfg: W.LayerConfig, rn: Dict[str, np.ndarray]):
    """The GPU's integer routing equals the oracle's steps 2-4 applied to the GPU's own logits."""
    z = rn["logits"].astype(np.float64)
    C = O.expert_capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.N) if cfg.capacity_factor > 0 else 0
    gating = O.TOPK_SOFTMAX if cfg.gating == W.GATE_TOPK_SOFTMAX else O.SOFTMAX_TOPK
    idx, w = O.route_from_logits(z, cfg.k, gating, C)
    assert np.array_equal(rn["idx"], idx), "top-k / capacity indices differ on identical logits"
    assert np.max(np.abs(rn["w"] - w)) <= 1e-6, float(np.max(np.abs(rn["w"] - w)))
    counts, offsets, perm, inv = O.group_by_expert(idx, cfg.N)
    assert np.array_equal(rn["counts"], counts)
    assert np.array_equal(rn["offsets"], offsets)
    assert np.array_equal(rn["perm"][: offsets[-1]], perm)
    assert np.array_equal(rn["inv"], inv)
    return idx, w


def near_tie_depth(cfg: W.LayerConfig, idx: np.ndarray, z: np.ndarray) -> int:
    """Ranks whose order decides the routing: k + 1 without capacity; with capacity one past
    the deepest rank any slot took."""
    if cfg.capacity_factor <= 0:
        return cfg.k
    order = O.rank_experts(z)
    pos = np.argsort(order, axis=1)          # pos[t, e] = rank of e
    taken = np.where(idx >= 0, np.take_along_axis(pos, np.maximum(idx, 0), axis=1), 0)
    return int(taken.max()) + 1


def check_routing_vs_fp64(cfg: W.LayerConfig, inp: Dict, rn: Dict[str, np.ndarray], thr: float = 1e-6):
    """GPU routing vs the oracle's routing from float64 logits: identical except on near-tie
    tokens (gap between adjacent deciding ranks below thr), which are counted and reported."""
    z64 = O.router_logits(f64(inp["x"]), f64(inp["w_router"]),
                          None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy())
    zerr = float(np.max(np.abs(rn["logits"].astype(np.float64) - z64)))
    C = O.expert_capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.N) if cfg.capacity_factor > 0 else 0
    gating = O.TOPK_SOFTMAX if cfg.gating == W.GATE_TOPK_SOFTMAX else O.SOFTMAX_TOPK
    idx64, _ = O.route_from_logits(z64, cfg.k, gating, C)
    depth = near_tie_depth(cfg, idx64, z64)
    ties = set(O.near_tie_tokens(z64, depth, thr).tolist())
    diff = np.nonzero((rn["idx"] != idx64).any(axis=1))[0]
    if cfg.capacity_factor > 0 and diff.size:
        # with capacity a flipped near-tie can move later tokens too: everything from the first
        # near-tie token on is reported, nothing before it may differ
        first_tie = min(ties) if ties else cfg.T
        assert diff.min() >= first_tie, (diff[:10], sorted(ties)[:10])
        bad = []
    else:
        bad = [t for t in diff.tolist() if t not in ties]
    log(f"[{cfg.name}] max|z_gpu - z_fp64| = {zerr:.3e}; near-tie tokens (<{thr:g}) = {len(ties)}; "
        f"tokens routed differently = {diff.size}")
    assert not bad, f"tokens routed differently without a near tie: {bad[:10]}"
    return zerr, len(ties), int(diff.size)
