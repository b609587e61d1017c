"""GPU parity of the int4 expert weights.

The quantisation kernel must give the oracle's codes and scales bit for bit
(both decide them in fp32).  A layer with int4 experts must match the
oracle's forward with the weights the codes stand for (scale * q, float64),
to the bf16 layers' bar.  Small layers use a selection router (exact logits,
so every token is routed alike and compared); the full Mixtral-shaped decode
layer is checked on every token, as the bf16 full-size layers are."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_48_amd as M
import oracle as O
import workloads as W
from gpu_harness import check_routing, check_y, desc_of, f64, log, routing_to_np

pytestmark = pytest.mark.gpu


def _gpu_quantize(w):
    n, K, rows = w.shape                                        # x W orientation
    codes = torch.empty((n, rows, K // 8), dtype=torch.int32, device="cuda")
    scales = torch.empty((n, K // 128, rows), dtype=torch.float32, device="cuda")
    M.moe_quantize_q4(w, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy().view(np.uint32), scales.cpu().numpy()


def _oracle_codes(w2d):
    q, sc = O.quantize_q4(w2d)
    return O.pack_q4(q), sc


@pytest.mark.parametrize("shape,seed", [((2, 192, 256), 91), ((1, 64, 4096), 92), ((3, 40, 384), 93)])
def test_quantize_bit_exact(shape, seed):
    log(f"[q4 quantize] {shape}")
    cfg = W.LayerConfig("q", T=1, d=shape[2], N=shape[0], k=1, d_ff=shape[1], dtype="bf16", ffn=W.FFN_RELU2,
                        gating=W.GATE_TOPK_SOFTMAX, seed=seed)
    w = W.make_inputs(cfg, "cuda")["w_up"]                      # [N, d, d_ff] = [mats, K, rows]
    w[0, :, 3] = 0.0                                            # an all-zero column (all-zero groups)
    codes, scales = _gpu_quantize(w)
    wf = w.float().cpu().numpy()
    for m in range(shape[0]):
        oc, osc = _oracle_codes(wf[m])
        assert np.array_equal(codes[m], oc), m
        assert np.array_equal(scales[m], osc.T), m


def test_quantize_ties_and_grid():
    # amax 7 -> scale 1: halves round to even; values on the grid come back exactly
    w = torch.zeros((1, 128, 2), dtype=torch.bfloat16, device="cuda")      # [K, rows]
    vals = [7.0, 2.5, -0.5, 3.5, -2.5, 1.5, -7.0, 0.5]
    w[0, :8, 0] = torch.tensor(vals)
    w[0, :, 1] = 0.375
    codes, scales = _gpu_quantize(w)
    oc, osc = _oracle_codes(w[0].float().cpu().numpy())
    assert np.array_equal(codes[0], oc) and np.array_equal(scales[0], osc.T)
    q = O.unpack_q4(codes[0], 128)
    assert q[0, :8].tolist() == [7, 2, 0, 4, -2, 2, -7, 0]
    assert q[1].tolist() == [7] * 128


class QExpertView:
    """Index -> one expert's dequantised weights (the oracle quantises the bf16 weights itself),
    computed on each access and not kept."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        q, sc = O.quantize_q4(self.t[int(e)].float().cpu().numpy())
        return O.dequantize_q4(q, sc)


def _oracle_q4_forward(cfg, inp, tokens=None, z=None):
    def dq(t):
        q, sc = O.quantize_q4(t.float().cpu().numpy())
        return O.dequantize_q4(q, sc)
    shared = None
    if cfg.has_shared:
        shared = (None if inp["sh_gate"] is None else dq(inp["sh_gate"]), dq(inp["sh_up"]), dq(inp["sh_down"]))
    return O.forward(f64(inp["x"]), f64(inp["w_router"]), QExpertView(inp["w_up"]), QExpertView(inp["w_down"]),
                     cfg.k, O.SWIGLU if cfg.ffn == W.FFN_SWIGLU else O.RELU2,
                     O.TOPK_SOFTMAX if cfg.gating == W.GATE_TOPK_SOFTMAX else O.SOFTMAX_TOPK,
                     w_gate=QExpertView(inp["w_gate"]) if inp["w_gate"] is not None else None,
                     logit_bias=None if inp["logit_bias"] is None else inp["logit_bias"].cpu().numpy(),
                     capacity_factor=cfg.capacity_factor, shared=shared, tokens=tokens, z=z)


LC = W.LayerConfig
SMALL = {
    "q4_decode_swiglu": (LC("q4_decode_swiglu", T=16, d=256, N=8, k=2, d_ff=384, dtype="bf16", ffn=W.FFN_SWIGLU,
                            gating=W.GATE_TOPK_SOFTMAX, seed=101), False),
    "q4_relu_shared": (LC("q4_relu_shared", T=24, d=128, N=16, k=2, d_ff=256, dtype="bf16", ffn=W.FFN_RELU2,
                          gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=102), False),
    "q4_many_rows": (LC("q4_many_rows", T=100, d=128, N=4, k=2, d_ff=128, dtype="bf16", ffn=W.FFN_SWIGLU,
                        gating=W.GATE_TOPK_SOFTMAX, seed=103), False),
    "q4_capacity": (LC("q4_capacity", T=64, d=128, N=16, k=2, d_ff=256, dtype="bf16", ffn=W.FFN_SWIGLU,
                       gating=W.GATE_TOPK_SOFTMAX, capacity_factor=1.0, seed=104), True),
    "q4_n256_shared": (LC("q4_n256_shared", T=8, d=256, N=256, k=8, d_ff=128, dtype="bf16", ffn=W.FFN_SWIGLU,
                          gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=105), False),
    "q4_odd_groups": (LC("q4_odd_groups", T=16, d=384, N=8, k=2, d_ff=640, dtype="bf16", ffn=W.FFN_SWIGLU,
                         gating=W.GATE_TOPK_SOFTMAX, seed=106), True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_q4_layer_small(name):
    cfg, grid_bias = SMALL[name]
    log(f"[{name}] T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} d_ff={cfg.d_ff} {cfg.ffn} shared={cfg.has_shared}")
    inp = W.make_selection_router_inputs(cfg, "cuda", levels=16, grid_bias=grid_bias)
    qw = M.quantize_weights_q4(inp)
    layer = M.MoELayer(desc_of(cfg), inp, qweights=qw)
    y, r = layer.forward(inp["x"], routing=True)
    torch.cuda.synchronize()
    ref = _oracle_q4_forward(cfg, inp)
    assert np.array_equal(r["idx"].cpu().numpy(), ref["idx"])
    check_y(cfg, f64(y), ref["y"])
    # the stage entry point on the same routing, gate weights applied by the combine
    rows = cfg.T * cfg.k + (cfg.T if cfg.has_shared else 0)
    yp = torch.empty((rows, cfg.d), dtype=torch.float32, device="cuda")
    M.moe_expert_ffn_q4(layer.desc, qw, inp["x"], r["perm"], r["offsets"], None, yp, layer.ws)
    y2 = torch.empty_like(y)
    M.moe_combine(layer.desc, yp, r["inv"], r["w"], y2)
    torch.cuda.synchronize()
    check_y(cfg, f64(y2), ref["y"], label=" (stage entry points):")


def test_q4_mixtral_decode_full_size():
    cfg = W.CONFIGS["mixtral_decode"]
    log(f"[q4 {cfg.name}] T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} d_ff={cfg.d_ff}")
    inp = W.make_inputs(cfg, "cuda")
    qw = M.quantize_weights_q4(inp)
    layer = M.MoELayer(desc_of(cfg), inp, qweights=qw)
    y, r = layer.forward(inp["x"], routing=True)
    torch.cuda.synchronize()
    rn = routing_to_np(r)
    z64, zerr, alike = check_routing(cfg, inp, rn)
    # codes of one full expert matrix, bit for bit
    codes = qw["w_gate_codes"][0].cpu().numpy().view(np.uint32)
    oc, osc = _oracle_codes(inp["w_gate"][0].float().cpu().numpy())
    assert np.array_equal(codes, oc) and np.array_equal(qw["w_gate_scales"][0].cpu().numpy(), osc.T)
    ref = _oracle_q4_forward(cfg, inp, z=z64)
    check_y(cfg, f64(y)[alike], ref["y"][alike], label=f" all {int(alike.sum())} of {cfg.T} tokens routed alike:")
