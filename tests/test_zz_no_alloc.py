"""The allocation-free forward, moe_layer_forward_noalloc, against moe_layer_forward.

The entry point runs the same kernels as moe_layer_forward on the library's built-in per-GPU
workspace, so its outputs must equal moe_layer_forward's bit for bit: y and every routing
tensor, on two calls in a row (the second with fewer tokens, on the workspace the first left
behind), for a plain top-2 layer, a capacity layer and a layer with a shared expert.  Layers
whose workspace exceeds the built-in array are rejected on the host before anything is enqueued.
"""
import ctypes
import os
import re

import pytest
import torch

import mixture_experts_layer_48_amd as M
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000   # never dereferenced: the calls below that use it fail validation on the host


def _desc(cfg, T=None):
    return M.make_desc(cfg.T if T is None else T, cfg.d, cfg.N, cfg.k, cfg.d_ff, cfg.dtype, cfg.ffn, cfg.gating,
                       cfg.capacity_factor, cfg.has_shared)


def test_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == M.MOE_NOALLOC_SCRATCH_BYTES


def test_too_large_layer_is_rejected_on_the_host():
    lib = M.load_library()
    cfg = W.CONFIGS["mixtral_prefill"]
    desc = _desc(cfg)
    assert M.moe_workspace_size(desc) > M.MOE_NOALLOC_SCRATCH_BYTES
    wt = M.moe_weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    r = M.moe_routing()
    assert lib.moe_layer_forward_noalloc(ctypes.byref(desc), ctypes.byref(wt), FAKE, FAKE, ctypes.byref(r),
                                         None) == M.MOE_ERR_UNSUPPORTED
    assert b"built-in scratch" in lib.moe_last_error()
    # argument errors come first, as in moe_layer_forward
    bad = M.make_desc(16, 4096, 8, 9, 14336)
    assert lib.moe_layer_forward_noalloc(ctypes.byref(bad), ctypes.byref(wt), FAKE, FAKE, ctypes.byref(r),
                                         None) == M.MOE_ERR_INVALID_ARG
    # the decode batch of the same layer fits
    assert M.moe_workspace_size(_desc(cfg, T=16)) <= M.MOE_NOALLOC_SCRATCH_BYTES
    assert M.moe_workspace_size(_desc(cfg, T=256)) <= M.MOE_NOALLOC_SCRATCH_BYTES


CASES = {
    "decode_top2": W.CONFIGS["mixtral_decode"].replace(name="noalloc_decode", T=64, d=512, d_ff=1024),
    "capacity": W.CONFIGS["skewed_capacity"].replace(name="noalloc_capacity", T=600, d=256, N=32, d_ff=256),
    "shared": W.CONFIGS["deepseek_v3"].replace(name="noalloc_shared", T=300, d=256, d_ff=192),
}


def _equal(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


@pytest.mark.gpu
@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_forward_on_two_calls(name):
    cfg = CASES[name]
    inp = W.make_inputs(cfg, "cuda")
    for T in (cfg.T, cfg.T // 3):                    # the second call is smaller
        print(f"[noalloc {name}] T={T}", flush=True)
        desc = _desc(cfg, T)
        x = inp["x"][:T].contiguous()
        layer = M.MoELayer(desc, inp)
        y_ref, r_ref = layer.forward(x, routing=True)
        y = torch.full_like(y_ref, 7.0)
        r = layer.routing_buffers()
        M.moe_layer_forward_noalloc(desc, inp, x, y, r)
        torch.cuda.synchronize()
        assert _equal(y, y_ref), T
        for key in ("logits", "idx", "w", "counts", "offsets", "inv"):
            assert torch.equal(r[key], r_ref[key]), (T, key)
        n = int(r_ref["offsets"][-1])
        assert torch.equal(r["perm"][:n], r_ref["perm"][:n]), T
        del layer


@pytest.mark.gpu
def test_noalloc_on_a_side_stream_and_without_routing_outputs():
    cfg = CASES["decode_top2"]
    inp = W.make_inputs(cfg, "cuda")
    desc = _desc(cfg)
    layer = M.MoELayer(desc, inp)
    y_ref = layer.forward(inp["x"])
    side = torch.cuda.Stream()
    y = torch.empty_like(y_ref)
    torch.cuda.synchronize()
    M.moe_layer_forward_noalloc(desc, inp, inp["x"], y, None, stream=side)
    side.synchronize()
    assert _equal(y, y_ref)
