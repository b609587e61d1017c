"""The two oracle implementations against each other on random small layers.

The plain C++ oracle (oracle/moe_oracle.cpp) and the NumPy one (oracle.moe_oracle) are written
independently and each is pinned by tests/test_oracle_pins.py; here they must agree on every
layer shape and option the GPU path supports: routing, capacity and grouping bit for bit (on the
same float64 logits), logits and outputs to float64 rounding.  Inputs are drawn in bf16 (read in
place by the C++ oracle, converted exactly for the NumPy one) and in float64.
"""
import numpy as np
import pytest
import torch

import oracle as O
import oracle.cpp as OC

CASES = [
    # T, d, N, k, d_ff, ffn, gating, capacity_factor, shared, bias
    (40, 16, 8, 2, 24, O.SWIGLU, O.TOPK_SOFTMAX, 0.0, False, False),
    (33, 32, 16, 4, 16, O.RELU2, O.SOFTMAX_TOPK, 0.0, True, False),
    (60, 16, 8, 2, 8, O.SWIGLU, O.TOPK_SOFTMAX, 1.0, False, True),
    (50, 8, 32, 3, 8, O.SWIGLU, O.SOFTMAX_TOPK, 0.5, True, True),     # drops: N*C < T*k
    (1, 8, 4, 4, 8, O.RELU2, O.TOPK_SOFTMAX, 0.0, False, False),
    (25, 8, 1, 1, 16, O.SWIGLU, O.TOPK_SOFTMAX, 0.0, True, False),
]


def _layer(rng, T, d, N, k, d_ff, ffn, shared, bias):
    g = torch.Generator().manual_seed(int(rng.integers(1 << 30)))

    def rnd(*shape, std=1.0):
        return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)
    x = rnd(T, d)
    wr = rnd(d, N, std=d ** -0.5)
    wg = rnd(N, d, d_ff, std=d ** -0.5) if ffn == O.SWIGLU else None
    wu = rnd(N, d, d_ff, std=d ** -0.5)
    wd = rnd(N, d_ff, d, std=d_ff ** -0.5)
    sh = None
    if shared:
        sh = (rnd(d, d_ff, std=d ** -0.5) if ffn == O.SWIGLU else None, rnd(d, d_ff, std=d ** -0.5),
              rnd(d_ff, d, std=d_ff ** -0.5))
    b = (-2.0 * np.log(np.arange(N) + 1.0)).astype(np.float32) if bias else None
    return x, wr, wg, wu, wd, sh, b


def _f64(t):
    return None if t is None else t.to(torch.float64).numpy()


@pytest.mark.parametrize("case", CASES)
def test_cpp_and_numpy_oracles_agree(case):
    T, d, N, k, d_ff, ffn, gating, cf, shared, bias = case
    rng = np.random.default_rng(100 + CASES.index(case))
    x, wr, wg, wu, wd, sh, b = _layer(rng, T, d, N, k, d_ff, ffn, shared, bias)
    c = OC.forward(x, wr, wu, wd, k, ffn, gating, w_gate=wg, logit_bias=b, capacity_factor=cf, shared=sh)
    n = O.forward(_f64(x), _f64(wr), _f64(wu), _f64(wd), k, ffn, gating, w_gate=_f64(wg), logit_bias=b,
                  capacity_factor=cf, shared=None if sh is None else tuple(_f64(t) for t in sh), z=c["z"])
    zn = O.router_logits(_f64(x), _f64(wr), b)
    assert np.allclose(c["z"], zn, rtol=1e-13, atol=1e-13)
    for key in ("idx", "counts", "offsets", "perm", "inv"):
        assert np.array_equal(c[key], n[key]), key
    assert c["C"] == n["C"]
    assert np.allclose(c["w"], n["w"], rtol=1e-13, atol=1e-15)
    assert np.allclose(c["y"], n["y"], rtol=1e-11, atol=1e-12)
    # a token subset gives the same rows
    sub = [T - 1, 0] if T > 1 else [0]
    cs = OC.forward(x, wr, wu, wd, k, ffn, gating, w_gate=wg, logit_bias=b, capacity_factor=cf, shared=sh,
                    tokens=sub)
    assert np.array_equal(cs["y"], c["y"][sub])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(3)
    x, wr, wg, wu, wd, sh, b = _layer(rng, 64, 16, 8, 2, 32, O.SWIGLU, True, True)
    outs = []
    for th in (1, 3, OC.max_threads()):
        OC.set_threads(th)
        outs.append(OC.forward(x, wr, wu, wd, 2, O.SWIGLU, O.TOPK_SOFTMAX, w_gate=wg, logit_bias=b,
                               capacity_factor=1.0, shared=sh))
    for o in outs[1:]:
        for key in ("z", "idx", "w", "perm", "y"):
            assert np.array_equal(o[key], outs[0][key]), key
