"""Seeded synthetic workloads for the sparse MoE layer forward.

This module is shared harness: it only draws inputs (tokens, router weights,
expert weights, the per-expert logit bias) and holds none of the layer's
arithmetic.  Both the CPU oracle's tests and the GPU path's tests, smoke run
and benchmark take their inputs from here, so the two sides see bit-identical
values.

Shapes come from the five layer configurations that the MoE pages describe in
prose (Mixtral-8x7B: 8 experts, top-2; DeepSeek-V3: 256 routed + 1 shared
expert, top-8; a 128-expert top-2 layer with an expert capacity of
capacity_factor 2.0).  The pages publish no dataset or trained weights for any
of them, so every tensor is drawn from a seeded Gaussian:

  x ~ N(0, 1);  router and input-side expert weights ~ N(0, 1/d);
  output-side expert weights ~ N(0, 1/d_ff);  values rounded to bf16 (RNE) on
  the bf16 layers and kept in fp32 on the fp32 layer.

The skewed layer adds a fixed per-expert logit bias b[e] = -2 ln(e + 1)
(a Zipf-like preference for low expert ids), computed in float64 and rounded
to fp32 once, so both sides read the same fp32 values.

Weight layout (the layout the C ABI takes, see include/moe.h): the x W
orientation of the configurations ("W_gate, W_up: d x d_ff; W_down: d_ff x d")
and of the pages' toy (router_W [d, N], x @ experts_W[e]), row-major:

  w_router [d, N]          z[t, e]   = sum_i x[t, i] * w_router[i, e]
  w_gate   [N, d, d_ff]    g[t, f]   = sum_i x[t, i] * w_gate[e, i, f]
  w_up     [N, d, d_ff]    u[t, f]   = sum_i x[t, i] * w_up[e, i, f]
  w_down   [N, d_ff, d]    y[t, o]   = sum_f h[t, f] * w_down[e, f, o]
  shared expert: sh_gate, sh_up [d, d_ff], sh_down [d_ff, d]

For the two-layer ReLU expert, w_up holds W1 and w_down holds W2; w_gate is
unused.

Random draws use torch's counter-based generator (Philox on the GPU, its CPU
generator on the host), one generator per tensor and per expert, seeded from
(config seed, tensor stream, expert).  Draws on the GPU and on the host give
different values for the same seed; a test that compares the two sides draws
once on the GPU and copies the values to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

# tensor streams (one generator stream per tensor)
STREAM_X, STREAM_ROUTER, STREAM_GATE, STREAM_UP, STREAM_DOWN = 1, 2, 3, 4, 5
STREAM_SH_GATE, STREAM_SH_UP, STREAM_SH_DOWN = 6, 7, 8
STREAM_GRID, STREAM_GRID_BIAS, STREAM_LOGITS, STREAM_TOKENS, STREAM_OWNER = 9, 10, 11, 12, 13

FFN_RELU2 = "relu2"
FFN_SWIGLU = "swiglu"
GATE_TOPK_SOFTMAX = "topk_softmax"     # top-k, then softmax over the k picked logits
GATE_SOFTMAX_TOPK = "softmax_topk"     # softmax over all N logits, then top-k, no renormalisation


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int                  # tokens (rows of x)
    d: int                  # model width
    N: int                  # routed experts
    k: int                  # experts per token
    d_ff: int               # expert hidden width
    dtype: str              # "f32" or "bf16": weights and activations
    ffn: str                # FFN_RELU2 or FFN_SWIGLU
    gating: str             # GATE_TOPK_SOFTMAX or GATE_SOFTMAX_TOPK
    capacity_factor: float = 0.0   # <= 0: unlimited
    has_shared: bool = False       # one shared expert applied to every token, weight 1
    zipf_bias: bool = False        # per-expert logit bias b[e] = -2 ln(e + 1)
    seed: int = 0

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


CONFIGS: Dict[str, LayerConfig] = {
    # tiny fp32 layer: 8 experts, top-2, two-layer ReLU experts d -> 256 -> d
    "tiny_fp32": LayerConfig("tiny_fp32", T=128, d=64, N=8, k=2, d_ff=256, dtype="f32",
                             ffn=FFN_RELU2, gating=GATE_TOPK_SOFTMAX, seed=1001),
    # Mixtral-8x7B-shaped layer, prefill batch
    "mixtral_prefill": LayerConfig("mixtral_prefill", T=4096, d=4096, N=8, k=2, d_ff=14336,
                                   dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_TOPK_SOFTMAX,
                                   seed=1002),
    # same layer, decode-sized batch
    "mixtral_decode": LayerConfig("mixtral_decode", T=16, d=4096, N=8, k=2, d_ff=14336,
                                  dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_TOPK_SOFTMAX,
                                  seed=1003),
    # DeepSeek-V3-shaped fine-grained layer: 256 routed + 1 shared, top-8 of a full softmax
    "deepseek_v3": LayerConfig("deepseek_v3", T=8192, d=7168, N=256, k=8, d_ff=2048,
                               dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_SOFTMAX_TOPK,
                               has_shared=True, seed=1004),
    # skewed routing with expert capacity ceil(2.0 * T * k / N)
    "skewed_capacity": LayerConfig("skewed_capacity", T=16384, d=3584, N=128, k=2, d_ff=2560,
                                   dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_TOPK_SOFTMAX,
                                   capacity_factor=2.0, zipf_bias=True, seed=1005),
    # Routing variants the pages name without layer widths (those are taken from the layers
    # above): top-1 over 128 experts with two-layer ReLU experts (Switch-style), top-1 over 16
    # SwiGLU experts (Llama 4 Scout-style), one shared expert plus top-7 of 256 routed ones
    # (the DeepSeek-V4 description: 8 active experts, the shared one included), and top-1
    # over 128 SwiGLU experts.
    "switch_top1": LayerConfig("switch_top1", T=4096, d=4096, N=128, k=1, d_ff=14336,
                               dtype="bf16", ffn=FFN_RELU2, gating=GATE_TOPK_SOFTMAX, seed=1006),
    "scout_top1": LayerConfig("scout_top1", T=4096, d=4096, N=16, k=1, d_ff=14336,
                              dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_TOPK_SOFTMAX, seed=1007),
    "v4_shared_top7": LayerConfig("v4_shared_top7", T=8192, d=7168, N=256, k=7, d_ff=2048,
                                  dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_SOFTMAX_TOPK,
                                  has_shared=True, seed=1008),
    # 128 experts with the 16-expert layer's active size per token (Llama 4 Maverick-style: the
    # page gives 128 experts per layer and the same active parameters as the top-1 16-expert
    # layer, read here as top-1 over 128 SwiGLU experts of the same width)
    "maverick_top1": LayerConfig("maverick_top1", T=4096, d=4096, N=128, k=1, d_ff=14336,
                                 dtype="bf16", ffn=FFN_SWIGLU, gating=GATE_TOPK_SOFTMAX, seed=1009),
}


def zipf_bias(N: int) -> torch.Tensor:
    """b[e] = -2 ln(e + 1), drawn once in float64 and rounded to fp32."""
    return torch.tensor([-2.0 * math.log(e + 1.0) for e in range(N)], dtype=torch.float64).float()


def _gen(device: torch.device, seed: int, stream: int, expert: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    # distinct, reproducible seed per (config, tensor, expert)
    g.manual_seed(((seed * 1009 + stream) * 1000003 + expert) & 0x7FFFFFFFFFFFFFFF)
    return g


def _normal(shape, std: float, dtype: torch.dtype, device, gen) -> torch.Tensor:
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(std)
    return v.to(dtype)


def make_inputs(cfg: LayerConfig, device="cpu", experts: Optional[range] = None) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer call on `device`.

    Returns a dict with x, w_router, logit_bias (or None), w_gate (None for
    ReLU), w_up, w_down and, when cfg.has_shared, sh_gate, sh_up, sh_down.
    Expert weights are drawn one expert at a time (bounded temporaries).
    """
    device = torch.device(device)
    dt = cfg.torch_dtype
    T, d, N, dff = cfg.T, cfg.d, cfg.N, cfg.d_ff
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, d), 1.0, dt, device, _gen(device, cfg.seed, STREAM_X))
    out["w_router"] = _normal((d, N), 1.0 / math.sqrt(d), dt, device, _gen(device, cfg.seed, STREAM_ROUTER))
    out["logit_bias"] = zipf_bias(N).to(device) if cfg.zipf_bias else None

    def expert_stack(stream, rows, cols, std):
        w = torch.empty((N, rows, cols), dtype=dt, device=device)
        for e in range(N):
            w[e].copy_(_normal((rows, cols), std, dt, device, _gen(device, cfg.seed, stream, e)))
        return w

    out["w_gate"] = expert_stack(STREAM_GATE, d, dff, 1.0 / math.sqrt(d)) if cfg.ffn == FFN_SWIGLU else None
    out["w_up"] = expert_stack(STREAM_UP, d, dff, 1.0 / math.sqrt(d))
    out["w_down"] = expert_stack(STREAM_DOWN, dff, d, 1.0 / math.sqrt(dff))
    if cfg.has_shared:
        out["sh_gate"] = (_normal((d, dff), 1.0 / math.sqrt(d), dt, device, _gen(device, cfg.seed, STREAM_SH_GATE))
                          if cfg.ffn == FFN_SWIGLU else None)
        out["sh_up"] = _normal((d, dff), 1.0 / math.sqrt(d), dt, device, _gen(device, cfg.seed, STREAM_SH_UP))
        out["sh_down"] = _normal((dff, d), 1.0 / math.sqrt(dff), dt, device, _gen(device, cfg.seed, STREAM_SH_DOWN))
    else:
        out["sh_gate"] = out["sh_up"] = out["sh_down"] = None
    return out


def make_selection_router_inputs(cfg: LayerConfig, device="cpu", levels: int = 16,
                                 grid_bias: bool = False) -> Dict[str, torch.Tensor]:
    """Inputs of one layer call whose router logits are exact in any summation order.

    As make_inputs, except: column e of w_router is the unit vector on input feature e, so that
    logit z[t, e] is x[t, e] itself; x[t, :N] takes values k/8 for integer k drawn uniformly
    from [-levels/2, levels/2) (few distinct values: many exactly tied logits); with
    grid_bias, logit_bias[e] is a multiple of 1/4 in [-1, 1] (the sum with x stays exact in
    fp32).  Needs d >= N."""
    if cfg.d < cfg.N:
        raise ValueError("a selection router needs d >= N")
    device = torch.device(device)
    out = make_inputs(cfg, device)
    g = _gen(device, cfg.seed, STREAM_GRID)
    steps = torch.randint(-(levels // 2), levels - levels // 2, (cfg.T, cfg.N), generator=g, device=device)
    out["x"][:, :cfg.N] = (steps.float() / 8.0).to(out["x"].dtype)
    wr = torch.zeros((cfg.d, cfg.N), dtype=out["x"].dtype, device=device)
    wr[torch.arange(cfg.N, device=device), torch.arange(cfg.N, device=device)] = 1.0
    out["w_router"] = wr
    if grid_bias:
        gb = _gen(device, cfg.seed, STREAM_GRID_BIAS)
        out["logit_bias"] = torch.randint(-4, 5, (cfg.N,), generator=gb, device=device).float() / 4.0
    return out


def make_logits(T: int, N: int, seed: int, device="cpu", levels: Optional[int] = None) -> torch.Tensor:
    """Router logits [T, N] fp32 for the routing-statistics cases: N(0, 1) draws, or with
    `levels`, values k/8 for integer k uniform in [-levels/2, levels/2) (exact ties)."""
    device = torch.device(device)
    g = _gen(device, seed, STREAM_LOGITS)
    if levels is None:
        return torch.randn((T, N), generator=g, device=device, dtype=torch.float32)
    return torch.randint(-(levels // 2), levels - levels // 2, (T, N), generator=g, device=device).float() / 8.0


def make_tokens(T: int, d: int, dtype: str, seed: int, device="cpu", grid_cols: int = 0,
                levels: int = 16) -> torch.Tensor:
    """One rank's tokens x [T, d] ~ N(0, 1) in `dtype`; with grid_cols, columns :grid_cols take
    values k/8 for integer k uniform in [-levels/2, levels/2) (for a selection router)."""
    device = torch.device(device)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = _normal((T, d), 1.0, dt, device, _gen(device, seed, STREAM_TOKENS))
    if grid_cols:
        g = _gen(device, seed, STREAM_GRID)
        steps = torch.randint(-(levels // 2), levels - levels // 2, (T, grid_cols), generator=g, device=device)
        x[:, :grid_cols] = (steps.float() / 8.0).to(dt)
    return x


def make_owner_map(N: int, G: int, kind: str = "contiguous", seed: int = 0):
    """Expert -> rank map of an expert-parallel placement: "contiguous" (rank r owns a block of
    about N/G experts), "interleaved" (expert e on rank e % G) or "random" (uniform ranks,
    seeded; a rank may own none)."""
    if kind == "contiguous":
        return [e * G // N for e in range(N)]
    if kind == "interleaved":
        return [e % G for e in range(N)]
    g = _gen(torch.device("cpu"), seed, STREAM_OWNER)
    return [int(v) for v in torch.randint(0, G, (N,), generator=g)]


def scaled(cfg: LayerConfig, **kw) -> LayerConfig:
    """A copy of `cfg` with some sizes changed (parity cases at reduced sizes)."""
    return cfg.replace(**kw)
