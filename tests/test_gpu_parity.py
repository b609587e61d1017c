"""GPU parity: the HIP path through the C ABI against the float64 CPU oracle.

Layered checks.  The oracle only ever sees the seeded inputs, never a value the
GPU computed.  Routing is integer work decided by floating point:
  P-a  exact logits: with a selection router (router rows are unit vectors and
       the selected inputs lie on a coarse grid, so every logit is exact in any
       summation order, with many exact ties) the GPU's logits, top-k /
       capacity indices, counts, offsets, perm and inv equal the oracle's bit
       for bit, and the gate weights agree within 1e-6;
  P-b  random routers: the GPU logits are within the error bound of their fp32
       chunked accumulation, the grouping is the stable grouping of the GPU's
       own indices (properties), and the routing equals the oracle's from its
       float64 logits except on near-tie tokens (adjacent deciding logits
       closer than 1e-6), which are counted and printed;
  P-c  y matches the oracle's forward on its own routing, on every token routed
       alike: max |err| / RMS(y) within 1e-4 (fp32 layers) or 2e-2 (bf16
       layers), plus half an ulp of the output format;
  P-d  routing statistics of the GPU's routing against the oracle's statistics
       of its own routing.
Every case, the full-size layers included, compares every token's output
(the tokens routed alike: all of them but counted near ties); small cases span
several tiles with ragged tails.
"""
import gc

import numpy as np
import pytest
import torch

import mixture_experts_layer_48_amd as M
import oracle as O
import workloads as W
from gpu_harness import (check_routing, check_stats, check_y, f64, gpu_routing_stats, h_rounding_bound, log,
                         oracle_forward, rel_rms_err, routing_to_np, run_layer, desc_of)

pytestmark = pytest.mark.gpu

C = W.CONFIGS
SMALL = {
    "tiny_fp32": C["tiny_fp32"],
    "mixtral_small": C["mixtral_prefill"].replace(name="mixtral_small", T=300, d=256, d_ff=384),
    "mixtral_decode_small": C["mixtral_decode"].replace(name="mixtral_decode_small", d=256, d_ff=384),
    "deepseek_small": C["deepseek_v3"].replace(name="deepseek_small", T=260, d=128, d_ff=192),
    "skewed_small": C["skewed_capacity"].replace(name="skewed_small", T=1000, d=128, N=32, d_ff=128),
    "relu_bf16": W.LayerConfig("relu_bf16", T=200, d=128, N=8, k=3, d_ff=192, dtype="bf16",
                               ffn=W.FFN_RELU2, gating=W.GATE_TOPK_SOFTMAX, seed=7),
    "swiglu_f32_shared": W.LayerConfig("swiglu_f32_shared", T=50, d=40, N=5, k=2, d_ff=24, dtype="f32",
                                       ffn=W.FFN_SWIGLU, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=8),
    "dense_k_eq_n": W.LayerConfig("dense_k_eq_n", T=70, d=64, N=4, k=4, d_ff=64, dtype="bf16",
                                  ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=9),
    "single_expert": W.LayerConfig("single_expert", T=33, d=64, N=1, k=1, d_ff=128, dtype="bf16",
                                   ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=10),
    "capacity_drops": W.LayerConfig("capacity_drops", T=100, d=64, N=4, k=2, d_ff=64, dtype="bf16",
                                    ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=0.25,
                                    zipf_bias=True, seed=11),
    "one_token": W.LayerConfig("one_token", T=1, d=64, N=8, k=2, d_ff=64, dtype="bf16",
                               ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=12),
    "relu_shared_modeb": W.LayerConfig("relu_shared_modeb", T=130, d=64, N=16, k=4, d_ff=128, dtype="bf16",
                                       ffn=W.FFN_RELU2, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=13),
    # >= 512 rows per expert: the large-tile GEMM configuration, with partial n-tiles
    "big_tiles_swiglu": W.LayerConfig("big_tiles_swiglu", T=700, d=128, N=2, k=2, d_ff=384, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=15),
    "big_tiles_relu": W.LayerConfig("big_tiles_relu", T=600, d=320, N=2, k=2, d_ff=320, dtype="bf16",
                                    ffn=W.FFN_RELU2, gating=W.GATE_TOPK_SOFTMAX, seed=16),
    # long out-projection K: the down projection runs as two K parts summed by the combine
    "split_k_out": W.LayerConfig("split_k_out", T=200, d=128, N=2, k=2, d_ff=8192, dtype="bf16",
                                 ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=17),
    # 256-row tiles at real-model K (a multiple of 256): several m-tiles and a short last one;
    # ReLU with a shared expert; a partial last column tile of the in-projection
    "tiles256_swiglu": W.LayerConfig("tiles256_swiglu", T=600, d=256, N=2, k=2, d_ff=512, dtype="bf16",
                                   ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=21),
    "tiles256_relu_shared": W.LayerConfig("tiles256_relu_shared", T=400, d=512, N=2, k=1, d_ff=768, dtype="bf16",
                                        ffn=W.FFN_RELU2, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=22),
    "tiles256_ragged_cols": W.LayerConfig("tiles256_ragged_cols", T=300, d=256, N=1, k=1, d_ff=448, dtype="bf16",
                                        ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=23),
    # 224-288 rows per expert on average: 320-row in-projection tiles.  Loads 253/255/255/277
    # and a 520-row shared expert (a 320-row and a 200-row tile); then skewed loads
    # 982/638/271/92/32/9/21/3 (full 320-row tiles, a 318-row one, 96-, 64- and 32-row ones)
    "tiles320_swiglu_shared": W.LayerConfig("tiles320_swiglu_shared", T=520, d=256, N=4, k=2, d_ff=320,
                                            dtype="bf16", ffn=W.FFN_SWIGLU, gating=W.GATE_SOFTMAX_TOPK,
                                            has_shared=True, seed=24),
    "tiles320_skewed": W.LayerConfig("tiles320_skewed", T=1024, d=128, N=8, k=2, d_ff=192, dtype="bf16",
                                     ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, zipf_bias=True, seed=25),
    # 320-row out-projection tiles with the long K split in two parts
    "split_k_tiles320": W.LayerConfig("split_k_tiles320", T=256, d=128, N=2, k=2, d_ff=8192, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=28),
    # about 256 rows per expert (195-298, 320-row tiles), more tiles than resident blocks: blocks
    # run several tiles in a row and each tile's last stages load the next tile's first ones;
    # every token is checked
    "multi_tile_blocks": W.LayerConfig("multi_tile_blocks", T=4096, d=512, N=32, k=2, d_ff=2048, dtype="bf16",
                                       ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=27),
    # 512 rows per expert: 256-row out-projection tiles, 512 of them, so every block claims
    # several in a row (its XCD range's counter, then the other XCDs' ranges), decoded from the
    # tile table; K of 4 stages (the next tile's first stages loaded by the current tile's last
    # ones) and of 3 (no chaining: the next tile loaded after a barrier)
    "claimed_out_chain": W.LayerConfig("claimed_out_chain", T=4096, d=4096, N=16, k=2, d_ff=256, dtype="bf16",
                                       ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=29),
    "claimed_out_nochain": W.LayerConfig("claimed_out_nochain", T=4096, d=4096, N=16, k=2, d_ff=192, dtype="bf16",
                                         ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=30),
    # capacity with 256 experts: scans that run past the ranked-list window kept in LDS (picks
    # deeper than 64 ranks), with slots dropped once every expert is full, and without drops
    "capacity_deep_drops": W.LayerConfig("capacity_deep_drops", T=300, d=64, N=256, k=2, d_ff=64, dtype="bf16",
                                         ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=0.5,
                                         zipf_bias=True, seed=24),
    "capacity_deep_n256": W.LayerConfig("capacity_deep_n256", T=2000, d=64, N=256, k=2, d_ff=64, dtype="bf16",
                                        ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=1.0,
                                        zipf_bias=True, seed=25),
    # fine-grained routing (8 of 64 experts, softmax over all of them) beside a shared expert: the
    # fused forward keeps the routed rows of the down projection in bf16 and the shared expert's in
    # fp32; about 75, 208 and 256 rows per expert take the 128-, 256- and 320-row out-projection
    # tiles
    "fine_shared_t128": W.LayerConfig("fine_shared_t128", T=600, d=128, N=64, k=8, d_ff=192, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=41),
    "fine_shared_t256": W.LayerConfig("fine_shared_t256", T=1664, d=128, N=64, k=8, d_ff=256, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=42),
    "fine_shared_t320": W.LayerConfig("fine_shared_t320", T=2048, d=256, N=64, k=8, d_ff=320, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=43),
    # 16384 slots with capacity drops: the grouping over many blocks (drops left out of every
    # expert's rows)
    "capacity_drops_many": W.LayerConfig("capacity_drops_many", T=8192, d=64, N=64, k=2, d_ff=64, dtype="bf16",
                                         ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=0.5,
                                         zipf_bias=True, seed=45),
    # 512 slots (128 tokens x top-4 of 32 experts, a logit bias): the routing finished in one block
    "finish_limits": W.LayerConfig("finish_limits", T=128, d=256, N=32, k=4, d_ff=192, dtype="bf16",
                                   ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, zipf_bias=True, seed=44),
    # at most 16 routed rows per expert on average: the weight-streaming decode GEMMs, here with a
    # shared expert longer than one 16-row tile, heavy experts, and capacity drops
    "skinny_relu_shared": W.LayerConfig("skinny_relu_shared", T=24, d=128, N=16, k=2, d_ff=192, dtype="bf16",
                                        ffn=W.FFN_RELU2, gating=W.GATE_SOFTMAX_TOPK, has_shared=True, seed=18),
    "skinny_skewed": W.LayerConfig("skinny_skewed", T=100, d=192, N=64, k=4, d_ff=128, dtype="bf16",
                                   ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, zipf_bias=True, seed=19),
    "skinny_capacity": W.LayerConfig("skinny_capacity", T=64, d=128, N=16, k=2, d_ff=256, dtype="bf16",
                                     ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=1.0,
                                     zipf_bias=True, seed=20),
    # the named routing variants at small widths: top-1 over 128 ReLU experts (about 23 rows
    # each, the 128-row tiles), top-1 over 16 SwiGLU experts, shared expert + top-7 of 256
    "switch_small": C["switch_top1"].replace(name="switch_small", T=3000, d=128, d_ff=256),
    "scout_small": C["scout_top1"].replace(name="scout_small", T=600, d=256, d_ff=384),
    "v4_small": C["v4_shared_top7"].replace(name="v4_small", T=260, d=128, d_ff=192),
    "maverick_small": C["maverick_top1"].replace(name="maverick_small", T=2000, d=128, d_ff=192),
}


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _stats_parity(cfg, layer, r, rn, z64, zerr, ref):
    g = gpu_routing_stats(layer, r)
    o = O.routing_stats(z64, ref["idx"], ref["counts"])
    slack = len(O.near_tie_tokens(z64, cfg.k, max(1e-6, 2.0 * zerr))) * cfg.k
    if not np.array_equal(rn["idx"], ref["idx"]):
        # counts differ where near-tie tokens went elsewhere: the count-based values are only
        # logged then
        log(f"[{cfg.name}] routing differs on near ties: statistics not compared")
        return g
    check_stats(cfg, g, o, zerr=zerr, reroute_slack=slack)
    return g


def _full_parity(cfg, inp):
    log(f"[{cfg.name}] T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} d_ff={cfg.d_ff} {cfg.dtype} {cfg.ffn} "
        f"{cfg.gating} cf={cfg.capacity_factor} shared={cfg.has_shared}")
    layer, y, r = run_layer(cfg, inp)
    rn = routing_to_np(r)
    z64, zerr, alike = check_routing(cfg, inp, rn)
    ref = oracle_forward(cfg, inp, z=z64)
    check_y(cfg, f64(y)[alike], ref["y"][alike], label=f" {int(alike.sum())} of {cfg.T} tokens:")
    _stats_parity(cfg, layer, r, rn, z64, zerr, ref)
    return layer, y, r


@pytest.mark.parametrize("name", list(SMALL))
def test_small_layer_parity(name):
    cfg = SMALL[name]
    inp = W.make_inputs(cfg, "cuda")
    _full_parity(cfg, inp)
    _free()


def test_all_tokens_to_one_expert():
    cfg = W.LayerConfig("all_to_one", T=600, d=64, N=8, k=2, d_ff=128, dtype="bf16", ffn=W.FFN_SWIGLU,
                        gating=W.GATE_TOPK_SOFTMAX, seed=14)
    inp = W.make_inputs(cfg, "cuda")
    inp["logit_bias"] = torch.tensor([40.0, 20.0] + [0.0] * 6, device="cuda")
    layer, y, r = _full_parity(cfg, inp)
    counts = r["counts"].cpu().numpy()
    assert counts[0] == 600 and counts[1] == 600 and counts[2:].sum() == 0
    _free()


@pytest.mark.parametrize("T", [700, 1024])
def test_small_experts_beside_the_tiled_gemm(T):
    # The gate/up projection runs routed experts with at most 64 rows as weight streams beside the
    # tiled GEMM (when experts average under 512 rows); here the loads sit at and around that
    # bound: 64, 65, 63, 1 and 0 rows, the rest on three large experts (128-row tiles at T=700,
    # 320-row tiles at T=1024).  A selection router (logit = x[t, e]) fixes each token's two
    # experts; every token is checked.
    cfg = W.LayerConfig(f"small_experts_{T}", T=T, d=128, N=8, k=2, d_ff=192, dtype="bf16", ffn=W.FFN_SWIGLU,
                        gating=W.GATE_TOPK_SOFTMAX, seed=31)
    inp = W.make_selection_router_inputs(cfg, "cuda")
    small = [64, 65, 63, 1]                              # experts 0-3; expert 4 gets none
    first = np.concatenate([np.full(n, e) for e, n in enumerate(small)] +
                           [5 + np.arange(T - sum(small)) % 3]).astype(np.int64)
    second = np.where(first >= 5, 5 + (first - 5 + 1) % 3, 5 + np.arange(T) % 3)
    x = inp["x"]
    x[:, :cfg.N] = -1.0
    x[torch.arange(T, device="cuda"), torch.as_tensor(first, device="cuda")] = 1.5
    x[torch.arange(T, device="cuda"), torch.as_tensor(second, device="cuda")] = 1.0
    inp["logit_bias"] = None
    layer, y, r = _full_parity(cfg, inp)
    counts = r["counts"].cpu().numpy()
    assert counts[:5].tolist() == [64, 65, 63, 1, 0], counts
    assert counts[5:].min() > 64, counts
    _free()


def test_large_batch():
    # 262144 tokens x top-2: half a million slots through the single-block grouping, the
    # router and the combine at scale (int32 row indexing well away from its limit)
    cfg = W.LayerConfig("large_batch", T=262144, d=64, N=16, k=2, d_ff=64, dtype="bf16", ffn=W.FFN_SWIGLU,
                        gating=W.GATE_TOPK_SOFTMAX, seed=26)
    inp = W.make_inputs(cfg, "cuda")
    layer, y, r = run_layer(cfg, inp)
    rn = routing_to_np(r)
    z64, zerr, alike = check_routing(cfg, inp, rn)
    ref = oracle_forward(cfg, inp, z=z64)
    # 262144 tokens reach |y| = 14.5 RMS, where the hidden state's bf16 rounding alone moves y by
    # more than 2e-2 RMS: the bar adds that rounding's elementwise bound
    extra = h_rounding_bound(cfg, inp, ref["idx"], ref["w"])
    check_y(cfg, f64(y)[alike], ref["y"][alike], label=f" {int(alike.sum())} of {cfg.T} tokens:",
            extra=extra[alike])
    del layer, y, r, inp
    _free()


def test_capacity_count_clears_do_not_change_routing(monkeypatch):
    # the capacity kernel stamps its proposal counts with the round number and clears them every
    # MOE_CAPACITY_ROUND_LIMIT rounds (0xFFFF by default); with a clear every 1, 2 or 3 rounds the
    # skewed layer's routing must be the same, bit for bit
    cfg = C["skewed_capacity"]
    inp = W.make_inputs(cfg, "cuda")
    layer, _, r_ref = run_layer(cfg, inp)
    for lim in ("1", "2", "3"):
        monkeypatch.setenv("MOE_CAPACITY_ROUND_LIMIT", lim)
        log(f"[capacity clears] every {lim} rounds")
        y, r = layer.forward(inp["x"], routing=True)
        torch.cuda.synchronize()
        for key in ("idx", "w", "counts", "offsets", "inv"):
            assert torch.equal(r[key], r_ref[key]), (lim, key)
    monkeypatch.delenv("MOE_CAPACITY_ROUND_LIMIT")
    for name in ("capacity_deep_drops", "skinny_capacity"):
        cfg = SMALL[name]
        inp = W.make_inputs(cfg, "cuda")
        layer, _, r_ref = run_layer(cfg, inp)
        monkeypatch.setenv("MOE_CAPACITY_ROUND_LIMIT", "1")
        y, r = layer.forward(inp["x"], routing=True)
        torch.cuda.synchronize()
        monkeypatch.delenv("MOE_CAPACITY_ROUND_LIMIT")
        for key in ("idx", "w", "counts", "inv"):
            assert torch.equal(r[key], r_ref[key]), (name, key)
    _free()


def test_deterministic_bitwise():
    for cfg in (SMALL["deepseek_small"], SMALL["skewed_small"], SMALL["mixtral_small"]):
        log(f"[determinism] {cfg.name}")
        inp = W.make_inputs(cfg, "cuda")
        layer, y1, r1 = run_layer(cfg, inp)
        y2, r2 = layer.forward(inp["x"], routing=True)
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16) if y1.dtype == torch.bfloat16 else y1,
                           y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2)
        for key in r1:
            assert torch.equal(r1[key], r2[key]), key
    _free()


def test_forward_on_a_side_stream():
    # every launch goes to the stream given: a forward enqueued on a side stream (default
    # priority), with the default stream idle and synchronised only through that stream's
    # completion, gives the default-stream result bit for bit
    cfg = SMALL["deepseek_small"]
    inp = W.make_inputs(cfg, "cuda")
    layer, y_ref, r_ref = run_layer(cfg, inp)
    side = torch.cuda.Stream()
    y = torch.empty_like(y_ref)
    r = layer.routing_buffers()
    torch.cuda.synchronize()
    M.moe_layer_forward(layer.desc, inp, inp["x"], y, r, layer.ws, stream=side)
    side.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    for key in ("idx", "counts", "perm", "inv"):
        assert torch.equal(r[key], r_ref[key]), key
    _free()


def test_forward_in_a_captured_graph():
    # the library allocates, clears and synchronises nothing, so a whole forward can be captured
    # into one graph; replays (with eager work and synchronisations between them) must all give
    # the eager result bit for bit
    for cfg in (SMALL["skewed_small"], SMALL["mixtral_decode_small"]):
        log(f"[graph] {cfg.name}")
        inp = W.make_inputs(cfg, "cuda")
        layer, y_ref, r_ref = run_layer(cfg, inp)
        y = torch.empty_like(y_ref)
        r = layer.routing_buffers()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                M.moe_layer_forward(layer.desc, inp, inp["x"], y, r, layer.ws)
        torch.cuda.synchronize()
        for rep in range(4):
            y.zero_()
            r["perm"].fill_(-7)
            layer.forward(inp["x"])                       # eager work between the replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y.view(torch.int16) if y.dtype == torch.bfloat16 else y,
                               y_ref.view(torch.int16) if y_ref.dtype == torch.bfloat16 else y_ref), rep
            for key in ("idx", "w", "counts", "offsets", "inv"):
                assert torch.equal(r[key], r_ref[key]), (rep, key)
            n = int(r_ref["offsets"][-1])
            assert torch.equal(r["perm"][:n], r_ref["perm"][:n]), rep
        del g
    _free()


def test_stage_entry_points_compose_to_forward():
    # (fine_shared_t320: the forward's routed rows in bf16, the stage entry points' in fp32)
    for cfg in (SMALL["deepseek_small"], SMALL["skewed_small"], SMALL["swiglu_f32_shared"], SMALL["fine_shared_t320"]):
        log(f"[stages] {cfg.name}")
        inp = W.make_inputs(cfg, "cuda")
        layer, y_ref, r_ref = run_layer(cfg, inp)
        desc = desc_of(cfg)
        T, N, k, d = cfg.T, cfg.N, cfg.k, cfg.d
        dev = "cuda"
        logits = torch.empty((T, N), dtype=torch.float32, device=dev)
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device=dev)
        M.moe_route(desc, inp["x"], inp["w_router"], inp["logit_bias"], logits, idx, w, ws)
        counts = torch.empty(N, dtype=torch.int32, device=dev)
        offsets = torch.empty(N + 1, dtype=torch.int32, device=dev)
        perm = torch.empty(T * k, dtype=torch.int32, device=dev)
        inv = torch.empty(T * k, dtype=torch.int32, device=dev)
        x_perm = torch.empty((T * k, d), dtype=inp["x"].dtype, device=dev)
        M.moe_permute(desc, idx, counts, offsets, perm, inv, inp["x"], x_perm)
        rows = T * k + (T if cfg.has_shared else 0)
        y_perm = torch.empty((rows, d), dtype=torch.float32, device=dev)
        M.moe_expert_ffn(desc, inp, inp["x"], perm, offsets, None, y_perm, ws)
        y = torch.empty_like(y_ref)
        M.moe_combine(desc, y_perm, inv, w, y)
        torch.cuda.synchronize()
        for key, t in (("logits", logits), ("idx", idx), ("w", w), ("counts", counts), ("offsets", offsets),
                       ("inv", inv)):
            assert torch.equal(t, r_ref[key]), key
        n = int(offsets[-1])
        assert torch.equal(perm[:n], r_ref["perm"][:n])
        tok = (perm[:n].long() // k)
        assert torch.equal(x_perm[:n], inp["x"][tok])
        # unscaled fp32 rows + weights in the combine vs rows scaled in the down projection (in bf16
        # for the routed rows of fine-grained layers with a shared expert): the two sums differ by
        # at most 2^-8 of each routed contribution (bf16 unit roundoff) plus fp32 summation order,
        # and each is rounded once to the output dtype, so a bf16 output may differ by one ulp on
        # top
        err = rel_rms_err(f64(y), f64(y_ref))
        log(f"[stages] {cfg.name}: max|y_stages - y_forward|/RMS = {err:.3e}")
        if cfg.dtype == "f32":
            assert err <= 1e-6, err
        else:
            yp = f64(y_perm)
            iv = inv.cpu().numpy().reshape(T, k)
            wn = np.abs(w.cpu().numpy().astype(np.float64))
            routed = np.zeros((T, d))
            for j in range(k):
                ok = iv[:, j] >= 0
                routed[ok] += wn[ok, j][:, None] * np.abs(yp[iv[ok, j]])
            shared = np.abs(yp[T * k:T * k + T]) if cfg.has_shared else 0.0
            ya, yb = f64(y), f64(y_ref)
            top = np.maximum(np.maximum(np.abs(ya), np.abs(yb)), 1e-30)
            ulp = np.exp2(np.floor(np.log2(top)) - 7)
            bound = 2.0 ** -8 * routed + ulp + 1e-5 * (routed + shared)
            assert (np.abs(ya - yb) <= bound).all(), float(np.max(np.abs(ya - yb) - bound))
    _free()


FULL = ["mixtral_prefill", "mixtral_decode", "deepseek_v3", "skewed_capacity", "switch_top1", "scout_top1",
        "v4_shared_top7", "maverick_top1"]


def test_hidden_state_beyond_4gib():
    # H holds 140000 rows x 16384 bf16 = 4.6 GB: the out-projection reads each tile's rows from
    # that tile's own base, since 32-bit byte offsets from the start of H end at row 131072;
    # every token is checked, at least six of them with rows past that
    cfg = W.LayerConfig("h_beyond_4gib", T=140000, d=64, N=2, k=1, d_ff=16384, dtype="bf16", ffn=W.FFN_SWIGLU,
                        gating=W.GATE_TOPK_SOFTMAX, seed=29)
    log(f"[{cfg.name}] T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} d_ff={cfg.d_ff}")
    inp = W.make_inputs(cfg, "cuda")
    layer, y, r = run_layer(cfg, inp)
    rn = routing_to_np(r)
    z64, zerr, alike = check_routing(cfg, inp, rn)
    far = np.nonzero(alike & (rn["inv"].reshape(cfg.T, cfg.k)[:, 0] >= (1 << 32) // (2 * cfg.d_ff)))[0]
    assert far.size >= 6
    ref = oracle_forward(cfg, inp, z=z64)
    check_y(cfg, f64(y)[alike], ref["y"][alike], label=f" {int(alike.sum())} of {cfg.T} tokens:")
    check_y(cfg, f64(y)[far], ref["y"][far], label=f" {far.size} tokens with rows past 4 GiB of H:")
    del layer, y, r, inp
    _free()


@pytest.mark.parametrize("name", FULL)
def test_full_size_layer(name):
    cfg = C[name]
    log(f"[{name}] full size: T={cfg.T} d={cfg.d} N={cfg.N} k={cfg.k} d_ff={cfg.d_ff}")
    inp = W.make_inputs(cfg, "cuda")
    layer, y, r = run_layer(cfg, inp)
    rn = routing_to_np(r)
    z64, zerr, alike = check_routing(cfg, inp, rn)
    yg = f64(y)
    del y
    ref = oracle_forward(cfg, inp, z=z64)         # every token, one expert at a time
    check_y(cfg, yg[alike], ref["y"][alike], label=f" all {int(alike.sum())} of {cfg.T} tokens routed alike:")
    _stats_parity(cfg, layer, r, rn, z64, zerr, ref)
    if cfg.capacity_factor > 0:
        C_ = O.expert_capacity(cfg.capacity_factor, cfg.T, cfg.k, cfg.N)
        assert rn["counts"].max() <= C_ and rn["counts"].sum() == cfg.T * cfg.k
        log(f"[{name}] capacity {C_}: experts full = {int((rn['counts'] == C_).sum())}, "
            f"slots outside their token's top {cfg.k} = "
            f"{int((~(ref['idx'][:, :, None] == O.rank_experts(z64)[:, None, :cfg.k]).any(2)).sum())}")
    del layer, r, inp
    _free()
