"""GPU parity of the routing steps and the routing statistics on exact logits.

With a selection router (row e of the router is the unit vector on input
feature e) every logit is an input value, exact in any summation order; the
inputs lie on a grid of multiples of 1/8, so many logits tie exactly.  The
GPU's logits, indices, grouping and statistics must then equal the oracle's
bit for bit (gate weights within 1e-6, float statistics within 1e-12
relative), and y within the layer's tolerance.  The statistics kernel is also
checked on its own, on seeded logits with routings the oracle produced and
the test then perturbed (dropped and swapped slots), at every expert count
the kernel specialises for and with ragged token counts."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_48_amd as M
import oracle as O
import workloads as W
from gpu_harness import check_stats, check_y, f64, gpu_routing_stats, log, oracle_forward, run_layer

pytestmark = pytest.mark.gpu

LC = W.LayerConfig
SW, RL = W.FFN_SWIGLU, W.FFN_RELU2
TS, ST = W.GATE_TOPK_SOFTMAX, W.GATE_SOFTMAX_TOPK
# name: (config, grid levels, grid bias)
EXACT = {
    "sel_topk_n8": (LC("sel_topk_n8", T=500, d=64, N=8, k=2, d_ff=64, dtype="bf16", ffn=SW, gating=TS, seed=31),
                    8, False),
    "sel_softmax_n256_k8": (LC("sel_softmax_n256_k8", T=300, d=256, N=256, k=8, d_ff=64, dtype="bf16", ffn=SW,
                               gating=ST, has_shared=True, seed=32), 16, False),
    "sel_capacity_n16": (LC("sel_capacity_n16", T=400, d=64, N=16, k=2, d_ff=64, dtype="bf16", ffn=SW, gating=TS,
                            capacity_factor=1.0, seed=33), 8, True),
    "sel_capacity_deep_n256": (LC("sel_capacity_deep_n256", T=300, d=256, N=256, k=2, d_ff=64, dtype="bf16",
                                  ffn=SW, gating=TS, capacity_factor=0.5, seed=34), 6, True),
    "sel_f32_relu": (LC("sel_f32_relu", T=50, d=40, N=5, k=2, d_ff=24, dtype="f32", ffn=RL, gating=ST, seed=35),
                     4, True),
    "sel_k_eq_n": (LC("sel_k_eq_n", T=70, d=64, N=4, k=4, d_ff=64, dtype="bf16", ffn=SW, gating=TS, seed=36),
                   4, False),
    "sel_one_token": (LC("sel_one_token", T=1, d=64, N=8, k=2, d_ff=64, dtype="bf16", ffn=SW, gating=TS, seed=37),
                      8, False),
    "sel_top1_n128": (LC("sel_top1_n128", T=600, d=128, N=128, k=1, d_ff=128, dtype="bf16", ffn=RL, gating=TS,
                         seed=38), 32, True),
    "sel_decode": (LC("sel_decode", T=16, d=256, N=8, k=2, d_ff=256, dtype="bf16", ffn=SW, gating=TS, seed=39),
                   8, False),
    # 16384 slots with capacity drops: the grouping over many blocks, bit for bit
    "sel_capacity_many": (LC("sel_capacity_many", T=8192, d=64, N=64, k=2, d_ff=64, dtype="bf16", ffn=SW,
                             gating=TS, capacity_factor=0.5, seed=42), 8, True),
    # K split in four parts (d = 1024) and summed in the same launch as top-k (1400 slots)
    "sel_reduce_topk": (LC("sel_reduce_topk", T=700, d=1024, N=16, k=2, d_ff=64, dtype="bf16", ffn=SW, gating=TS,
                           seed=41), 8, True),
    # a batch at the single-block routing finish's limit of 512 slots (64 tokens x top-8), over 100
    # experts (more than one wave's 64 lanes, an expert count the fused router does not take)
    "sel_finish_limits": (LC("sel_finish_limits", T=64, d=256, N=100, k=8, d_ff=64, dtype="bf16", ffn=SW,
                             gating=ST, seed=40), 16, True),
}


@pytest.mark.parametrize("name", list(EXACT))
def test_exact_logits_routing_and_stats(name):
    cfg, levels, grid_bias = EXACT[name]
    log(f"[{name}] selection router: T={cfg.T} N={cfg.N} k={cfg.k} {cfg.gating} cf={cfg.capacity_factor} "
        f"levels={levels} bias={grid_bias}")
    inp = W.make_selection_router_inputs(cfg, "cuda", levels=levels, grid_bias=grid_bias)
    layer, y, r = run_layer(cfg, inp)
    rn = {k: v.cpu().numpy() for k, v in r.items()}
    ref = oracle_forward(cfg, inp)
    assert np.array_equal(rn["logits"].astype(np.float64), ref["z"]), "logits"
    ties = int(sum((np.sort(row)[::-1][:cfg.k + 1][:-1] == np.sort(row)[::-1][1:cfg.k + 1]).any()
                   for row in ref["z"]))
    log(f"[{name}] tokens with a tie among their first {cfg.k + 1} ranks: {ties}")
    assert np.array_equal(rn["idx"], ref["idx"]), "idx"
    assert float(np.max(np.abs(rn["w"] - ref["w"]))) <= 1e-6
    assert np.array_equal(rn["counts"], ref["counts"]) and np.array_equal(rn["offsets"], ref["offsets"])
    assert np.array_equal(rn["perm"][: ref["offsets"][-1]], ref["perm"]) and np.array_equal(rn["inv"], ref["inv"])
    check_y(cfg, f64(y), ref["y"])
    for alpha in (0.01, 0.05):
        g = gpu_routing_stats(layer, r, alpha=alpha)
        check_stats(cfg, g, O.routing_stats(ref["z"], ref["idx"], ref["counts"], alpha=alpha), alpha=alpha)
    del layer, y, r, inp
    torch.cuda.empty_cache()


def _stats_direct(T, N, k, seed, levels=None, C=0, drop_frac=0.0, swap_frac=0.0, alpha=0.01):
    """moe_routing_stats on seeded logits and an oracle routing that the test perturbs."""
    z = W.make_logits(T, N, seed, "cuda", levels=levels)
    z64 = z.cpu().numpy().astype(np.float64)
    if C > 0:
        idx, _, _ = O.capacity_route(z64, k, C)
    else:
        idx, _ = O.topk_route(z64, k, O.TOPK_SOFTMAX)
    rng = np.random.default_rng(seed)
    idx = idx.copy()
    if swap_frac > 0 and k > 1:
        rows = rng.random(T) < swap_frac
        idx[rows, 0], idx[rows, 1] = idx[rows, 1].copy(), idx[rows, 0].copy()
    if drop_frac > 0:
        idx[rng.random(idx.shape) < drop_frac] = -1
    counts, _, _, _ = O.group_by_expert(idx, N)
    ref = O.routing_stats(z64, idx, counts, alpha=alpha)
    desc = M.make_desc(T, 64, N, k, 64)
    ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
    stats = torch.empty(M.MOE_NUM_STATS, dtype=torch.float64, device="cuda")
    top3 = torch.empty(3, dtype=torch.int32, device="cuda")
    pm = torch.empty(N, dtype=torch.float64, device="cuda")
    idx_d = torch.from_numpy(idx.astype(np.int32)).cuda()
    cnt_d = torch.from_numpy(counts.astype(np.int32)).cuda()
    M.moe_routing_stats(desc, z, idx_d, cnt_d, stats, top3, ws, alpha=alpha, prob_mean=pm)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    g = {n: float(st[i]) for i, n in enumerate(M.STAT_NAMES)}
    g["top3"] = top3.cpu().numpy().tolist()
    g["prob_mean"] = pm.cpu().numpy()
    return g, ref


STATS_CASES = [
    # T, N, k, seed, levels, C, drop, swap
    (1, 1, 1, 41, None, 0, 0.0, 0.0),
    (17, 2, 1, 42, 4, 0, 0.0, 0.0),
    (33, 3, 2, 43, None, 0, 0.1, 0.2),
    (1000, 8, 2, 44, None, 0, 0.0, 0.3),
    (5000, 64, 4, 45, 8, 0, 0.05, 0.1),
    (777, 65, 2, 46, None, 0, 0.0, 0.0),
    (4099, 128, 2, 47, None, 40, 0.0, 0.0),      # capacity: re-routed and dropped slots
    (300, 200, 6, 48, 16, 0, 0.02, 0.05),
    (6000, 256, 8, 49, None, 0, 0.0, 0.0),
    (2000, 256, 2, 50, 16, 10, 0.0, 0.1),
]


@pytest.mark.parametrize("case", STATS_CASES, ids=[f"T{c[0]}_N{c[1]}_k{c[2]}" for c in STATS_CASES])
def test_routing_stats_direct(case):
    T, N, k, seed, levels, C, drop, swap = case
    log(f"[stats] T={T} N={N} k={k} levels={levels} C={C} drop={drop} swap={swap}")
    cfg = LC(f"stats_T{T}_N{N}", T=T, d=64, N=N, k=k, d_ff=64, dtype="bf16", ffn=SW, gating=TS, seed=seed)
    g, ref = _stats_direct(T, N, k, seed, levels=levels, C=C, drop_frac=drop, swap_frac=swap, alpha=0.02)
    check_stats(cfg, g, ref, alpha=0.02)


def test_routing_stats_no_kept_slot():
    T, N, k = 40, 8, 2
    z = W.make_logits(T, N, 51, "cuda")
    idx = torch.full((T, k), -1, dtype=torch.int32, device="cuda")
    counts = torch.zeros(N, dtype=torch.int32, device="cuda")
    desc = M.make_desc(T, 64, N, k, 64)
    ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
    stats = torch.empty(M.MOE_NUM_STATS, dtype=torch.float64, device="cuda")
    top3 = torch.empty(3, dtype=torch.int32, device="cuda")
    M.moe_routing_stats(desc, z, idx, counts, stats, top3, ws)
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    ref = O.routing_stats(z.cpu().numpy(), idx.cpu().numpy(), counts.cpu().numpy())
    for i, n in enumerate(M.STAT_NAMES):
        if np.isnan(ref[n]):
            assert np.isnan(st[i]), n
        else:
            assert st[i] == ref[n], n
    assert top3.cpu().numpy().tolist() == ref["top3"] == [0, 1, 2]


def test_routing_stats_deterministic():
    g1, _ = _stats_direct(6000, 256, 8, 52)
    g2, _ = _stats_direct(6000, 256, 8, 52)
    for n in M.STAT_NAMES:
        assert g1[n] == g2[n] or (np.isnan(g1[n]) and np.isnan(g2[n])), n
    assert np.array_equal(g1["prob_mean"], g2["prob_mean"])
