"""GPU parity of the expert-parallel layouts, with G ranks simulated on one GPU.

The send layout (destination-major grouping, split sizes, packed rows) and the
receive layout (grouping of the received rows by local expert) must equal the
oracle's bit for bit.  End to end, every simulated rank routes its own tokens,
packs its send buffer, the test moves the blocks between ranks as the two
all-to-alls would (plain device copies), each rank runs the grouped FFN on the
rows it received with its own experts' weights and unpacks them, and each
source combines what comes back: y must match the oracle's single-device
forward of the same tokens.  The router is a selection router (exact logits),
so the oracle's routing is the GPU's and every layout compares bit for bit."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_48_amd as M
import oracle as O
import workloads as W
from gpu_harness import check_y, f64, log

pytestmark = pytest.mark.gpu

I32 = dict(dtype=torch.int32, device="cuda")


def _dispatch(desc, idx, owner, G, x=None):
    T, k, N = desc.T, desc.k, desc.N
    out = dict(counts=torch.empty(N, **I32), expert_offsets=torch.empty(N + 1, **I32),
               send_counts=torch.empty(G, **I32), send_offsets=torch.empty(G + 1, **I32),
               perm=torch.empty(T * k, **I32), inv=torch.empty(T * k, **I32))
    send_buf = None if x is None else torch.empty((T * k, x.shape[1]), dtype=x.dtype, device="cuda")
    M.moe_ep_dispatch(desc, idx, owner, G, out["counts"], out["expert_offsets"], out["send_counts"],
                      out["send_offsets"], out["perm"], out["inv"], x, send_buf)
    return out, send_buf


def _np(d):
    return {k: v.cpu().numpy().astype(np.int64) for k, v in d.items()}


DISPATCH_CASES = [
    # T, N, k, G, owner kind, seed, capacity C (0 = none), levels
    (300, 8, 2, 8, "contiguous", 61, 0, None),
    (1000, 64, 4, 8, "interleaved", 62, 0, 8),
    (777, 256, 8, 16, "random", 63, 0, None),
    (60, 16, 2, 64, "random", 64, 0, None),
    (2000, 32, 2, 4, "random", 65, 80, None),      # capacity: dropped slots
    (1, 8, 2, 2, "interleaved", 66, 0, None),
]


@pytest.mark.parametrize("case", DISPATCH_CASES, ids=[f"T{c[0]}_N{c[1]}_G{c[3]}_{c[4]}" for c in DISPATCH_CASES])
def test_ep_dispatch_and_pack(case):
    T, N, k, G, kind, seed, C, levels = case
    log(f"[ep dispatch] T={T} N={N} k={k} G={G} {kind} C={C}")
    owner = W.make_owner_map(N, G, kind, seed)
    z = W.make_logits(T, N, seed, "cuda", levels=levels).cpu().numpy().astype(np.float64)
    idx = O.capacity_route(z, k, C)[0] if C else O.topk_route(z, k, O.TOPK_SOFTMAX)[0]
    desc = M.make_desc(T, 128, N, k, 128)
    x = W.make_tokens(T, 128, "bf16", seed, "cuda")
    g, send_buf = _dispatch(desc, torch.from_numpy(idx.astype(np.int32)).cuda(), owner, G, x)
    torch.cuda.synchronize()
    g = _np(g)
    ref = O.ep_dispatch_layout(idx, owner, G)
    for key in ("counts", "expert_offsets", "send_counts", "send_offsets", "inv"):
        assert np.array_equal(g[key], ref[key]), key
    n = int(ref["send_offsets"][-1])
    assert np.array_equal(g["perm"][:n], ref["perm"])
    assert torch.equal(send_buf[:n], x[torch.from_numpy(ref["perm"] // k).cuda()])


RECEIVE_CASES = [
    # N, G, owner kind, sources' T, k, seed
    (8, 8, "contiguous", [300, 20, 1, 77, 500, 3, 64, 128], 2, 71),
    (64, 4, "interleaved", [1000, 10, 333, 1], 4, 72),
    (256, 16, "random", [100] * 16, 8, 73),
    (16, 64, "random", [5] * 64, 2, 74),
]


@pytest.mark.parametrize("case", RECEIVE_CASES, ids=[f"N{c[0]}_G{c[1]}_{c[2]}" for c in RECEIVE_CASES])
def test_ep_receive_layout(case):
    N, G, kind, Ts, k, seed = case
    log(f"[ep receive] N={N} G={G} {kind}")
    owner = W.make_owner_map(N, G, kind, seed)
    counts = []
    for s, T in enumerate(Ts):
        z = W.make_logits(T, N, seed * 100 + s, "cuda").cpu().numpy().astype(np.float64)
        counts.append(O.ep_dispatch_layout(O.topk_route(z, k, O.TOPK_SOFTMAX)[0], owner, G)["counts"])
    rc = np.array(counts)
    rc_d = torch.from_numpy(rc.astype(np.int32)).cuda()
    for rank in range(G):
        ref = O.ep_receive_layout(rc, owner, rank)
        R = int(ref["recv_offsets"][-1])
        nl = len(ref["local_experts"])
        ro = torch.empty(G + 1, **I32)
        lo = torch.empty(nl + 1, **I32)
        rp = torch.empty(max(R, 1), **I32)
        ri = torch.empty(max(R, 1), **I32)
        M.moe_ep_receive_layout(N, G, owner, rank, rc_d, R, ro, lo, rp, ri)
        torch.cuda.synchronize()
        assert np.array_equal(ro.cpu().numpy(), ref["recv_offsets"]), rank
        assert np.array_equal(lo.cpu().numpy(), ref["local_offsets"]), rank
        assert np.array_equal(rp.cpu().numpy()[:R], ref["recv_perm"]), rank
        assert np.array_equal(ri.cpu().numpy()[:R], ref["recv_inv"]), rank


EP_FORWARD = [
    # name, layer config, G, owner kind, tokens per rank
    ("ep4_interleaved", W.LayerConfig("ep4_interleaved", T=0, d=128, N=16, k=2, d_ff=192, dtype="bf16",
                                      ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, seed=81),
     4, "interleaved", [300, 123, 1, 77]),
    ("ep8_contiguous_relu", W.LayerConfig("ep8_contiguous_relu", T=0, d=128, N=64, k=4, d_ff=128, dtype="bf16",
                                          ffn=W.FFN_RELU2, gating=W.GATE_SOFTMAX_TOPK, seed=82),
     8, "contiguous", [200, 64, 17, 300, 5, 128, 90, 256]),
    ("ep3_random_capacity", W.LayerConfig("ep3_random_capacity", T=0, d=64, N=8, k=2, d_ff=128, dtype="bf16",
                                          ffn=W.FFN_SWIGLU, gating=W.GATE_TOPK_SOFTMAX, capacity_factor=0.5,
                                          seed=83),
     3, "random", [400, 50, 201]),
]


@pytest.mark.parametrize("name", [c[0] for c in EP_FORWARD])
def test_ep_forward_simulated_ranks(name):
    _, cfg, G, kind, Ts = next(c for c in EP_FORWARD if c[0] == name)
    N, k, d, dff = cfg.N, cfg.k, cfg.d, cfg.d_ff
    owner = W.make_owner_map(N, G, kind, cfg.seed)
    log(f"[{name}] G={G} owner={owner} tokens={Ts}")
    wts = W.make_selection_router_inputs(cfg.replace(T=1), "cuda")     # weights shared by every rank
    mk = lambda T, n, kk, cf=0.0: M.make_desc(T, d, n, kk, dff, cfg.dtype, cfg.ffn, cfg.gating, cf)  # noqa: E731
    src = []
    for s, T in enumerate(Ts):
        x = W.make_tokens(T, d, cfg.dtype, cfg.seed * 100 + s, "cuda", grid_cols=N, levels=16)
        desc = mk(T, N, k, cfg.capacity_factor)
        ws = torch.empty(M.moe_workspace_size(desc), dtype=torch.uint8, device="cuda")
        logits = torch.empty((T, N), dtype=torch.float32, device="cuda")
        idx = torch.empty((T, k), **I32)
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        M.moe_route(desc, x, wts["w_router"], None, logits, idx, w, ws)
        lay, send_buf = _dispatch(desc, idx, owner, G, x)
        src.append(dict(x=x, desc=desc, idx=idx, w=w, lay=lay, send_buf=send_buf))
    torch.cuda.synchronize()
    # count exchange: every rank receives every source's full count vector
    rc = torch.stack([s["lay"]["counts"] for s in src])
    so = [s["lay"]["send_offsets"].cpu().tolist() for s in src]
    ret = {}
    for r in range(G):
        loc = [e for e in range(N) if owner[e] == r]
        recv_buf = torch.cat([s["send_buf"][so[i][r]:so[i][r + 1]] for i, s in enumerate(src)])
        R = recv_buf.shape[0]
        ro = torch.empty(G + 1, **I32)
        if R == 0 or not loc:
            ret[r] = (torch.zeros((0, d), dtype=torch.float32, device="cuda"), [0] * (G + 1))
            continue
        lo = torch.empty(len(loc) + 1, **I32)
        rp = torch.empty(R, **I32)
        ri = torch.empty(R, **I32)
        M.moe_ep_receive_layout(N, G, owner, r, rc, R, ro, lo, rp, ri)
        li = torch.tensor(loc, device="cuda")
        lw = {key: (None if wts[key] is None else wts[key].index_select(0, li).contiguous())
              for key in ("w_gate", "w_up", "w_down")}
        dr = mk(R, len(loc), 1)
        ws = torch.empty(M.moe_workspace_size(dr), dtype=torch.uint8, device="cuda")
        yg = torch.empty((R, d), dtype=torch.float32, device="cuda")
        M.moe_expert_ffn(dr, lw, recv_buf, rp, lo, None, yg, ws)
        back = torch.empty_like(yg)
        M.moe_ep_unpack(G, R, d * 4, ro, ri, yg, back)
        torch.cuda.synchronize()
        ret[r] = (back, ro.cpu().tolist())
        # receive layout vs the oracle's on the oracle's own counts (checked below per source)
    for i, s in enumerate(src):
        # return exchange: rank order is the source's send order
        back = torch.cat([ret[r][0][ret[r][1][i]:ret[r][1][i + 1]] for r in range(G)])
        y = torch.empty((Ts[i], d), dtype=cfg.torch_dtype, device="cuda")
        M.moe_combine(s["desc"], back, s["lay"]["inv"], s["w"], y)
        torch.cuda.synchronize()
        ref = O.forward(f64(s["x"]), f64(wts["w_router"]), f64(wts["w_up"]), f64(wts["w_down"]), k,
                        O.SWIGLU if cfg.ffn == W.FFN_SWIGLU else O.RELU2,
                        O.TOPK_SOFTMAX if cfg.gating == W.GATE_TOPK_SOFTMAX else O.SOFTMAX_TOPK,
                        w_gate=None if wts["w_gate"] is None else f64(wts["w_gate"]),
                        capacity_factor=cfg.capacity_factor)
        assert np.array_equal(s["idx"].cpu().numpy(), ref["idx"]), i
        lay = O.ep_dispatch_layout(ref["idx"], owner, G)
        g = _np(s["lay"])
        for key in ("counts", "send_counts", "send_offsets", "inv"):
            assert np.array_equal(g[key], lay[key]), (i, key)
        check_y(cfg.replace(T=Ts[i]), f64(y), ref["y"], label=f" rank {i} ({Ts[i]} tokens):")
    # every rank's receive layout against the oracle's, on the oracle's counts
    rc_ref = np.array([O.ep_dispatch_layout(s["idx"].cpu().numpy(), owner, G)["counts"] for s in src])
    assert np.array_equal(rc.cpu().numpy(), rc_ref)
