"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each test checks it against a
value the pages print, a closed form, brute force, a special case that
reduces to a plain product written out with loops, or the independent
capacity implementation in capacity_fixed_point.py.

The oracle has two implementations, the plain C++ one (oracle/moe_oracle.cpp,
through oracle.cpp) and the NumPy one (oracle.moe_oracle); every pin of a step
both implement runs against each of them (the `impl` fixture).
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle as O
import oracle.cpp as OC
from capacity_fixed_point import capacity_route_fixed_point

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


@pytest.fixture(params=["numpy", "cpp"])
def impl(request):
    """The oracle implementation under test: NumPy or the plain C++ one."""
    return O if request.param == "numpy" else OC


# ---------------------------------------------------------------- helpers written out with loops
def naive_matmul(a, w):
    """a [M, K] times w [K, Nout]; pure Python loops in float64."""
    M, K = len(a), len(a[0])
    return [[sum(float(a[m][i]) * float(w[i][n]) for i in range(K)) for n in range(len(w[0]))] for m in range(M)]


def naive_ffn(x, w_up, w_down, ffn, w_gate=None):
    if ffn == O.RELU2:
        h = [[max(v, 0.0) for v in row] for row in naive_matmul(x, w_up)]
    else:
        g = naive_matmul(x, w_gate)
        u = naive_matmul(x, w_up)
        h = [[gv / (1.0 + math.exp(-gv)) * uv for gv, uv in zip(gr, ur)] for gr, ur in zip(g, u)]
    return np.array(naive_matmul(h, w_down))


def naive_softmax(v):
    m = max(v)
    e = [math.exp(a - m) for a in v]
    s = sum(e)
    return [a / s for a in e]


def rand_layer(rng, T, d, N, d_ff, ffn):
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((d, N)) / math.sqrt(d)
    wg = rng.standard_normal((N, d, d_ff)) / math.sqrt(d) if ffn == O.SWIGLU else None
    wu = rng.standard_normal((N, d, d_ff)) / math.sqrt(d)
    wd = rng.standard_normal((N, d_ff, d)) / math.sqrt(d_ff)
    if ffn != O.SWIGLU:
        wg = None
    return x, wr, wg, wu, wd


# ---------------------------------------------------------------- counting (printed values)
def test_toy_param_count_matches_page():
    (row,) = _golden_rows("toy_param_count.txt")
    kv = dict(item.split("=") for item in row)
    total, active = O.param_counts(int(kv["N"]), int(kv["d"]), int(kv["k"]), O.LINEAR)
    assert total == int(kv["total"]) and active == int(kv["active"])
    assert f"{active / total:.2f}" == kv["ratio"]


def test_active_expert_fraction_matches_pages():
    for N, k, pct, dec in _golden_rows("active_fraction.txt"):
        N, k, dec = int(N), int(k), int(dec)
        total, active = O.param_counts(N, 64, k, O.SWIGLU, d_ff=32)
        router = 64 * N
        frac = 100.0 * (active - router) / (total - router)
        assert f"{frac:.{dec}f}" == pct, (N, k, frac, pct)


def test_param_counts_shared_expert_counts_as_always_active():
    t0, a0 = O.param_counts(256, 7168, 8, O.SWIGLU, d_ff=2048)
    t1, a1 = O.param_counts(256, 7168, 8, O.SWIGLU, d_ff=2048, n_shared=1)
    per = 3 * 7168 * 2048
    assert t1 - t0 == per and a1 - a0 == per


# ---------------------------------------------------------------- worked combine (page 1, step 6)
@pytest.mark.parametrize("gating", [O.TOPK_SOFTMAX, O.SOFTMAX_TOPK])
def test_worked_combine_two_experts(impl, gating):
    # Experts 2 and 5 get scores 0.6 and 0.4; the output is 0.6 E2(x) + 0.4 E5(x).
    # Expert e is relu(x I) (c_e I): on x > 0 it returns c_e * x exactly.
    N, d = 8, 4
    z = np.full((1, N), -200.0)
    z[0, 2] = math.log(0.6)
    z[0, 5] = math.log(0.4)
    c = np.arange(1, N + 1, dtype=np.float64)
    w_up = np.stack([np.eye(d)] * N)
    w_down = np.stack([c[e] * np.eye(d) for e in range(N)])
    x = np.array([[0.5, 1.0, 2.0, 3.0]])
    out = impl.forward(x, None, w_up, w_down, 2, O.RELU2, gating, z=z)
    assert out["idx"].tolist() == [[2, 5]]
    assert np.allclose(out["w"], [[0.6, 0.4]], atol=1e-12, rtol=0)
    assert np.allclose(out["y"], (0.6 * c[2] + 0.4 * c[5]) * x, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- top-k
def test_topk_set_is_brute_force_best_subset_with_ties(impl):
    rng = np.random.default_rng(5)
    for trial in range(40):
        N = int(rng.integers(1, 7))
        z = rng.integers(-2, 3, size=(30, N)).astype(np.float64)   # many exact ties
        for k in range(1, N + 1):
            idx, _ = impl.topk_route(z, k, O.TOPK_SOFTMAX)
            for t in range(z.shape[0]):
                best = max(itertools.combinations(range(N), k),
                           key=lambda s: (sum(z[t, list(s)]), [-e for e in s]))
                assert sorted(idx[t].tolist()) == list(best)
                zs = z[t, idx[t]]
                for j in range(k - 1):            # slot order: descending, ties to lower id
                    assert zs[j] > zs[j + 1] or (zs[j] == zs[j + 1] and idx[t, j] < idx[t, j + 1])


def test_both_gating_modes_pick_the_same_experts(impl):
    rng = np.random.default_rng(6)
    z = rng.standard_normal((64, 16))
    ia, _ = impl.topk_route(z, 4, O.TOPK_SOFTMAX)
    ib, _ = impl.topk_route(z, 4, O.SOFTMAX_TOPK)
    assert np.array_equal(ia, ib)


def test_gate_weight_invariants_and_closed_forms(impl):
    rng = np.random.default_rng(7)
    z = 3.0 * rng.standard_normal((50, 12))
    for k in (1, 2, 5, 12):
        ia, wa = impl.topk_route(z, k, O.TOPK_SOFTMAX)
        ib, wb = impl.topk_route(z, k, O.SOFTMAX_TOPK)
        assert np.allclose(wa.sum(axis=1), 1.0, atol=1e-12)
        assert (np.diff(wa, axis=1) <= 1e-15).all()           # best slot has the largest weight
        for t in range(z.shape[0]):
            p = naive_softmax(z[t].tolist())
            assert np.allclose(wb[t], [p[e] for e in ib[t]], atol=1e-14, rtol=0)
            assert np.allclose(wa[t], naive_softmax([z[t, e] for e in ia[t]]), atol=1e-14, rtol=0)
        assert (wb.sum(axis=1) <= 1.0 + 1e-12).all()
        if k == 12:
            assert np.allclose(wb.sum(axis=1), 1.0, atol=1e-12)
            assert np.allclose(wa, wb, atol=1e-14)               # k = N: the two modes coincide
    # k = 1 in mode A always gives weight exactly 1
    _, w1 = impl.topk_route(z, 1, O.TOPK_SOFTMAX)
    assert (w1 == 1.0).all()


def test_softmax_is_shift_invariant_and_stable_for_large_logits(impl):
    z = np.array([[1000.0, 999.0, -1000.0]])
    _, w = impl.topk_route(z, 2, O.TOPK_SOFTMAX)
    e = math.exp(-1.0)
    assert np.allclose(w, [[1 / (1 + e), e / (1 + e)]], atol=1e-15, rtol=0)


# ---------------------------------------------------------------- FFN
def test_silu_closed_form_points():
    u = np.array([0.0, 1.0, -1.0, 2.0, -30.0, 40.0])
    want = [0.0, 0.7310585786300049, -0.2689414213699951, 1.7615941559557649,
            -30.0 * 9.357622968840175e-14, 40.0]
    assert np.allclose(O.silu(u), want, rtol=1e-12, atol=1e-20)


@pytest.mark.parametrize("ffn", [O.RELU2, O.SWIGLU])
def test_expert_ffn_against_written_out_products(impl, ffn):
    rng = np.random.default_rng(8)
    M, d, d_ff = 3, 5, 7                      # non-square: a transposed operand cannot pass
    x = rng.standard_normal((M, d))
    wg = rng.standard_normal((d, d_ff))
    wu = rng.standard_normal((d, d_ff))
    wd = rng.standard_normal((d_ff, d))
    got = impl.expert_ffn(x, wu, wd, ffn, wg if ffn == O.SWIGLU else None)
    want = naive_ffn(x.tolist(), wu.tolist(), wd.tolist(), ffn, wg.tolist())
    assert got.shape == (M, d)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)


def test_router_logits_against_written_out_product_and_bias(impl):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 6))
    wr = rng.standard_normal((6, 3))
    b = np.array([0.5, -1.0, 2.0], dtype=np.float32)      # the bias is an fp32 input
    want = np.array(naive_matmul(x.tolist(), wr.tolist())) + b.astype(np.float64)
    assert np.allclose(impl.router_logits(x, wr, b), want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- whole-layer special cases
@pytest.mark.parametrize("ffn", [O.RELU2, O.SWIGLU])
def test_k_equals_n_is_dense_softmax_mixture(impl, ffn):
    rng = np.random.default_rng(10)
    T, d, N, d_ff = 6, 4, 5, 3
    x, wr, wg, wu, wd = rand_layer(rng, T, d, N, d_ff, ffn)
    z = O.router_logits(x, wr)
    expert_out = [naive_ffn(x.tolist(), wu[e].tolist(), wd[e].tolist(), ffn,
                            None if wg is None else wg[e].tolist()) for e in range(N)]
    want = np.zeros((T, d))
    for t in range(T):
        p = naive_softmax(z[t].tolist())
        for e in range(N):
            want[t] += p[e] * expert_out[e][t]
    for gating in (O.TOPK_SOFTMAX, O.SOFTMAX_TOPK):
        out = impl.forward(x, wr, wu, wd, N, ffn, gating, w_gate=wg)
        assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("ffn", [O.RELU2, O.SWIGLU])
def test_identical_experts_reduce_to_one_ffn(impl, ffn):
    rng = np.random.default_rng(11)
    T, d, N, d_ff, k = 7, 4, 6, 5, 3
    x, wr, wg, wu, wd = rand_layer(rng, T, d, N, d_ff, ffn)
    wu[:] = wu[0]
    wd[:] = wd[0]
    if wg is not None:
        wg[:] = wg[0]
    want = naive_ffn(x.tolist(), wu[0].tolist(), wd[0].tolist(), ffn, None if wg is None else wg[0].tolist())
    out = impl.forward(x, wr, wu, wd, k, ffn, O.TOPK_SOFTMAX, w_gate=wg)
    assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-12)
    outb = impl.forward(x, wr, wu, wd, k, ffn, O.SOFTMAX_TOPK, w_gate=wg)
    assert np.allclose(outb["y"], outb["w"].sum(axis=1, keepdims=True) * want, rtol=1e-12, atol=1e-12)


def test_single_expert_is_plain_ffn(impl):
    rng = np.random.default_rng(12)
    x, wr, wg, wu, wd = rand_layer(rng, 5, 4, 1, 6, O.SWIGLU)
    out = impl.forward(x, wr, wu, wd, 1, O.SWIGLU, O.TOPK_SOFTMAX, w_gate=wg)
    want = naive_ffn(x.tolist(), wu[0].tolist(), wd[0].tolist(), O.SWIGLU, wg[0].tolist())
    assert np.allclose(out["y"], want, rtol=1e-12, atol=1e-12)
    assert out["counts"].tolist() == [5]


def test_page_toy_layer_semantics(impl):
    # The toy of page 2 (section 代码): experts are single d x d linears, top-k by
    # argsort, softmax over the picked logits, weighted sum of x @ W_e.  A ReLU
    # expert with W1 = I sees x > 0 unchanged, so it is the toy's linear expert.
    rng = np.random.default_rng(13)
    N, d, k, T = 8, 16, 2, 10
    experts_W = rng.standard_normal((N, d, d)) / d
    router_W = rng.standard_normal((d, N))
    x = np.abs(rng.standard_normal((T, d))) + 0.01
    want = np.zeros((T, d))
    for t in range(T):
        gate = [sum(x[t, i] * router_W[i, e] for i in range(d)) for e in range(N)]
        top = sorted(range(N), key=lambda e: gate[e])[-k:]
        w = naive_softmax([gate[e] for e in top])
        for wi, e in zip(w, top):
            want[t] += wi * np.array(naive_matmul([x[t].tolist()], experts_W[e].tolist())[0])
    # router_W and experts_W are taken as the toy lays them out (x @ W)
    out = impl.forward(x, router_W, np.stack([np.eye(d)] * N), experts_W, k, O.RELU2, O.TOPK_SOFTMAX)
    assert np.allclose(out["y"], want, rtol=1e-11, atol=1e-12)


def test_shared_expert_adds_plain_ffn_with_weight_one(impl):
    rng = np.random.default_rng(14)
    T, d, N, d_ff, k = 6, 4, 5, 3, 2
    x, wr, wg, wu, wd = rand_layer(rng, T, d, N, d_ff, O.SWIGLU)
    sg, su, sd = rng.standard_normal((d, d_ff)), rng.standard_normal((d, d_ff)), rng.standard_normal((d_ff, d))
    base = impl.forward(x, wr, wu, wd, k, O.SWIGLU, O.SOFTMAX_TOPK, w_gate=wg)
    with_sh = impl.forward(x, wr, wu, wd, k, O.SWIGLU, O.SOFTMAX_TOPK, w_gate=wg, shared=(sg, su, sd))
    want_sh = naive_ffn(x.tolist(), su.tolist(), sd.tolist(), O.SWIGLU, sg.tolist())
    assert np.allclose(with_sh["y"] - base["y"], want_sh, rtol=1e-11, atol=1e-12)
    assert with_sh["counts"].sum() == T * k


def test_token_subset_matches_full_evaluation(impl):
    rng = np.random.default_rng(15)
    x, wr, wg, wu, wd = rand_layer(rng, 20, 8, 6, 5, O.SWIGLU)
    full = impl.forward(x, wr, wu, wd, 2, O.SWIGLU, O.TOPK_SOFTMAX, w_gate=wg, capacity_factor=1.0)
    sub = impl.forward(x, wr, wu, wd, 2, O.SWIGLU, O.TOPK_SOFTMAX, w_gate=wg, capacity_factor=1.0,
                    tokens=[19, 3, 7])
    assert np.allclose(sub["y"], full["y"][[19, 3, 7]], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- grouping by expert
def test_group_by_expert_invariants_and_brute_force(impl):
    rng = np.random.default_rng(16)
    for trial in range(20):
        T, k, N = int(rng.integers(1, 40)), int(rng.integers(1, 4)), int(rng.integers(1, 9))
        idx = rng.integers(-1 if trial % 3 == 0 else 0, N, size=(T, k))
        counts, offsets, perm, inv = impl.group_by_expert(idx, N)
        flat = idx.reshape(-1)
        kept = [s for s in range(T * k) if flat[s] >= 0]
        assert perm.tolist() == sorted(kept, key=lambda s: (flat[s], s))
        assert counts.tolist() == [int((flat == e).sum()) for e in range(N)]
        assert offsets[0] == 0 and offsets[-1] == len(kept)
        assert np.array_equal(np.diff(offsets), counts)
        for r, s in enumerate(perm):
            assert inv[s] == r
        assert all(inv[s] == -1 for s in range(T * k) if flat[s] < 0)


# ---------------------------------------------------------------- capacity
def test_capacity_value_of_the_skewed_layer():
    assert O.expert_capacity(2.0, 16384, 2, 128) == 512
    assert O.expert_capacity(2.0, 100, 2, 8) == 50
    assert O.expert_capacity(1.0, 10, 1, 3) == 4           # ceil(10/3)


def test_capacity_64_reading(impl):
    # capacity 64: a token whose first choice already holds 63 slots still fits
    # (it becomes the 64th); the next one is re-routed to its next-best expert.
    T, N = 66, 4
    z = np.tile(np.array([3.0, 2.0, 1.0, 0.0]), (T, 1))
    idx, w, fill = impl.capacity_route(z, 1, 64)
    assert idx[:64, 0].tolist() == [0] * 64
    assert idx[64:, 0].tolist() == [1, 1]
    assert fill.tolist() == [64, 2, 0, 0]
    assert (w == 1.0).all()


def test_capacity_drop_when_no_room_anywhere(impl):
    z = np.array([[1.0, 0.0], [1.0, 0.0]])
    idx, w, fill = impl.capacity_route(z, 2, 1)
    assert idx.tolist() == [[0, -1], [1, -1]]
    assert w.tolist() == [[1.0, 0.0], [1.0, 0.0]]
    assert fill.tolist() == [1, 1]


def _replay_ok(z, idx, C):
    """Every slot's expert is the best one it could take at its turn."""
    T, N = z.shape
    k = idx.shape[1]
    fill = [0] * N
    for j in range(k):
        for t in range(T):
            e = idx[t, j]
            held = set(idx[t, :j].tolist())
            better = [f for f in range(N) if (z[t, f] > (z[t, e] if e >= 0 else -np.inf)) or
                      (e >= 0 and z[t, f] == z[t, e] and f < e)]
            if any(f not in held and fill[f] < C for f in better):
                return False
            if e < 0:
                if any(f not in held and fill[f] < C for f in range(N)):
                    return False
            else:
                if e in held or fill[e] >= C:
                    return False
                fill[e] += 1
    return True


def test_capacity_serial_equals_independent_fixed_point(impl):
    rng = np.random.default_rng(17)
    for trial in range(60):
        T = int(rng.integers(1, 60))
        N = int(rng.integers(2, 9))
        k = int(rng.integers(1, min(3, N) + 1))
        C = int(rng.integers(1, max(2, T * k // N + 2)))
        z = rng.standard_normal((T, N)) - 2.0 * np.log(np.arange(N) + 1.0)[None, :]
        if trial % 4 == 0:
            z = np.round(z)                       # exact ties
        idx, w, fill = impl.capacity_route(z, k, C)
        idx2, fill2 = capacity_route_fixed_point(z, k, C)
        assert np.array_equal(idx, idx2), (trial, T, N, k, C)
        assert np.array_equal(fill, fill2)
        assert (fill <= C).all()
        for t in range(T):
            kept = [e for e in idx[t] if e >= 0]
            assert len(kept) == len(set(kept))
        assert _replay_ok(z, idx, C)
        if fill.sum() == T * k:
            assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)


def test_capacity_large_enough_equals_plain_topk(impl):
    rng = np.random.default_rng(18)
    z = rng.standard_normal((40, 6))
    for k in (1, 2, 3):
        C = O.expert_capacity(6 / k, 40, k, 6)          # cf = N/k -> C = T: never binds
        idx, w, _ = impl.capacity_route(z, k, C)
        idx0, w0 = impl.topk_route(z, k, O.TOPK_SOFTMAX)
        assert np.array_equal(idx, idx0)
        assert np.allclose(w, w0, atol=0, rtol=0)


def test_near_tie_detection():
    z = np.array([[1.0, 1.0 + 5e-7, 0.0], [3.0, 2.0, 1.0], [0.0, 0.5, 0.5 + 2e-6]])
    assert O.near_tie_tokens(z, depth=1).tolist() == [0]
    assert O.near_tie_tokens(z, depth=2, threshold=3e-6).tolist() == [0, 2]


# ---------------------------------------------------------------- routing health statistics
def _uniform_routing(T, N, k):
    """Token t takes experts (t*k + j) mod N in slot j: every expert gets T*k/N slots when N
    divides T*k; logits rank exactly those experts first."""
    idx = np.array([[(t * k + j) % N for j in range(k)] for t in range(T)])
    z = np.zeros((T, N))
    for t in range(T):
        for j in range(k):
            z[t, idx[t, j]] = 10.0 - j
    counts = np.bincount(idx.ravel(), minlength=N)
    return z, idx, counts


def test_routing_entropy_of_uniform_128_experts_is_the_printed_ideal():
    for N, val, dec in ((int(r[0]), float(r[1]), int(r[2])) for r in _golden_rows("router_entropy.txt")):
        z, idx, counts = _uniform_routing(T=N * 4, N=N, k=2)
        st = O.routing_stats(z, idx, counts)
        assert round(st["entropy_bits"], dec) == val
        assert st["entropy_bits"] == pytest.approx(st["entropy_ideal_bits"], abs=1e-12)
        assert st["top3_share"] == pytest.approx(3.0 / N) and st["cv"] == pytest.approx(0.0, abs=1e-15)
        assert st["reroute_rate"] == 0.0 and st["experts_touched"] == N


def test_routing_stats_all_slots_on_one_expert():
    T, N = 12, 8
    z = np.full((T, N), -1.0)
    z[:, 5] = 3.0
    idx = np.full((T, 1), 5)
    counts = np.bincount(idx.ravel(), minlength=N)
    st = O.routing_stats(z, idx, counts)
    assert st["entropy_bits"] == 0.0 and st["top3_share"] == 1.0 and st["max_share"] == 1.0
    assert st["top3"] == [5, 0, 1]                     # ties among the empty experts: lower id first
    assert st["cv"] == pytest.approx(math.sqrt(N - 1))  # counts (0,..,T,..,0): std = T*sqrt(N-1)/N, mean = T/N


def test_routing_stats_hand_worked_counts():
    # two experts with counts 3 and 1: shares 3/4 and 1/4, entropy 2 - (3/4) log2 3, mean 2, std 1
    z = np.array([[1.0, 0.0]] * 3 + [[0.0, 1.0]])
    idx = np.array([[0], [0], [0], [1]])
    st = O.routing_stats(z, idx, np.array([3, 1]))
    assert st["entropy_bits"] == pytest.approx(2.0 - 0.75 * math.log2(3.0), abs=1e-15)
    assert st["cv"] == pytest.approx(0.5) and st["top3"] == [0, 1, -1] and st["top3_share"] == 1.0
    # p_0 averaged over tokens = (3 s + (1 - s)) / 4 with s = e/(1+e); loss = a*N*(3/4 p_0 + 1/4 p_1)
    s = math.e / (1.0 + math.e)
    p0 = (3 * s + (1 - s)) / 4
    assert st["balance_loss"] == pytest.approx(0.01 * 2 * (0.75 * p0 + 0.25 * (1 - p0)), abs=1e-15)


def test_balance_loss_closed_forms():
    # uniform shares and uniform probabilities (all logits equal): a * N * N * (1/N)(1/N) = a
    for N in (4, 8, 128):
        T = 2 * N
        idx = np.array([[t % N] for t in range(T)])
        st = O.routing_stats(np.zeros((T, N)), idx, np.bincount(idx.ravel(), minlength=N), alpha=0.01)
        assert st["balance_loss"] == pytest.approx(0.01, abs=1e-15)
    # every slot on expert 0: f = (1, 0, ..); the loss is a * N * mean probability of expert 0
    rng = np.random.default_rng(3)
    z = rng.standard_normal((30, 6))
    p0 = np.mean([naive_softmax(list(row))[0] for row in z])
    idx = np.zeros((30, 1), dtype=int)
    st = O.routing_stats(z, idx, np.bincount(idx.ravel(), minlength=6), alpha=0.05)
    assert st["balance_loss"] == pytest.approx(0.05 * 6 * p0, rel=1e-13)
    # the mean probabilities are a distribution over the experts
    assert st["prob_mean"].sum() == pytest.approx(1.0, abs=1e-15) and st["prob_mean"][0] == pytest.approx(p0)


def test_routing_stats_no_kept_slot_is_undefined():
    st = O.routing_stats(np.zeros((4, 5)), np.full((4, 2), -1), np.zeros(5, dtype=int))
    for key in ("entropy_bits", "top3_share", "max_share", "cv", "balance_loss"):
        assert math.isnan(st[key]), key
    assert st["reroute_rate"] == 1.0 and st["experts_touched"] == 0 and st["top3"] == [0, 1, 2]


def test_reroute_rate_hand_worked_capacity():
    # three tokens, both prefer expert 0, capacity 1, k = 1: token 0 keeps expert 0, token 1 moves
    # to expert 1, token 2 finds no room (dropped): two of three slots re-routed
    z = np.array([[2.0, 1.0]] * 3)
    idx, _, fill = O.capacity_route(z, k=1, C=1)
    assert idx.ravel().tolist() == [0, 1, -1] and fill.tolist() == [1, 1]
    st = O.routing_stats(z, idx, fill)
    assert st["reroute_rate"] == pytest.approx(2.0 / 3.0) and st["experts_touched"] == 2


def test_reroute_rate_counts_experts_not_slot_positions():
    # two tokens ranking e0 > e1 > e2, k = 2, capacity 1.  First slots: token 0 takes e0, token 1
    # finds e0 full and takes e1.  Second slots: token 0 finds e1 full and takes e2; token 1 finds
    # e0 and e2 full (and holds e1): dropped.  Token 1's e1 is one of its two best experts, so of
    # the four slots two are re-routed (token 0's e2 and token 1's dropped slot), not three.
    z = np.array([[3.0, 2.0, 1.0]] * 2)
    idx, _, fill = O.capacity_route(z, k=2, C=1)
    assert idx.tolist() == [[0, 2], [1, -1]] and fill.tolist() == [1, 1, 1]
    st = O.routing_stats(z, idx, fill)
    assert st["reroute_rate"] == 0.5 and st["experts_touched"] == 3 and st["entropy_bits"] == pytest.approx(math.log2(3))


# ---------------------------------------------------------------- expert parallelism layouts
def test_ep_dispatch_one_rank_is_the_grouping_by_expert():
    rng = np.random.default_rng(21)
    idx = rng.integers(-1, 6, size=(40, 3))
    a = O.ep_dispatch_layout(idx, [0] * 6, 1)
    counts, offsets, perm, inv = O.group_by_expert(idx, 6)
    assert np.array_equal(a["perm"], perm) and np.array_equal(a["inv"], inv)
    assert np.array_equal(a["counts"], counts) and np.array_equal(a["expert_offsets"], offsets)
    assert a["send_counts"].tolist() == [offsets[-1]] and a["send_offsets"].tolist() == [0, offsets[-1]]


def test_ep_dispatch_contiguous_owners_keep_expert_order():
    # ranks owning contiguous expert blocks: destination-major order is expert-major order
    rng = np.random.default_rng(22)
    idx = rng.integers(0, 8, size=(50, 2))
    owner = [e // 2 for e in range(8)]
    a = O.ep_dispatch_layout(idx, owner, 4)
    counts, offsets, perm, inv = O.group_by_expert(idx, 8)
    assert np.array_equal(a["perm"], perm)
    assert a["send_counts"].tolist() == [int(counts[2 * r] + counts[2 * r + 1]) for r in range(4)]


def test_ep_dispatch_hand_worked_interleaved_owners():
    # T=3, k=2, N=4, G=2, rank 0 owns experts 0 and 2, rank 1 owns 1 and 3.
    # slots: s0->e1, s1->e0, s2->e2, s3->e3, s4->e0, s5->e1.  Rank 0's rows: e0 (s1, s4), e2 (s2);
    # rank 1's rows: e1 (s0, s5), e3 (s3).
    idx = np.array([[1, 0], [2, 3], [0, 1]])
    a = O.ep_dispatch_layout(idx, [0, 1, 0, 1], 2)
    assert a["perm"].tolist() == [1, 4, 2, 0, 5, 3]
    assert a["inv"].tolist() == [3, 0, 2, 5, 1, 4]
    assert a["send_counts"].tolist() == [3, 3] and a["send_offsets"].tolist() == [0, 3, 6]
    assert a["counts"].tolist() == [2, 2, 1, 1] and a["expert_offsets"].tolist() == [0, 3, 2, 5, 6]


def test_ep_receive_hand_worked():
    # rank 0 owns experts 0 and 2 of 4; source 0 sends 2 rows for e0 and 1 for e2, source 1 sends
    # 1 for e0 and 3 for e2.  Receive rows: s0: e0 e0 e2 | s1: e0 e2 e2 e2.  Grouped: e0 from s0
    # (rows 0, 1) and s1 (row 3), then e2 from s0 (row 2) and s1 (rows 4-6).
    rc = np.array([[2, 9, 1, 9], [1, 9, 3, 9]])
    b = O.ep_receive_layout(rc, [0, 1, 0, 1], 0)
    assert b["recv_perm"].tolist() == [0, 1, 3, 2, 4, 5, 6]
    assert b["recv_inv"].tolist() == [0, 1, 3, 2, 4, 5, 6]
    assert b["local_offsets"].tolist() == [0, 3, 7] and b["recv_offsets"].tolist() == [0, 3, 7]
    assert b["local_experts"].tolist() == [0, 2]


def test_ep_round_trip_brute_force():
    # G sources with their own routings; simulate both exchanges.  Each rank's grouped rows for
    # a local expert must be exactly the (source, slot) pairs routed to it, in (source, slot)
    # order, and every slot's output must come back to the row its source's inv names.
    rng = np.random.default_rng(23)
    N, G, k = 7, 3, 2
    owner = [int(v) for v in rng.integers(0, G, size=N)]
    owner[0], owner[1], owner[2] = 0, 1, 2
    srcs = [rng.integers(-1, N, size=(int(rng.integers(1, 12)), k)) for _ in range(G)]
    disp = [O.ep_dispatch_layout(i, owner, G) for i in srcs]
    # what each source sends: its send rows, tagged (source, slot)
    send = [[(s, int(d["perm"][r])) for r in range(len(d["perm"]))] for s, d in enumerate(disp)]
    recv_counts = np.array([d["counts"] for d in disp])
    back = [dict() for _ in range(G)]
    for r in range(G):
        recv = [row for s in range(G) for row in send[s][disp[s]["send_offsets"][r]:disp[s]["send_offsets"][r + 1]]]
        b = O.ep_receive_layout(recv_counts, owner, r)
        assert b["recv_offsets"][-1] == len(recv)
        grouped = [recv[i] for i in b["recv_perm"]]
        for le, e in enumerate(b["local_experts"]):
            rows = grouped[b["local_offsets"][le]:b["local_offsets"][le + 1]]
            want = [(s, t * k + j) for s in range(G) for t in range(srcs[s].shape[0]) for j in range(k)
                    if srcs[s][t, j] == e]
            assert rows == want
        # expert "outputs" = the grouped rows' tags; unpack into receive order, return by source
        ret = [grouped[b["recv_inv"][i]] for i in range(len(recv))]
        assert ret == recv
        for s in range(G):
            back[s][r] = ret[b["recv_offsets"][s]:b["recv_offsets"][s + 1]]
    for s in range(G):
        returned = [row for r in range(G) for row in back[s][r]]     # rank order = send order
        flat = srcs[s].reshape(-1)
        for slot in range(flat.size):
            if 0 <= flat[slot] < N:
                assert returned[disp[s]["inv"][slot]] == (s, slot)
            else:
                assert disp[s]["inv"][slot] == -1


# ---------------------------------------------------------------- int4 expert weights
def test_q4_pack_hand_worked_word():
    # one row, one group: q = k mod 16 - 8 for k < 128.  Word a*4 + s holds k = 32 s + 8 a + i with
    # code (k mod 16) at bit 4 (i // 2) + 16 (i % 2).  Word 0 (a = 0, s = 0): k = 0..7, codes 0..7:
    # low half nibbles 0, 2, 4, 6 -> 0x6420, high half 1, 3, 5, 7 -> 0x7531.
    q = np.array([[(k % 16) - 8 for k in range(128)]])
    w = O.pack_q4(q)
    assert int(w[0, 0]) == 0x75316420
    # word 4 (a = 1, s = 0): k = 8..15, codes 8..15 -> low 8, 10, 12, 14 and high 9, 11, 13, 15
    assert int(w[0, 4]) == 0xFDB9ECA8
    # word 1 (a = 0, s = 1): k = 32..39, codes 0..7 again
    assert int(w[0, 1]) == 0x75316420
    assert np.array_equal(O.unpack_q4(w, 128), q)


def test_q4_pack_round_trip_random():
    rng = np.random.default_rng(31)
    q = rng.integers(-8, 8, size=(5, 384))
    assert np.array_equal(O.unpack_q4(O.pack_q4(q), 384), q)


def test_q4_quantize_bounds_and_grid():
    rng = np.random.default_rng(32)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    w[2, 128:] = 0.0                                   # an all-zero group
    q, sc = O.quantize_q4(w.T)                         # x W orientation: [K, rows]
    assert q.min() >= -7 and q.max() <= 7            # scale = amax / 7: the codes stay symmetric
    assert sc[2, 1] == 0 and np.all(q[2, 128:] == 0)
    wh = O.dequantize_q4(q, sc).T
    # round to nearest: each weight is within half a step of its code's value
    step = np.repeat(sc.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(wh - w) <= 0.5 * step * (1 + 1e-6) + 1e-12)
    # the largest |w| of every nonzero group maps to +-7
    for r in range(6):
        for g in range(2):
            blk = np.abs(w[r, 128 * g:128 * (g + 1)])
            if blk.max() > 0:
                assert abs(int(q[r, 128 * g + int(np.argmax(blk))])) == 7
    # weights already on a group's grid come back exactly
    grid = (np.arange(-7, 8, dtype=np.float32) * np.float32(0.125))
    wg = np.tile(grid, 20)[:256].reshape(1, 256).astype(np.float32)
    wg[0, 0] = np.float32(0.875)                        # amax 7/8 in both groups -> scale 1/8
    wg[0, 128] = np.float32(-0.875)
    q2, sc2 = O.quantize_q4(wg.T)
    assert np.all(sc2 == np.float32(0.125)) and np.array_equal(O.dequantize_q4(q2, sc2), wg.T.astype(np.float64))


def test_q4_rounding_ties_to_even():
    # amax 7 -> scale exactly 1; w = 2.5 and -0.5 are ties: rint gives 2 and -0 (to even)
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, :4] = [7.0, 2.5, -0.5, 3.5]
    q, sc = O.quantize_q4(w.T)
    assert sc[0, 0] == 1.0 and q[0, :4].tolist() == [7, 2, 0, 4]
