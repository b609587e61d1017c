"""Plain float64 CPU definition of the sparse MoE layer forward.

TEST INFRASTRUCTURE.  This module is the oracle that the GPU library is
checked against.  Only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import it.  It shares no code with the HIP path and the
HIP path never calls it.

Every step is written as its plain definition, in float64, from the exact
input values (fp32 or bf16 inputs are exactly representable in float64).
Library primitives used as steps: numpy matmul, exp, lexsort.

Sources (five web pages on mixture-of-experts layers):
  [P1] "MoE 分片：混合專家模型的平行化策略" (optiversetech.com blog)
  [P2] "MoE 推理：激活参数 vs 总参数与专家路由" (inference-learning-path)
  [P3] "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析" (yunthe.com)
  [P4] "MoE 架构科普：为什么大模型要「混合专家」" (lidayun.com)
  [P5] "MoE稀疏激活原理与工程实践：揭秘大模型参数幻觉" (blog.csdn.net)

The layer (one GPU's whole expert set, no cross-device step):
  1. router logits   z = x W_r (+ b)                [P1 什麼是 MoE 模型; P2 深入原理; P5 §2.2]
  2. ranking + gating (two softmax placements)      [P2 代码 toy; P3 核心机制 routing formula]
  3. expert capacity with re-routing (optional)     [P5 §2.2 专家容量]
  4. grouping of (token, slot) pairs by expert      [P5 §3.1 token-level batching]
  5. expert FFN on each expert's rows               [P1 什麼是 MoE 模型: two linear maps + activation]
  6. shared expert on every token (optional)        [P4 专家粒度; P3 DeepSeek-V4 架构细节]
  7. gate-weighted combine                          [P1 動態 token 路由 step 6; P2 代码]
Beside the layer: routing statistics [P5 §4.2, §2.2/§3.3; P3 核心机制] and the
send / receive layouts of expert parallelism [P1 專家平行化詳解, 動態 token 路由];
int4 expert weights (a format defined here: the pages name INT4 experts only).

Readings taken where the pages leave a step open (each also listed in the
design notes): equal logits rank the lower expert id first; slot 0 is the
best-ranked expert; a slot fits an expert iff fill < C before it is placed;
an overflowing slot takes the token's next-ranked expert that it does not
already hold and that still has room; a slot with no room anywhere is dropped
(index -1, weight 0); rows of an expert's group are in ascending (token, slot)
order; experts and the shared expert have no biases.

Parity pins: every function here is pinned by tests/test_oracle_pins.py
against worked values, closed forms, brute force or an independent second
implementation.  Outputs at the full layer sizes have no printed values on
the pages: there the oracle is trusted through those pins.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np

TOPK_SOFTMAX = "topk_softmax"   # rank, keep top-k, softmax over the k kept logits
SOFTMAX_TOPK = "softmax_topk"   # softmax over all N logits, keep top-k probabilities as weights
RELU2 = "relu2"                 # relu(x W1) W2
SWIGLU = "swiglu"               # (silu(x Wg) * (x Wu)) Wd
LINEAR = "linear"               # single d x d linear expert (the toy of [P2] 代码), counting only

__all__ = [
    "TOPK_SOFTMAX", "SOFTMAX_TOPK", "RELU2", "SWIGLU", "LINEAR",
    "router_logits", "rank_experts", "gate_weights", "topk_route", "expert_capacity",
    "capacity_route", "route_from_logits", "group_by_expert", "silu", "expert_ffn",
    "combine", "forward", "param_counts", "near_tie_tokens", "routing_stats",
    "ep_dispatch_layout", "ep_receive_layout",
    "Q4_GROUP", "quantize_q4", "dequantize_q4", "pack_q4", "unpack_q4",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- step 1
def router_logits(x, w_router, logit_bias=None) -> np.ndarray:
    """z[t, e] = sum_i x[t, i] * w_router[i, e]  (+ b[e]).

    The router is a learned linear layer giving one score per expert
    ([P1] 什麼是 MoE 模型; [P2] 深入原理; [P5] §2.2).  w_router is [d, N],
    the toy's router_W ([P2] 代码: gate = x @ router_W).  The optional bias
    b[e] is part of the logit.
    """
    z = _f64(x) @ _f64(w_router)
    if logit_bias is not None:
        z = z + _f64(logit_bias)[None, :]
    return z


# ---------------------------------------------------------------- step 2
def rank_experts(z) -> np.ndarray:
    """order[t, r] = the expert of rank r for token t.

    Descending logit; equal logits put the lower expert id first (the pages
    use argsort, whose order on ties is unspecified).
    """
    z = _f64(z)
    T, N = z.shape
    ids = np.broadcast_to(np.arange(N), (T, N))
    # lexsort: last key is primary -> -z ascending, then expert id ascending
    return np.lexsort((ids, -z), axis=-1)


def gate_weights(z, idx, gating: str) -> np.ndarray:
    """Gate weights of the chosen slots (idx = -1 marks a dropped slot, weight 0).

    TOPK_SOFTMAX: softmax over the logits of the kept experts only, the toy's
    rule ([P2] 代码; 深入原理 "top-k softmax").
    SOFTMAX_TOPK: p = softmax over all N logits, w_j = p[idx_j], with no
    renormalisation ([P3] 核心机制, the standard routing formula).
    Both use the max-subtracted form exp(z - max) / sum exp(z - max).
    """
    z = _f64(z)
    idx = np.asarray(idx)
    T, k = idx.shape
    w = np.zeros((T, k), dtype=np.float64)
    kept = idx >= 0
    if gating == TOPK_SOFTMAX:
        for t in range(T):
            sel = idx[t][kept[t]]
            if sel.size == 0:
                continue
            zs = z[t, sel]
            ez = np.exp(zs - zs.max())
            w[t, kept[t]] = ez / ez.sum()
    elif gating == SOFTMAX_TOPK:
        ez = np.exp(z - z.max(axis=1, keepdims=True))
        p = ez / ez.sum(axis=1, keepdims=True)
        safe = np.where(kept, idx, 0)
        w = np.where(kept, np.take_along_axis(p, safe, axis=1), 0.0)
    else:
        raise ValueError(f"unknown gating {gating!r}")
    return w


def topk_route(z, k: int, gating: str):
    """Top-k routing without a capacity limit: idx[t, j] is the expert of rank j."""
    order = rank_experts(z)
    idx = np.ascontiguousarray(order[:, :k])
    return idx, gate_weights(z, idx, gating)


# ---------------------------------------------------------------- step 3
def expert_capacity(capacity_factor: float, T: int, k: int, N: int) -> int:
    """C = ceil(capacity_factor * T * k / N): capacity_factor times the even
    share of the T*k slots ([P5] §2.2 专家容量, capacity_factor 2.0)."""
    return int(math.ceil(capacity_factor * T * k / N))


def capacity_route(z, k: int, C: int, gating: str = TOPK_SOFTMAX):
    """Routing under a per-expert capacity C, as one serial pass per slot.

    Each expert has a queue with a fill count; an expert that is full sends
    the token on to its next-best expert ([P5] §2.2 专家容量).  Slot priority:
    every token's first slot in token order, then every token's second slot,
    and so on.  A slot takes the highest-ranked expert that the token does
    not already hold and whose fill is still below C; if none has room the
    slot is dropped (idx -1).  Weights: gate_weights over the final experts.
    Returns idx, w, fill.
    """
    z = _f64(z)
    T, N = z.shape
    order = rank_experts(z).tolist()
    fill = [0] * N
    idx = [[-1] * k for _ in range(T)]
    for j in range(k):                 # pass j: all j-th slots, token order
        for t in range(T):
            held = idx[t][:j]
            for e in order[t]:
                if e in held:
                    continue
                if fill[e] < C:
                    idx[t][j] = e
                    fill[e] += 1
                    break
    idx = np.array(idx, dtype=np.int64)
    return idx, gate_weights(z, idx, gating), np.array(fill, dtype=np.int64)


def route_from_logits(z, k: int, gating: str, C: Optional[int] = None):
    """Steps 2-3 from given logits: (idx, w); C None or <= 0 means no capacity."""
    if C is None or C <= 0:
        return topk_route(z, k, gating)
    idx, w, _ = capacity_route(z, k, C, gating)
    return idx, w


# ---------------------------------------------------------------- step 4
def group_by_expert(idx, N: int):
    """Group the (token, slot) pairs by expert ([P5] §3.1 token-level batching).

    Slot s = t*k + j.  counts[e] = number of slots routed to e;
    offsets = exclusive prefix sum of counts (offsets[N] = number of kept
    slots); perm[r] = the slot placed in row r, rows of expert e are
    offsets[e] .. offsets[e+1]-1 in ascending slot order; inv[s] = row of
    slot s, or -1 for a dropped slot.
    """
    flat = np.asarray(idx).reshape(-1)
    counts = np.zeros(N, dtype=np.int64)
    for e in flat:
        if e >= 0:
            counts[e] += 1
    offsets = np.zeros(N + 1, dtype=np.int64)
    for e in range(N):
        offsets[e + 1] = offsets[e] + counts[e]
    nxt = offsets[:N].copy()
    perm = np.zeros(int(offsets[N]), dtype=np.int64)
    inv = np.full(flat.size, -1, dtype=np.int64)
    for s, e in enumerate(flat):
        if e < 0:
            continue
        perm[nxt[e]] = s
        inv[s] = nxt[e]
        nxt[e] += 1
    return counts, offsets, perm, inv


# ---------------------------------------------------------------- step 5/6
def silu(u):
    """silu(u) = u * sigmoid(u) = u / (1 + exp(-u))."""
    u = _f64(u)
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def expert_ffn(xr, w_up, w_down, ffn: str, w_gate=None) -> np.ndarray:
    """One expert's FFN on rows xr [M, d]: two linear maps with an activation
    between them ([P1] 什麼是 MoE 模型), no biases.

    RELU2:  relu(xr W1) W2, W1 = w_up [d, d_ff], W2 = w_down [d_ff, d]
    SWIGLU: (silu(xr Wg) * (xr Wu)) Wd, Wg/Wu [d, d_ff], Wd [d_ff, d]
    (the x W orientation of the toy's x @ experts_W[e], [P2] 代码)
    """
    xr = _f64(xr)
    if ffn == RELU2:
        h = np.maximum(xr @ _f64(w_up), 0.0)
    elif ffn == SWIGLU:
        h = silu(xr @ _f64(w_gate)) * (xr @ _f64(w_up))
    else:
        raise ValueError(f"unknown ffn {ffn!r}")
    return h @ _f64(w_down)


# ---------------------------------------------------------------- step 7
def combine(slot_out, w, y_shared=None) -> np.ndarray:
    """y[t] = sum_j w[t, j] * slot_out[t, j]  (+ y_shared[t], weight 1), summed
    in slot order ([P1] 動態 token 路由 step 6; [P2] 代码; [P3] routing
    formula).  slot_out [T, k, d]; dropped slots carry w = 0."""
    slot_out = _f64(slot_out)
    w = _f64(w)
    y = np.zeros((slot_out.shape[0], slot_out.shape[2]), dtype=np.float64)
    for j in range(slot_out.shape[1]):
        y = y + w[:, j:j + 1] * slot_out[:, j, :]
    if y_shared is not None:
        y = y + _f64(y_shared)
    return y


# ---------------------------------------------------------------- whole layer
def forward(x, w_router, w_up, w_down, k: int, ffn: str, gating: str, w_gate=None,
            logit_bias=None, capacity_factor: float = 0.0, shared: Optional[Sequence] = None,
            tokens: Optional[Sequence[int]] = None, z=None) -> Dict[str, np.ndarray]:
    """The whole layer forward, steps 1-7.

    x [T, d]; w_router [d, N].  Expert weights are indexed per expert
    (w_gate[e], w_up[e] [d, d_ff], w_down[e] [d_ff, d]); any object that
    returns one expert's array on indexing works, so large weight sets can be
    converted to float64 one expert at a time.
    shared = (sh_gate, sh_up, sh_down) or None.
    tokens: evaluate the FFN/combine only for these tokens (routing always
    covers every token, since capacity couples them).
    z: use these logits instead of computing step 1 (logits the caller
    already computed with router_logits, reused).
    Returns z, idx, w, counts, offsets, perm, inv, C, y (rows = tokens).
    """
    x = np.asarray(x)
    T = x.shape[0]
    if z is None:
        z = router_logits(x, w_router, logit_bias)
    z = _f64(z)
    N = z.shape[1]
    C = expert_capacity(capacity_factor, T, k, N) if capacity_factor > 0 else 0
    idx, w = route_from_logits(z, k, gating, C)
    counts, offsets, perm, inv = group_by_expert(idx, N)

    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    d = x.shape[1]
    slot_out = np.zeros((tok.size, k, d), dtype=np.float64)
    sub_idx = idx[tok]
    for e in np.unique(sub_idx[sub_idx >= 0]):
        rows, slots = np.nonzero(sub_idx == e)
        wg = w_gate[e] if ffn == SWIGLU else None
        slot_out[rows, slots, :] = expert_ffn(x[tok[rows]], w_up[e], w_down[e], ffn, wg)
    y_sh = None
    if shared is not None:          # same FFN form as the routed experts
        sg, su, sd = shared
        y_sh = expert_ffn(x[tok], su, sd, ffn, sg)
    y = combine(slot_out, w[tok], y_sh)
    return dict(z=z, idx=idx, w=w, counts=counts, offsets=offsets, perm=perm, inv=inv, C=C, y=y,
                y_shared=y_sh)


# ---------------------------------------------------------------- expert parallelism
def ep_dispatch_layout(idx, owner: Sequence[int], G: int) -> Dict[str, np.ndarray]:
    """Send-side layout when the experts are spread over G ranks ([P1]
    專家平行化詳解: each GPU owns some experts; 動態 token 路由 steps 3-4:
    every token goes to the GPUs that own its experts).

    owner[e] = rank holding expert e.  Slot s = t*k + j is kept iff its
    expert e = idx[t, j] lies in [0, N).  Kept slots are ordered by the key
    (owner[e], e, s): rank r's rows come out contiguous, and inside them each
    expert's rows in slot order.  Returns counts [N]; expert_offsets [N+1]
    (row of expert e's first slot = kept slots with a smaller (owner, expert)
    key; [N] = kept slots); send_counts [G]; send_offsets [G+1]; perm (row ->
    slot); inv (slot -> row, -1 if dropped).
    """
    flat = [int(e) for e in np.asarray(idx).reshape(-1)]
    N = len(owner)
    kept = [s for s, e in enumerate(flat) if 0 <= e < N]
    order = sorted(kept, key=lambda s: (owner[flat[s]], flat[s], s))
    perm = np.array(order, dtype=np.int64)
    inv = np.full(len(flat), -1, dtype=np.int64)
    for r, s in enumerate(order):
        inv[s] = r
    counts = np.zeros(N, dtype=np.int64)
    for s in kept:
        counts[flat[s]] += 1
    expert_offsets = np.zeros(N + 1, dtype=np.int64)
    for e in range(N):
        expert_offsets[e] = sum(int(counts[e2]) for e2 in range(N) if (owner[e2], e2) < (owner[e], e))
    expert_offsets[N] = len(kept)
    send_counts = np.zeros(G, dtype=np.int64)
    for s in kept:
        send_counts[owner[flat[s]]] += 1
    send_offsets = np.zeros(G + 1, dtype=np.int64)
    for r in range(G):
        send_offsets[r + 1] = send_offsets[r] + send_counts[r]
    return dict(counts=counts, expert_offsets=expert_offsets, send_counts=send_counts,
                send_offsets=send_offsets, perm=perm, inv=inv)


def ep_receive_layout(recv_counts, owner: Sequence[int], rank: int) -> Dict[str, np.ndarray]:
    """Receive-side layout on rank `rank` ([P1] 動態 token 路由 steps 3-5).

    recv_counts[s][e] = rows source s sends for expert e.  The receive buffer
    holds the sources in order; inside source s's block, this rank's experts
    in ascending id, each with its recv_counts[s][e] rows.  The grouped order
    that the experts run on takes local expert by local expert (ascending
    id), and inside one expert the sources in order, each source's rows in
    its order.  Returns recv_offsets [G+1] (first receive row of each
    source), local_offsets [n_local+1], recv_perm (grouped row -> receive
    row), recv_inv (receive row -> grouped row).
    """
    rc = np.asarray(recv_counts, dtype=np.int64)
    G, N = rc.shape
    local = [e for e in range(N) if owner[e] == rank]
    rows = [(s, e, i) for s in range(G) for e in local for i in range(int(rc[s, e]))]
    grouped = sorted(range(len(rows)), key=lambda r: (local.index(rows[r][1]), rows[r][0], rows[r][2]))
    recv_perm = np.array(grouped, dtype=np.int64)
    recv_inv = np.zeros(len(rows), dtype=np.int64)
    for g, r in enumerate(grouped):
        recv_inv[r] = g
    recv_offsets = np.zeros(G + 1, dtype=np.int64)
    for s in range(G):
        recv_offsets[s + 1] = recv_offsets[s] + sum(int(rc[s, e]) for e in local)
    local_offsets = np.zeros(len(local) + 1, dtype=np.int64)
    for le, e in enumerate(local):
        local_offsets[le + 1] = local_offsets[le] + int(rc[:, e].sum())
    return dict(recv_offsets=recv_offsets, local_offsets=local_offsets, recv_perm=recv_perm,
                recv_inv=recv_inv, local_experts=np.array(local, dtype=np.int64))


# ---------------------------------------------------------------- int4 expert weights
Q4_GROUP = 128      # input features per scale group


def quantize_q4(w):
    """Weight-only int4 quantisation of one weight matrix w [K, rows] in the
    x W orientation (K inputs, one column per output; the pages name
    GPTQ/AWQ INT4 expert weights at a quarter of the memory, [P3]
    DeepSeek-V4的MoE架构工程细节 and [P5] §3.1's AWQ deployment, and give no
    format; this one is defined here).

    Per output (row of the result) and group of Q4_GROUP consecutive inputs:
    scale = amax / 7 with amax the largest |w| of the group, and
    q = clamp(rint(w / scale), -8, 7) (round half to even); an all-zero group
    has scale 0 and q = 0.  The scale and the division are taken in fp32, the
    precision in which the kernel decides the codes.  Returns q [rows, K] int8
    (one row per output) and scales [rows, K / Q4_GROUP] fp32.  The weight it
    stands for is scale * q (dequantize_q4).
    """
    w = np.asarray(w, dtype=np.float32).T
    rows, K = w.shape
    blk = w.reshape(rows, K // Q4_GROUP, Q4_GROUP)
    amax = np.max(np.abs(blk), axis=2)                              # [rows, groups], exact
    scales = (amax / np.float32(7.0)).astype(np.float32)            # fp32 division
    safe = np.where(scales > 0, scales, np.float32(1.0))[:, :, None]
    q = np.clip(np.rint(blk / safe), -8, 7)                          # fp32 division, ties to even
    q = np.where(amax[:, :, None] > 0, q, 0).astype(np.int8)         # all-zero group: q = 0
    return q.reshape(rows, K), scales


def dequantize_q4(q, scales):
    """The weight matrix [K, rows] (x W orientation) an int4 matrix stands for:
    element (k, r) = scale[r, g] * q[r, k] for k in group g, exactly (float64)."""
    q = np.asarray(q, dtype=np.float64)
    sc = np.repeat(np.asarray(scales, dtype=np.float64), Q4_GROUP, axis=1)
    return (sc * q).T


def pack_q4(q):
    """Codes (q + 8, four bits each) of a [rows, K] int4 matrix as uint32
    words [rows, K / 8].  Words follow the order the kernel loads them in:
    within row r and group g, word a*4 + s (a, s in 0..3) holds the inputs
    k = 128 g + 32 s + 8 a + i, i = 0..7, with input i's code at bit
    4 * (i // 2) + 16 * (i % 2).
    """
    q = np.asarray(q, dtype=np.int64)
    rows, K = q.shape
    c = (q + 8).astype(np.uint64).reshape(rows, K // Q4_GROUP, 4, 4, 8)   # [r, g, s, a, i]
    c = c.transpose(0, 1, 3, 2, 4)                                      # [r, g, a, s, i]
    shift = np.array([4 * (i // 2) + 16 * (i % 2) for i in range(8)], dtype=np.uint64)
    words = np.bitwise_or.reduce(c << shift, axis=4)                     # [r, g, a, s]
    return words.reshape(rows, K // 8).astype(np.uint32)


def unpack_q4(words, K: int):
    """Inverse of pack_q4: q [rows, K] from the words."""
    words = np.asarray(words, dtype=np.int64)
    rows = words.shape[0]
    w = words.reshape(rows, K // Q4_GROUP, 4, 4, 1)                       # [r, g, a, s, 1]
    shift = np.array([4 * (i // 2) + 16 * (i % 2) for i in range(8)], dtype=np.int64)
    q = ((w >> shift) & 0xF) - 8                                         # [r, g, a, s, i]
    return q.transpose(0, 1, 3, 2, 4).reshape(rows, K).astype(np.int8)   # [r, g, s, a, i]


# ---------------------------------------------------------------- counting
def param_counts(N: int, d: int, k: int, ffn: str = LINEAR, d_ff: int = 0, n_shared: int = 0):
    """(total, active) parameters of one MoE layer: all experts are resident,
    only k routed experts (plus the shared ones) compute per token; the
    router is used by every token ([P1] 總參數量與活躍參數量; [P2] 代码).
    LINEAR is the toy's single d x d expert."""
    per_expert = {LINEAR: d * d, RELU2: 2 * d * d_ff, SWIGLU: 3 * d * d_ff}[ffn]
    router = d * N
    total = (N + n_shared) * per_expert + router
    active = (k + n_shared) * per_expert + router
    return total, active


def near_tie_tokens(z, depth: int, threshold: float = 1e-6) -> np.ndarray:
    """Tokens whose float64 logit gap between ranks r and r+1 is below
    `threshold` for some r < depth (the near-tie instability of top-k,
    [P5] §2.2).  Returns their token ids."""
    z = _f64(z)
    order = rank_experts(z)
    zs = np.take_along_axis(z, order, axis=1)
    depth = min(depth, z.shape[1] - 1)
    gaps = zs[:, :depth] - zs[:, 1:depth + 1]
    return np.nonzero((gaps < threshold).any(axis=1))[0]



# ---------------------------------------------------------------- routing health
def routing_stats(z, idx, counts, alpha: float = 0.01) -> Dict[str, object]:
    """Health statistics of one layer call's routing.

    From [P5] §4.2 (路由质量诊断): the entropy in bits of the experts' share of
    the routed slots (log2 N when every expert gets the same share), the three
    most used experts and their share of the slots, and the ratio of the
    standard deviation of the per-expert counts to their mean (the term of its
    online calibration).  From [P3] (核心机制, the load-balancing loss): the
    value alpha * N * sum_i f_i * p_i, with f_i expert i's share of the routed
    slots and p_i its routing probability averaged over the tokens (softmax over
    all N logits).  From [P5] §2.2 (expert capacity: a token whose choice is
    full is sent on to its next-best expert) and §3.3 (the re-route rate it
    monitors): the share of the T*k slots whose expert is not one of the
    token's own k best-ranked experts, a dropped slot included.

    Readings: a slot counts as re-routed by the expert it holds, not by its
    position (the capacity passes fill slots in order, so a token can hold its
    k best experts in another slot order); shares are of the kept slots (the counts); empty experts add 0 to
    the entropy; the standard deviation is the population one (over the N
    experts); ties among the three most used experts go to the lower id; with
    fewer than three experts the missing ids are -1; with no kept slot every
    share-based value is NaN.  prob_mean is p_i for each expert.
    """
    z = _f64(z)
    idx = np.asarray(idx, dtype=np.int64)
    c = np.asarray(counts, dtype=np.float64)
    T, N = z.shape
    k = idx.shape[1]
    S = c.sum()
    nan = float("nan")
    share = c / S if S > 0 else np.full(N, nan)
    nz = c > 0
    entropy = float(-(share[nz] * np.log2(share[nz])).sum()) if S > 0 else nan
    order = np.lexsort((np.arange(N), -c))              # count descending, then id ascending
    top = [int(e) for e in order[:3]] + [-1] * max(0, 3 - N)
    top3_share = float(c[order[:3]].sum() / S) if S > 0 else nan
    mean = S / N
    cv = float(math.sqrt(((c - mean) ** 2).mean()) / mean) if S > 0 else nan
    zm = z.max(axis=1, keepdims=True)
    p = np.exp(z - zm)
    p /= p.sum(axis=1, keepdims=True)
    p_mean = p.mean(axis=0)
    balance = float(alpha * N * (share * p_mean).sum())
    ranked = rank_experts(z)[:, :k]
    own = (idx[:, :, None] == ranked[:, None, :]).any(axis=2)    # slot's expert in the top k
    rerouted = int((~own).sum())
    return dict(entropy_bits=entropy, entropy_ideal_bits=math.log2(N), top3_share=top3_share,
                max_share=float(share.max()), cv=cv, balance_loss=balance,
                reroute_rate=rerouted / float(T * k), experts_touched=int((c > 0).sum()), top3=top,
                prob_mean=p_mean)
