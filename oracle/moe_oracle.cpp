// Plain float64 CPU oracle of the sparse mixture-of-experts layer forward (C++17, OpenMP).
//
// TEST INFRASTRUCTURE.  This is the definition the GPU library is checked against.  Only the
// tests, the smoke run and the CPU-baseline leg of the benchmark may load it.  It shares no code
// with the HIP library (no header, helper, table or generator in common) and neither calls the
// other.
//
// Every step is its plain definition, evaluated in float64 from the exact input values (fp32 and
// bf16 inputs are exactly representable in float64); weights are read from their own storage
// (fp32, bf16 or float64) one element at a time.  OpenMP only splits independent tokens or rows
// between threads: no sum is reordered, every output element is summed in ascending index order,
// and the results do not depend on the thread count.
//
// Sources (web pages on mixture-of-experts layers, cited by title and section):
//   [P1] "MoE 分片：混合專家模型的平行化策略": 什麼是 MoE 模型 (a learned linear router, the top-k
//        experts run, their outputs weighted by the router's scores; an expert is two linear maps
//        around an activation); 動態 token 路由 step 6 (the weighted combine).
//   [P2] "MoE 推理：激活参数 vs 总参数与专家路由": 代码 (router_W [d, N], top-k, softmax over the
//        picked logits, weighted sum of x @ W_e).
//   [P3] "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析": MoE核心机制 (softmax over all
//        experts, top-K, un-renormalised weights).
//   [P4] "MoE 架构科普：为什么大模型要「混合专家」": 专家粒度 (a shared expert every token passes).
//   [P5] "MoE稀疏激活原理与工程实践：揭秘大模型参数幻觉": 2.2 (expert capacity: a full expert
//        hands the token to its next-best one) and 3.1 (tokens regrouped by expert id).
//
// Layouts (row-major, the x W orientation of the pages' toy): x [T, d]; w_router [d, N];
// w_gate, w_up [N, d, d_ff]; w_down [N, d_ff, d]; shared expert [d, d_ff], [d, d_ff], [d_ff, d].
// For the two-layer ReLU expert w_up holds W1 and w_down W2 (y = relu(x W1) W2).
//
// Readings where the pages leave a step open: equal logits rank the lower expert id first; slot 0
// is the best-ranked expert; a slot fits an expert iff its fill is below C before the slot is
// placed; an overflowing slot takes the token's next-ranked expert that it does not hold and that
// has room; a slot with no room anywhere is dropped (index -1, weight 0); an expert's rows are in
// ascending slot order (slot s = t * k + j); experts have no biases.
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F64 = 2 };
enum { RELU2 = 0, SWIGLU = 1 };
enum { TOPK_SOFTMAX = 0, SOFTMAX_TOPK = 1 };

// Element i of an array stored as fp32, bf16 (the upper 16 bits of an fp32) or float64.
inline double elem(const void* p, size_t i, int dt) {
    if (dt == DT_F64) return static_cast<const double*>(p)[i];
    if (dt == DT_F32) return static_cast<const float*>(p)[i];
    const uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16;
    float f;
    std::memcpy(&f, &bits, sizeof f);
    return f;
}

// n consecutive elements starting at element i0, as float64.
void read_row(const void* p, size_t i0, size_t n, int dt, double* out) {
    for (size_t j = 0; j < n; ++j) out[j] = elem(p, i0 + j, dt);
}

// silu(u) = u * sigmoid(u) = u / (1 + e^-u).
double silu(double u) { return u / (1.0 + std::exp(-u)); }

// v [n] := a [m] W, W stored [m, n] (element offset w0): v[c] = sum_r a[r] W[r, c], summed over
// ascending r (row by row, each product rounded and then added).
void vec_mat(const double* a, size_t m, const void* W, size_t w0, int dt, size_t n, double* v,
             std::vector<double>& row) {
    row.resize(n);
    std::fill(v, v + n, 0.0);
    for (size_t r = 0; r < m; ++r) {
        read_row(W, w0 + r * n, n, dt, row.data());
        const double ar = a[r];
        for (size_t c = 0; c < n; ++c) v[c] += ar * row[c];
    }
}

// One expert on one row xr [d]: y [d] = act(xr W_in) W_down ([P1] 什麼是 MoE 模型: two linear
// maps with an activation between them).  SWIGLU: h = silu(xr Wg) * (xr Wu); RELU2: h = relu(xr W1).
// Each weight is given by its array and the element offset of this expert's matrix.
void expert_row(const double* xr, int d, int d_ff, int ffn, const void* wg, size_t g0, const void* wu,
                size_t u0, const void* wd, size_t d0, int dt, double* y) {
    std::vector<double> h(d_ff), u(d_ff), row;
    vec_mat(xr, d, wu, u0, dt, d_ff, u.data(), row);
    if (ffn == SWIGLU) {
        vec_mat(xr, d, wg, g0, dt, d_ff, h.data(), row);
        for (int f = 0; f < d_ff; ++f) h[f] = silu(h[f]) * u[f];
    } else {
        for (int f = 0; f < d_ff; ++f) h[f] = u[f] > 0.0 ? u[f] : 0.0;
    }
    vec_mat(h.data(), d_ff, wd, d0, dt, d, y, row);
}

}  // namespace

extern "C" {

int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }

// Step 1, router logits ([P1] 什麼是 MoE 模型; [P2] 代码 gate = x @ router_W):
// z[t, e] = sum_i x[t, i] w_router[i, e]  (+ b[e]), w_router [d, N].
void orc_router_logits(int T, int d, int N, const void* x, int x_dt, const void* wr, int wr_dt,
                       const float* bias, double* z) {
#pragma omp parallel
    {
        std::vector<double> xr(d), row;
#pragma omp for schedule(static)
        for (int t = 0; t < T; ++t) {
            read_row(x, (size_t)t * d, d, x_dt, xr.data());
            double* zt = z + (size_t)t * N;
            vec_mat(xr.data(), d, wr, 0, wr_dt, N, zt, row);
            if (bias)
                for (int e = 0; e < N; ++e) zt[e] += (double)bias[e];
        }
    }
}

// Ranking: order[t, r] = the expert of rank r: descending logit, equal logits lower id first
// (a stable sort of the ids 0..N-1 by descending logit).
void orc_rank_experts(int T, int N, const double* z, int32_t* order) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double* zt = z + (size_t)t * N;
        int32_t* o = order + (size_t)t * N;
        for (int e = 0; e < N; ++e) o[e] = e;
        std::stable_sort(o, o + N, [zt](int32_t a, int32_t b) { return zt[a] > zt[b]; });
    }
}

// Gate weights of the slots idx [T, k] (-1 = dropped slot, weight 0).
// TOPK_SOFTMAX: softmax over the kept slots' logits ([P2] 代码).
// SOFTMAX_TOPK: p = softmax over all N logits, w_j = p[idx_j], not renormalised ([P3] MoE核心机制).
// Both in the max-subtracted form exp(z - max) / sum exp(z - max), sums in slot / expert order.
void orc_gate_weights(int T, int N, int k, const double* z, const int32_t* idx, int gating, double* w) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double* zt = z + (size_t)t * N;
        const int32_t* it = idx + (size_t)t * k;
        double* wt = w + (size_t)t * k;
        for (int j = 0; j < k; ++j) wt[j] = 0.0;
        if (gating == TOPK_SOFTMAX) {
            bool any = false;
            double m = 0.0;
            for (int j = 0; j < k; ++j)
                if (it[j] >= 0 && (!any || zt[it[j]] > m)) {
                    m = zt[it[j]];
                    any = true;
                }
            if (!any) continue;
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                if (it[j] >= 0) s += std::exp(zt[it[j]] - m);
            for (int j = 0; j < k; ++j)
                if (it[j] >= 0) wt[j] = std::exp(zt[it[j]] - m) / s;
        } else {
            double m = zt[0];
            for (int e = 1; e < N; ++e) m = zt[e] > m ? zt[e] : m;
            double s = 0.0;
            for (int e = 0; e < N; ++e) s += std::exp(zt[e] - m);
            for (int j = 0; j < k; ++j)
                if (it[j] >= 0) wt[j] = std::exp(zt[it[j]] - m) / s;
        }
    }
}

// Steps 2 without capacity: idx[t, j] = the expert of rank j, then the gate weights.
void orc_topk_route(int T, int N, int k, const double* z, int gating, int32_t* idx, double* w) {
    std::vector<int32_t> order((size_t)T * N);
    orc_rank_experts(T, N, z, order.data());
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) idx[(size_t)t * k + j] = order[(size_t)t * N + j];
    orc_gate_weights(T, N, k, z, idx, gating, w);
}

// Step 3, expert capacity C ([P5] 2.2: a full expert sends the token on to its next-best
// expert): one serial pass per slot position -- every token's slot 0 in token order, then every
// token's slot 1, ...; a slot takes the token's highest-ranked expert that it does not already
// hold and whose fill is below C, or is dropped (-1) if there is none.  fill [N] out.
void orc_capacity_route(int T, int N, int k, int64_t C, const double* z, int gating, int32_t* idx, double* w,
                        int64_t* fill) {
    std::vector<int32_t> order((size_t)T * N);
    orc_rank_experts(T, N, z, order.data());
    for (int e = 0; e < N; ++e) fill[e] = 0;
    for (size_t s = 0; s < (size_t)T * k; ++s) idx[s] = -1;
    for (int j = 0; j < k; ++j) {
        for (int t = 0; t < T; ++t) {
            const int32_t* o = order.data() + (size_t)t * N;
            int32_t* it = idx + (size_t)t * k;
            for (int r = 0; r < N; ++r) {
                const int e = o[r];
                bool held = false;
                for (int jj = 0; jj < j; ++jj) held = held || it[jj] == e;
                if (held) continue;
                if (fill[e] < C) {
                    it[j] = e;
                    ++fill[e];
                    break;
                }
            }
        }
    }
    orc_gate_weights(T, N, k, z, idx, gating, w);
}

// Step 4, grouping by expert ([P5] 3.1): counts[e] = slots routed to e; offsets = exclusive
// prefix sum (offsets[N] = kept slots); rows of expert e hold its slots s = t * k + j in
// ascending s: perm[row] = s, inv[s] = row (or -1 for a dropped slot).
void orc_group_by_expert(int T, int k, int N, const int32_t* idx, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv) {
    const size_t S = (size_t)T * k;
    for (int e = 0; e < N; ++e) counts[e] = 0;
    for (size_t s = 0; s < S; ++s)
        if (idx[s] >= 0) ++counts[idx[s]];
    offsets[0] = 0;
    for (int e = 0; e < N; ++e) offsets[e + 1] = offsets[e] + counts[e];
    std::vector<int32_t> next(offsets, offsets + N);
    for (size_t s = 0; s < S; ++s) {
        const int e = idx[s];
        if (e < 0) {
            inv[s] = -1;
            continue;
        }
        perm[next[e]] = (int32_t)s;
        inv[s] = next[e]++;
    }
}

// Step 5 for one expert on M rows xr [M, d]: y [M, d]; weights [d, d_ff], [d, d_ff], [d_ff, d].
void orc_expert_ffn(int M, int d, int d_ff, int ffn, const void* xr, int x_dt, const void* w_gate,
                    const void* w_up, const void* w_down, int w_dt, double* y) {
#pragma omp parallel
    {
        std::vector<double> xv(d);
#pragma omp for schedule(static)
        for (int m = 0; m < M; ++m) {
            read_row(xr, (size_t)m * d, d, x_dt, xv.data());
            expert_row(xv.data(), d, d_ff, ffn, w_gate, 0, w_up, 0, w_down, 0, w_dt, y + (size_t)m * d);
        }
    }
}

typedef struct {
    int32_t T, d, N, k, d_ff, ffn, gating, has_shared;
    double capacity_factor;            // <= 0: no capacity
    const void* x;                     // [T, d]
    int32_t x_dt;
    const void* w_router;              // [d, N]
    int32_t wr_dt;
    const float* logit_bias;           // [N] or NULL
    const void *w_gate, *w_up, *w_down;          // [N, d, d_ff], [N, d, d_ff], [N, d_ff, d]
    const void *sh_gate, *sh_up, *sh_down;       // [d, d_ff], [d, d_ff], [d_ff, d] (has_shared)
    int32_t w_dt;
    const double* z_in;                // [T, N] logits to use instead of step 1, or NULL
} orc_layer;

typedef struct {
    double* z;                         // [T, N]
    int32_t* idx;                      // [T, k]
    double* w;                         // [T, k]
    int32_t *counts, *offsets, *perm, *inv;   // [N], [N + 1], [T * k], [T * k]
    int64_t* C;                        // capacity (0: none)
    double* y;                         // [n_tokens, d]
} orc_out;

// The whole layer, steps 1-7.  Routing covers every token (capacity couples them); the expert
// FFNs and the combine are evaluated for the n_tokens tokens listed (all T if tokens is NULL),
// y[i] being token tokens[i]:
//   y[t] = sum_j w[t, j] FFN_{idx[t, j]}(x[t])  (+ FFN_shared(x[t]), weight 1),
// summed in slot order ([P1] 動態 token 路由 step 6; [P2] 代码; [P4] 专家粒度).
int orc_forward(const orc_layer* L, int n_tokens, const int32_t* tokens, orc_out* out) {
    const int T = L->T, d = L->d, N = L->N, k = L->k, d_ff = L->d_ff;
    if (T < 0 || d < 1 || N < 1 || k < 1 || k > N || d_ff < 1) return 1;
    if (L->z_in)
        std::memcpy(out->z, L->z_in, sizeof(double) * (size_t)T * N);
    else
        orc_router_logits(T, d, N, L->x, L->x_dt, L->w_router, L->wr_dt, L->logit_bias, out->z);
    int64_t C = 0;
    if (L->capacity_factor > 0.0) {
        C = (int64_t)std::ceil(L->capacity_factor * (double)T * (double)k / (double)N);
        std::vector<int64_t> fill(N);
        orc_capacity_route(T, N, k, C, out->z, L->gating, out->idx, out->w, fill.data());
    } else {
        orc_topk_route(T, N, k, out->z, L->gating, out->idx, out->w);
    }
    *out->C = C;
    orc_group_by_expert(T, k, N, out->idx, out->counts, out->offsets, out->perm, out->inv);
    const int n = tokens ? n_tokens : T;
    const size_t wsz = (size_t)d * d_ff;
#pragma omp parallel
    {
        std::vector<double> xv(d), part(d);
#pragma omp for schedule(dynamic, 1)
        for (int i = 0; i < n; ++i) {
            const int t = tokens ? tokens[i] : i;
            double* yt = out->y + (size_t)i * d;
            std::fill(yt, yt + d, 0.0);
            read_row(L->x, (size_t)t * d, d, L->x_dt, xv.data());
            for (int j = 0; j < k; ++j) {
                const int e = out->idx[(size_t)t * k + j];
                if (e < 0) continue;
                const size_t o = (size_t)e * wsz;
                expert_row(xv.data(), d, d_ff, L->ffn, L->w_gate, o, L->w_up, o, L->w_down, o, L->w_dt,
                           part.data());
                const double wj = out->w[(size_t)t * k + j];
                for (int c = 0; c < d; ++c) yt[c] += wj * part[c];
            }
            if (L->has_shared) {
                expert_row(xv.data(), d, d_ff, L->ffn, L->sh_gate, 0, L->sh_up, 0, L->sh_down, 0, L->w_dt,
                           part.data());
                for (int c = 0; c < d; ++c) yt[c] += part[c];
            }
        }
    }
    return 0;
}

}  // extern "C"
