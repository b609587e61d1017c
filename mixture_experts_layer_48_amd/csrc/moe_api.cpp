// C ABI of the MoE layer library: argument validation, workspace carving and the launch
// sequence of each step.  Every entry point checks all of its arguments on the host before it
// enqueues anything, never synchronises, never allocates and keeps no pointer after returning.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdio>
#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "moe_kernels.h"

// Workspace of moe_layer_forward_noalloc: one array of MOE_NOALLOC_SCRATCH_BYTES per GPU the
// library runs on, created with the code object and held until the process ends.  Host code
// never uses this name as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

// slots (T * k) from which the fused forward groups them over many blocks, measured against the
// single block: 65536 slots (DeepSeek-V3 shape) 0.077 -> 0.025 ms, 32768 (skewed layer) 0.036 ->
// 0.016 ms, 8192 (Mixtral prefill) 14.0 -> 12.7 us; at 4096 (top-1 of 16) 10-12 -> 12.3 us
#define PERMUTE_MULTI_MIN_SLOTS 8192

namespace {

thread_local std::string g_err;

moe_status fail(moe_status s, const std::string& msg) {
    g_err = msg;
    return s;
}
moe_status hip_fail(hipError_t e, const char* where) {
    g_err = std::string(where) + ": " + hipGetErrorString(e);
    return MOE_ERR_HIP;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

size_t elem_bytes(const moe_layer_desc& d) { return d.dtype == MOE_BF16 ? 2 : 4; }
bool has_capacity(const moe_layer_desc& d) { return d.capacity_factor > 0.0f; }
long long rows_total(const moe_layer_desc& d) {
    return (long long)d.T * d.k + (d.has_shared ? d.T : 0);
}

// Expert capacity C = ceil(capacity_factor * T * k / N), clamped to int range.
int capacity_of(const moe_layer_desc& d) {
    const double c = std::ceil((double)d.capacity_factor * (double)d.T * (double)d.k / (double)d.N);
    return c >= (double)INT_MAX ? INT_MAX : (int)c;
}

moe_status check_desc(const moe_layer_desc* d) {
    if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
    if (d->T < 0) return fail(MOE_ERR_INVALID_ARG, "T < 0");
    if (d->d < 1 || d->d_ff < 1) return fail(MOE_ERR_INVALID_ARG, "d and d_ff must be >= 1");
    if (d->N < 1) return fail(MOE_ERR_INVALID_ARG, "N must be >= 1");
    if (d->k < 1 || d->k > d->N) return fail(MOE_ERR_INVALID_ARG, "k must satisfy 1 <= k <= N");
    if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
    if (d->ffn != MOE_FFN_RELU2 && d->ffn != MOE_FFN_SWIGLU) return fail(MOE_ERR_INVALID_ARG, "unknown ffn");
    if (d->gating != MOE_GATE_TOPK_SOFTMAX && d->gating != MOE_GATE_SOFTMAX_TOPK)
        return fail(MOE_ERR_INVALID_ARG, "unknown gating");
    if (d->has_shared != 0 && d->has_shared != 1) return fail(MOE_ERR_INVALID_ARG, "has_shared must be 0 or 1");
    if (std::isnan(d->capacity_factor) || std::isinf(d->capacity_factor))
        return fail(MOE_ERR_INVALID_ARG, "capacity_factor must be finite");
    if (d->N > 256) return fail(MOE_ERR_UNSUPPORTED, "N > 256 experts");
    if (d->dtype == MOE_BF16 && (d->d % 64 != 0 || d->d_ff % 64 != 0))
        return fail(MOE_ERR_UNSUPPORTED, "bf16 layers need d % 64 == 0 and d_ff % 64 == 0");
    if ((long long)d->T * d->k + d->T + 1 >= (long long)INT_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "T*k + T exceeds int32 row indexing");
    if ((long long)d->T * d->d >= (long long)INT_MAX * 64LL)
        return fail(MOE_ERR_UNSUPPORTED, "T*d too large");
    // the grouped GEMM gathers x rows through 32-bit byte offsets from one base
    if (d->dtype == MOE_BF16 && (long long)d->T * d->d * 2 >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "bf16 x larger than 4 GiB (T*d*2 >= 2^32)");
    // and reads one expert's weight matrix through 32-bit byte offsets from the matrix's start
    if (d->dtype == MOE_BF16 && (long long)d->d * d->d_ff * 2 >= (1LL << 32))
        return fail(MOE_ERR_UNSUPPORTED, "bf16 expert weight matrix of 4 GiB or more (d*d_ff*2 >= 2^32)");
    return MOE_OK;
}

moe_status check_weights(const moe_layer_desc& d, const moe_weights* w, bool need_router, bool need_ffn) {
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    if (need_router && !w->w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
    if (need_ffn) {
        if (!w->w_up || !w->w_down) return fail(MOE_ERR_INVALID_ARG, "w_up / w_down is NULL");
        if (d.ffn == MOE_FFN_SWIGLU && !w->w_gate) return fail(MOE_ERR_INVALID_ARG, "w_gate is NULL (SwiGLU)");
        if (d.has_shared) {
            if (!w->sh_up || !w->sh_down) return fail(MOE_ERR_INVALID_ARG, "shared expert weights are NULL");
            if (d.ffn == MOE_FFN_SWIGLU && !w->sh_gate) return fail(MOE_ERR_INVALID_ARG, "sh_gate is NULL");
        }
    }
    return MOE_OK;
}

int ksplit_of(const moe_layer_desc& d) {
    return ffn_out_ksplit(d.T, d.k, d.N, d.d, d.d_ff, d.has_shared, d.dtype);
}

// the grouped GEMMs' schedule memory: claim counters, then a tile table
size_t sched_bytes(const moe_layer_desc& d, int ksplit) {
    return align256(ffn_sched_bytes(d.T, d.k, d.N, d.d, d.d_ff, d.has_shared, ksplit));
}

// Workspace of the whole forward, carved in this order (each piece 256-byte aligned).
struct Layout {
    size_t z, ranked, idx, w, counts, offsets, perm, inv, h, yp, ctr, total;
};
Layout layout_of(const moe_layer_desc& d) {
    Layout L{};
    size_t o = 0;
    const size_t T = (size_t)d.T, N = (size_t)d.N, k = (size_t)d.k;
    L.z = o; o += align256(T * N * 4);
    L.ranked = o; o += has_capacity(d) ? align256(capacity_workspace_bytes(d.T, d.N)) : 0;
    L.idx = o; o += align256(T * k * 4);
    L.w = o; o += align256(T * k * 4);
    L.counts = o; o += align256(N * 4);
    L.offsets = o; o += align256((N + 1) * 4);
    L.perm = o; o += align256(T * k * 4);
    L.inv = o; o += align256(T * k * 4);
    // the router's partial logits are dead before the hidden state is written: they share space
    // (before H is written it holds the router's K-part sums, then the grouping's block counts)
    L.h = o; o += std::max({align256((size_t)rows_total(d) * d.d_ff * elem_bytes(d)),
                            align256(router_workspace_bytes(d.T, d.d, d.N, d.dtype)),
                            align256(permute_multi_workspace_bytes(d.T, d.k, d.N))});
    // fp32 expert rows, one copy per K part of the out-projection
    L.yp = o; o += align256((size_t)rows_total(d) * d.d * 4 * ksplit_of(d));
    // the grouped GEMMs' schedule: tile-claim counters and a tile table
    L.ctr = o; o += sched_bytes(d, ksplit_of(d));
    // moe_routing_stats() reuses the workspace from offset 0 for its partial sums
    L.total = std::max(o, align256(stats_workspace_bytes(d.T, d.N)));
    return L;
}
size_t route_ws_bytes(const moe_layer_desc& d, bool have_logits) {
    return (have_logits ? 0 : align256((size_t)d.T * d.N * 4)) +
           (has_capacity(d) ? align256(capacity_workspace_bytes(d.T, d.N)) : 0) +
           align256(router_workspace_bytes(d.T, d.d, d.N, d.dtype));
}
// hidden state H, then the grouped GEMMs' schedule (one K part for the out-projection)
size_t ffn_ws_bytes(const moe_layer_desc& d) {
    return align256((size_t)rows_total(d) * d.d_ff * elem_bytes(d)) + sched_bytes(d, 1);
}
unsigned int* ffn_ctr_of(const moe_layer_desc& d, void* ws) {
    return (unsigned int*)((char*)ws + align256((size_t)rows_total(d) * d.d_ff * elem_bytes(d)));
}

char* at(void* ws, size_t off) { return (char*)ws + off; }

// ---- stages (arguments already validated)
// Steps 1-3.  z: where the logits go; want_z: whether anyone reads them afterwards (the caller, or
// the capacity step) -- the fused router then writes them, and otherwise keeps them on chip.
moe_status stage_route(const moe_layer_desc& d, const void* x, const void* wr, const float* bias, float* z,
                       bool want_z, void* rpart, uint8_t* ranked, int32_t* idx, float* w, hipStream_t s,
                       hipEvent_t ev_mid) {
    hipError_t e;
    if (router_fused_supported(d.N, d.dtype)) {
        const bool cap = has_capacity(d);
        e = launch_router_topk(x, wr, bias, (want_z || cap) ? z : nullptr, d.T, d.d, d.N, d.k, d.gating,
                               cap ? nullptr : idx, w, s);
        if (e != hipSuccess) return hip_fail(e, "router launch");
    } else if (!has_capacity(d) && router_k_parts(d.T, d.d, d.N, d.dtype) > 1) {
        // the K-part sum and top-k in one launch
        e = launch_router_logits(x, wr, bias, z, rpart, d.T, d.d, d.N, d.dtype, s, false);
        if (e != hipSuccess) return hip_fail(e, "router logits launch");
        e = launch_reduce_topk(rpart, router_k_parts(d.T, d.d, d.N, d.dtype), bias, z, d.T, d.N, d.k, d.gating, idx, w,
                               s);
        if (e != hipSuccess) return hip_fail(e, "top-k launch");
    } else {
        e = launch_router_logits(x, wr, bias, z, rpart, d.T, d.d, d.N, d.dtype, s);
        if (e != hipSuccess) return hip_fail(e, "router logits launch");
        if (!has_capacity(d)) {
            e = launch_topk_gate(z, d.T, d.N, d.k, d.gating, idx, w, s);
            if (e != hipSuccess) return hip_fail(e, "top-k launch");
        }
    }
    if (ev_mid) {
        e = hipEventRecord(ev_mid, s);
        if (e != hipSuccess) return hip_fail(e, "event record");
    }
    if (has_capacity(d)) {
        e = launch_capacity(z, ranked, d.T, d.N, d.k, capacity_of(d), d.gating, idx, w, s);
        if (e != hipSuccess) return hip_fail(e, "capacity launch");
    }
    return MOE_OK;
}

FfnLaunch ffn_args(const moe_layer_desc& d, const moe_weights& wt, const void* x, const int32_t* perm,
                   const int32_t* offsets, const float* row_scale, void* h, void* yp) {
    FfnLaunch f{};
    f.T = d.T; f.d = d.d; f.N = d.N; f.k = d.k; f.d_ff = d.d_ff;
    f.dtype = d.dtype; f.ffn = d.ffn; f.has_shared = d.has_shared;
    f.x = x; f.perm = perm; f.offsets = offsets;
    f.w_gate = wt.w_gate; f.w_up = wt.w_up; f.w_down = wt.w_down;
    f.sh_gate = wt.sh_gate; f.sh_up = wt.sh_up; f.sh_down = wt.sh_down;
    f.row_scale = row_scale; f.h = h; f.y_perm = yp;
    f.ksplit = 1;
    return f;
}

moe_status record(hipEvent_t ev, hipStream_t s) {
    if (!ev) return MOE_OK;
    hipError_t e = hipEventRecord(ev, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "event record");
}

}  // namespace

extern "C" {

size_t moe_workspace_size(const moe_layer_desc* desc) {
    if (check_desc(desc) != MOE_OK) return 0;
    return layout_of(*desc).total;
}

moe_status moe_route(const moe_layer_desc* desc, const void* x, const void* w_router,
                     const float* logit_bias, float* logits, int32_t* idx, float* w, void* ws,
                     size_t ws_bytes, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    if (d.T == 0) return MOE_OK;
    if (!x || !w_router || !idx || !w) return fail(MOE_ERR_INVALID_ARG, "x, w_router, idx and w are required");
    const size_t need = route_ws_bytes(d, logits != nullptr);
    if (need > 0 && (!ws || ws_bytes < need))
        return fail(MOE_ERR_WORKSPACE, "workspace too small for moe_route: need " + std::to_string(need));
    size_t o = 0;
    float* z = logits;
    if (!z) { z = (float*)at(ws, o); o += align256((size_t)d.T * d.N * 4); }
    uint8_t* ranked = nullptr;
    if (has_capacity(d)) { ranked = (uint8_t*)at(ws, o); o += align256(capacity_workspace_bytes(d.T, d.N)); }
    void* rpart = router_workspace_bytes(d.T, d.d, d.N, d.dtype) ? at(ws, o) : nullptr;
    return stage_route(d, x, w_router, logit_bias, z, logits != nullptr, rpart, ranked, idx, w, (hipStream_t)stream,
                       nullptr);
}

moe_status moe_permute(const moe_layer_desc* desc, const int32_t* idx, int32_t* counts, int32_t* offsets,
                       int32_t* perm, int32_t* inv, const void* x, void* x_perm, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    if (d.T == 0) return MOE_OK;
    if (!idx || !counts || !offsets || !perm || !inv)
        return fail(MOE_ERR_INVALID_ARG, "idx, counts, offsets, perm and inv are required");
    if ((x == nullptr) != (x_perm == nullptr)) return fail(MOE_ERR_INVALID_ARG, "give both x and x_perm or neither");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_permute(idx, d.T, d.k, d.N, counts, offsets, perm, inv, s);
    if (e != hipSuccess) return hip_fail(e, "permute launch");
    if (x_perm) {
        e = launch_gather_rows(x, perm, offsets, d.T, d.k, d.N, (int)(d.d * elem_bytes(d)), x_perm, s);
        if (e != hipSuccess) return hip_fail(e, "gather launch");
    }
    return MOE_OK;
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                          const int32_t* perm, const int32_t* offsets, const float* row_scale, void* y_perm,
                          void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    st = check_weights(d, weights, false, true);
    if (st != MOE_OK) return st;
    if (d.T == 0) return MOE_OK;
    if (!x || !perm || !offsets || !y_perm) return fail(MOE_ERR_INVALID_ARG, "x, perm, offsets and y_perm are required");
    const size_t need = ffn_ws_bytes(d);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace too small for moe_expert_ffn: need " + std::to_string(need));
    hipStream_t s = (hipStream_t)stream;
    FfnLaunch f = ffn_args(d, *weights, x, perm, offsets, row_scale, ws, y_perm);
    f.ctr = ffn_ctr_of(d, ws);
    f.sched_bytes = sched_bytes(d, 1);
    hipError_t e = launch_ffn_in(f, s);
    if (e != hipSuccess) return hip_fail(e, "ffn in-projection launch");
    e = launch_ffn_out(f, s);
    if (e != hipSuccess) return hip_fail(e, "ffn out-projection launch");
    return MOE_OK;
}

moe_status moe_combine(const moe_layer_desc* desc, const void* y_perm, const int32_t* inv, const float* w,
                       void* y, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    if (d.T == 0) return MOE_OK;
    if (!y_perm || !inv || !y) return fail(MOE_ERR_INVALID_ARG, "y_perm, inv and y are required");
    hipError_t e = launch_combine(y_perm, inv, w, y, d.T, d.k, d.d, d.has_shared, d.dtype, 1, 0, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "combine launch");
}

}  // extern "C"

namespace {
// The whole layer; q4 != nullptr selects the int4 expert weights (the FFN weight pointers of
// `weights` are then ignored).
moe_status forward_impl(const moe_layer_desc& d, const moe_weights& weights, const FfnQ4Weights* q4,
                        const void* x, void* y, const moe_routing* routing, void* ws, size_t ws_bytes,
                        hipStream_t s, void* const* events) {
    if (d.T == 0) return MOE_OK;
    if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "x and y are required");
    const Layout L = layout_of(d);
    if (!ws || ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE, "workspace too small for moe_layer_forward: need " + std::to_string(L.total));
    auto ev = [&](int i) -> hipEvent_t { return events ? (hipEvent_t)events[i] : nullptr; };
    const moe_routing none{};
    const moe_routing& R = routing ? *routing : none;
    float* z = R.logits ? R.logits : (float*)at(ws, L.z);
    int32_t* idx = R.idx ? R.idx : (int32_t*)at(ws, L.idx);
    float* w = R.w ? R.w : (float*)at(ws, L.w);
    int32_t* counts = R.counts ? R.counts : (int32_t*)at(ws, L.counts);
    int32_t* offsets = R.offsets ? R.offsets : (int32_t*)at(ws, L.offsets);
    int32_t* perm = R.perm ? R.perm : (int32_t*)at(ws, L.perm);
    int32_t* inv = R.inv ? R.inv : (int32_t*)at(ws, L.inv);
    void* h = at(ws, L.h);
    void* yp = at(ws, L.yp);

    moe_status st;
    hipError_t e;
    if ((st = record(ev(0), s)) != MOE_OK) return st;
    if (!has_capacity(d) && !router_fused_supported(d.N, d.dtype) && route_finish_small_supported(d.T, d.N, d.k)) {
        // a decode-sized batch: the router's logits (fp64 K-part sums), then their sum, top-k,
        // gate weights and the grouping in one block (the stage events that follow mark empty
        // stages)
        void* rpart = at(ws, L.h);
        e = launch_router_logits(x, weights.w_router, weights.logit_bias, z, rpart, d.T, d.d, d.N, d.dtype, s, false);
        if (e != hipSuccess) return hip_fail(e, "router logits launch");
        e = launch_route_finish_small(rpart, router_k_parts(d.T, d.d, d.N, d.dtype), weights.logit_bias, z, d.T, d.N,
                                      d.k, d.gating, idx, w, counts, offsets, perm, inv, s);
        if (e != hipSuccess) return hip_fail(e, "routing launch");
        if ((st = record(ev(1), s)) != MOE_OK) return st;
        if ((st = record(ev(2), s)) != MOE_OK) return st;
    } else {
        st = stage_route(d, x, weights.w_router, weights.logit_bias, z, R.logits != nullptr, at(ws, L.h),
                         (uint8_t*)at(ws, L.ranked), idx, w, s, ev(1));
        if (st != MOE_OK) return st;
        if ((st = record(ev(2), s)) != MOE_OK) return st;
        // large slot counts: the grouping over many blocks, its per-block counts in the hidden
        // state's region (unused until the in-projection)
        if ((long long)d.T * d.k >= PERMUTE_MULTI_MIN_SLOTS)
            e = launch_permute_multi(idx, d.T, d.k, d.N, counts, offsets, perm, inv, (int32_t*)at(ws, L.h), s);
        else
            e = launch_permute(idx, d.T, d.k, d.N, counts, offsets, perm, inv, s);
        if (e != hipSuccess) return hip_fail(e, "permute launch");
    }
    if ((st = record(ev(3), s)) != MOE_OK) return st;
    FfnLaunch f = ffn_args(d, weights, x, perm, offsets, w, h, yp);
    f.ctr = (unsigned int*)at(ws, L.ctr);
    f.sched_bytes = sched_bytes(d, ksplit_of(d));
    if (q4) f.q4 = *q4;
    f.ksplit = q4 ? 1 : ksplit_of(d);
    // the expert outputs are this call's own workspace: on fine-grained layers whose gate weights
    // are probabilities of a softmax over all experts, routed rows may be stored in bf16
    // (ffn_out_routed_bf16 has the rest of the rule and the reason)
    f.routed_bf16_ok = (!q4 && d.gating == MOE_GATE_SOFTMAX_TOPK && 8LL * d.k <= d.N) ? 1 : 0;
    const int routed_bf16 = ffn_out_routed_bf16(f);
    e = q4 ? launch_ffn_in_q4(f, s) : launch_ffn_in(f, s);
    if (e != hipSuccess) return hip_fail(e, "ffn in-projection launch");
    if ((st = record(ev(4), s)) != MOE_OK) return st;
    e = q4 ? launch_ffn_out_q4(f, s) : launch_ffn_out(f, s);
    if (e != hipSuccess) return hip_fail(e, "ffn out-projection launch");
    if ((st = record(ev(5), s)) != MOE_OK) return st;
    e = launch_combine(yp, inv, nullptr, y, d.T, d.k, d.d, d.has_shared, d.dtype, f.ksplit, routed_bf16, s);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return record(ev(6), s);
}

moe_status check_q4(const moe_layer_desc& d, const moe_weights_q4* w, bool need_router, FfnQ4Weights* out) {
    if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
    if (d.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "int4 expert weights need a bf16 layer");
    if (d.d % 128 != 0 || d.d_ff % 128 != 0)
        return fail(MOE_ERR_UNSUPPORTED, "int4 expert weights need d % 128 == 0 and d_ff % 128 == 0");
    if (need_router && !w->w_router) return fail(MOE_ERR_INVALID_ARG, "w_router is NULL");
    auto full = [](const moe_q4_matrix& m) { return m.codes && m.scales; };
    if (!full(w->w_up) || !full(w->w_down)) return fail(MOE_ERR_INVALID_ARG, "w_up / w_down codes or scales are NULL");
    if (d.ffn == MOE_FFN_SWIGLU && !full(w->w_gate)) return fail(MOE_ERR_INVALID_ARG, "w_gate is NULL (SwiGLU)");
    if (d.has_shared) {
        if (!full(w->sh_up) || !full(w->sh_down)) return fail(MOE_ERR_INVALID_ARG, "shared expert weights are NULL");
        if (d.ffn == MOE_FFN_SWIGLU && !full(w->sh_gate)) return fail(MOE_ERR_INVALID_ARG, "sh_gate is NULL");
    }
    out->gate = w->w_gate.codes; out->gate_scales = w->w_gate.scales;
    out->up = w->w_up.codes; out->up_scales = w->w_up.scales;
    out->down = w->w_down.codes; out->down_scales = w->w_down.scales;
    out->sh_gate = w->sh_gate.codes; out->sh_gate_scales = w->sh_gate.scales;
    out->sh_up = w->sh_up.codes; out->sh_up_scales = w->sh_up.scales;
    out->sh_down = w->sh_down.codes; out->sh_down_scales = w->sh_down.scales;
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_layer_forward_timed(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                                   void* y, const moe_routing* routing, void* ws, size_t ws_bytes,
                                   moe_stream_t stream, void* const* events) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_weights(*desc, weights, true, true);
    if (st != MOE_OK) return st;
    return forward_impl(*desc, *weights, nullptr, x, y, routing, ws, ws_bytes, (hipStream_t)stream, events);
}

moe_status moe_layer_forward_q4(const moe_layer_desc* desc, const moe_weights_q4* weights, const void* x, void* y,
                                const moe_routing* routing, void* ws, size_t ws_bytes, moe_stream_t stream,
                                void* const* events) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    FfnQ4Weights q4{};
    if ((st = check_q4(*desc, weights, true, &q4)) != MOE_OK) return st;
    moe_weights router{};
    router.w_router = weights->w_router;
    router.logit_bias = weights->logit_bias;
    return forward_impl(*desc, router, &q4, x, y, routing, ws, ws_bytes, (hipStream_t)stream, events);
}

moe_status moe_expert_ffn_q4(const moe_layer_desc* desc, const moe_weights_q4* weights, const void* x,
                             const int32_t* perm, const int32_t* offsets, const float* row_scale, void* y_perm,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    FfnQ4Weights q4{};
    if ((st = check_q4(d, weights, false, &q4)) != MOE_OK) return st;
    if (d.T == 0) return MOE_OK;
    if (!x || !perm || !offsets || !y_perm) return fail(MOE_ERR_INVALID_ARG, "x, perm, offsets and y_perm are required");
    const size_t need = ffn_ws_bytes(d);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace too small for moe_expert_ffn_q4: need " + std::to_string(need));
    hipStream_t s = (hipStream_t)stream;
    FfnLaunch f = ffn_args(d, moe_weights{}, x, perm, offsets, row_scale, ws, y_perm);
    f.q4 = q4;
    hipError_t e = launch_ffn_in_q4(f, s);
    if (e != hipSuccess) return hip_fail(e, "ffn in-projection launch");
    e = launch_ffn_out_q4(f, s);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ffn out-projection launch");
}

moe_status moe_quantize_q4(const void* w, int32_t n_mats, int32_t rows, int32_t K, uint32_t* codes, float* scales,
                           moe_stream_t stream) {
    g_err.clear();
    if (n_mats < 0 || rows < 0 || K < 0) return fail(MOE_ERR_INVALID_ARG, "negative size");
    if (K % 128 != 0) return fail(MOE_ERR_UNSUPPORTED, "K must be a multiple of 128");
    if ((long long)n_mats * rows * K == 0) return MOE_OK;
    if (!w || !codes || !scales) return fail(MOE_ERR_INVALID_ARG, "w, codes and scales are required");
    if ((long long)n_mats * rows * (K / 128) >= (1LL << 33))
        return fail(MOE_ERR_UNSUPPORTED, "too many groups for one call");
    hipError_t e = launch_q4_quantize(w, n_mats, rows, K, codes, scales, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "quantize launch");
}

moe_status moe_layer_forward(const moe_layer_desc* desc, const moe_weights* weights, const void* x, void* y,
                             const moe_routing* routing, void* ws, size_t ws_bytes, moe_stream_t stream) {
    return moe_layer_forward_timed(desc, weights, x, y, routing, ws, ws_bytes, stream, nullptr);
}

}  // extern "C"

namespace {
#define MOE_NOALLOC_MAX_DEVICES 64
std::mutex g_scratch_mu;
void* g_scratch_ptr[MOE_NOALLOC_MAX_DEVICES] = {};

// Device address of the current device's scratch array, looked up with that device current on
// its first use and kept per device (each GPU holds its own copy of the array).  `stream` must
// belong to the current device.
moe_status noalloc_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= MOE_NOALLOC_MAX_DEVICES)
        return fail(MOE_ERR_UNSUPPORTED, "device index beyond " + std::to_string(MOE_NOALLOC_MAX_DEVICES));
    if (stream) {
        int sdev = -1;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        if (sdev != dev)
            return fail(MOE_ERR_INVALID_ARG, "stream belongs to device " + std::to_string(sdev) +
                                                 ", the current device is " + std::to_string(dev));
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_layer_forward_noalloc(const moe_layer_desc* desc, const moe_weights* weights, const void* x,
                                     void* y, const moe_routing* routing, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    st = check_weights(*desc, weights, true, true);
    if (st != MOE_OK) return st;
    const size_t need = layout_of(*desc).total;
    if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
        return fail(MOE_ERR_UNSUPPORTED, "moe_layer_forward_noalloc: this layer needs " + std::to_string(need) +
                                             " bytes of workspace; the built-in scratch holds " +
                                             std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES) +
                                             " (use moe_layer_forward with a workspace)");
    if (desc->T == 0) return MOE_OK;
    if (!x || !y) return fail(MOE_ERR_INVALID_ARG, "x and y are required");
    void* ws = nullptr;
    if ((st = noalloc_scratch((hipStream_t)stream, &ws)) != MOE_OK) return st;
    // nothing in the forward's workspace has to start at zero: every piece is written before it
    // is read within the call, so the previous call's contents do no harm
    return forward_impl(*desc, *weights, nullptr, x, y, routing, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                        (hipStream_t)stream, nullptr);
}

moe_status moe_routing_stats(const moe_layer_desc* desc, const float* logits, const int32_t* idx,
                             const int32_t* counts, double alpha, double* stats, int32_t* top3, double* prob_mean,
                             void* ws, size_t ws_bytes, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    if (d.T < 1) return fail(MOE_ERR_INVALID_ARG, "routing statistics need T >= 1");
    if (!logits || !idx || !counts || !stats || !top3)
        return fail(MOE_ERR_INVALID_ARG, "logits, idx, counts, stats and top3 are required");
    if (std::isnan(alpha) || std::isinf(alpha)) return fail(MOE_ERR_INVALID_ARG, "alpha must be finite");
    const size_t need = stats_workspace_bytes(d.T, d.N);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace too small for moe_routing_stats: need " + std::to_string(need));
    hipError_t e = launch_routing_stats(logits, idx, counts, d.T, d.N, d.k, alpha, ws, stats, top3, prob_mean,
                                        (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "routing statistics launch");
}

}  // extern "C"

namespace {
moe_status check_owner(const int32_t* owner, int N, int G) {
    if (G < 1 || G > MOE_EP_MAX_RANKS) return fail(MOE_ERR_INVALID_ARG, "G must satisfy 1 <= G <= 64");
    if (!owner) return fail(MOE_ERR_INVALID_ARG, "owner is NULL");
    for (int e = 0; e < N; ++e)
        if (owner[e] < 0 || owner[e] >= G)
            return fail(MOE_ERR_INVALID_ARG, "owner[" + std::to_string(e) + "] outside [0, G)");
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_ep_dispatch(const moe_layer_desc* desc, const int32_t* idx, const int32_t* owner, int32_t G,
                           int32_t* counts, int32_t* expert_offsets, int32_t* send_counts, int32_t* send_offsets,
                           int32_t* perm, int32_t* inv, const void* x, void* send_buf, moe_stream_t stream) {
    g_err.clear();
    moe_status st = check_desc(desc);
    if (st != MOE_OK) return st;
    const moe_layer_desc& d = *desc;
    if ((st = check_owner(owner, d.N, G)) != MOE_OK) return st;
    if (d.T == 0) return MOE_OK;
    if (!idx || !counts || !expert_offsets || !send_counts || !send_offsets || !perm || !inv)
        return fail(MOE_ERR_INVALID_ARG, "idx, counts, expert_offsets, send_counts, send_offsets, perm and inv are required");
    if ((x == nullptr) != (send_buf == nullptr)) return fail(MOE_ERR_INVALID_ARG, "give both x and send_buf or neither");
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_ep_dispatch(idx, d.T, d.k, d.N, owner, G, counts, expert_offsets, send_counts,
                                      send_offsets, perm, inv, s);
    if (e != hipSuccess) return hip_fail(e, "ep dispatch launch");
    if (send_buf) {
        // rows of every destination, in send order: send row r <- x[perm[r] / k], r < send_offsets[G]
        e = launch_gather_rows(x, perm, send_offsets, d.T, d.k, G, (int)(d.d * elem_bytes(d)), send_buf, s);
        if (e != hipSuccess) return hip_fail(e, "ep pack launch");
    }
    return MOE_OK;
}

moe_status moe_ep_receive_layout(int32_t N, int32_t G, const int32_t* owner, int32_t rank,
                                 const int32_t* recv_counts, int32_t max_rows, int32_t* recv_offsets,
                                 int32_t* local_offsets, int32_t* recv_perm, int32_t* recv_inv,
                                 moe_stream_t stream) {
    g_err.clear();
    if (N < 1 || N > 256) return fail(MOE_ERR_INVALID_ARG, "N must satisfy 1 <= N <= 256");
    moe_status st = check_owner(owner, N, G);
    if (st != MOE_OK) return st;
    if (rank < 0 || rank >= G) return fail(MOE_ERR_INVALID_ARG, "rank outside [0, G)");
    if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "max_rows < 0");
    if (!recv_counts || !recv_offsets || !local_offsets || (max_rows > 0 && (!recv_perm || !recv_inv)))
        return fail(MOE_ERR_INVALID_ARG, "recv_counts, recv_offsets, local_offsets, recv_perm and recv_inv are required");
    int n_local = 0;
    for (int e = 0; e < N; ++e) n_local += owner[e] == rank;
    if ((long long)G * n_local > 4096) return fail(MOE_ERR_UNSUPPORTED, "G * n_local > 4096");
    hipError_t e = launch_ep_receive_layout(recv_counts, N, G, owner, rank, max_rows, recv_offsets, local_offsets,
                                            recv_perm, recv_inv, (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ep receive layout launch");
}

moe_status moe_ep_unpack(int32_t G, int32_t max_rows, int32_t row_bytes, const int32_t* recv_offsets,
                         const int32_t* recv_inv, const void* y_grouped, void* ret, moe_stream_t stream) {
    g_err.clear();
    if (G < 1 || G > MOE_EP_MAX_RANKS) return fail(MOE_ERR_INVALID_ARG, "G must satisfy 1 <= G <= 64");
    if (max_rows < 0) return fail(MOE_ERR_INVALID_ARG, "max_rows < 0");
    if (row_bytes < 16 || row_bytes % 16 != 0) return fail(MOE_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 16");
    if (max_rows == 0) return MOE_OK;
    if (!recv_offsets || !recv_inv || !y_grouped || !ret)
        return fail(MOE_ERR_INVALID_ARG, "recv_offsets, recv_inv, y_grouped and ret are required");
    hipError_t e = launch_ep_unpack(y_grouped, recv_inv, recv_offsets, G, max_rows, row_bytes, ret,
                                    (hipStream_t)stream);
    return e == hipSuccess ? MOE_OK : hip_fail(e, "ep unpack launch");
}

const char* moe_status_str(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "unknown moe_status";
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

}  // extern "C"
