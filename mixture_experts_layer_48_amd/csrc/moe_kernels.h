// Host-side launchers of the MoE kernels (one per .hip file group).  All enqueue on `s` and
// return the launch status; none synchronises.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// workspace of the router: fp64 partial logits [K parts, T, N] when K is split, else nothing
size_t router_workspace_bytes(int T, int d, int N, int dtype);
// sum_parts false: with K split (router_k_parts > 1) only the fp64 part sums are written (to ws),
// for launch_route_finish_small to add up
hipError_t launch_router_logits(const void* x, const void* wr, const float* bias, float* z, void* ws,
                                int T, int d, int N, int dtype, hipStream_t s, bool sum_parts = true);
int router_k_parts(int T, int d, int N, int dtype);
// the fp64 K-part sums of launch_router_logits (sum_parts false, ks > 1) summed into z and ranked:
// idx / w [T, k], one launch
hipError_t launch_reduce_topk(const void* part, int ks, const float* bias, float* z, int T, int N, int k,
                             int gating, int32_t* idx, float* w, hipStream_t s);
// a batch of at most 512 slots and 8192 logits: the K-part sum (when ks > 1), top-k, gate
// weights and the grouping (counts, offsets, perm, inv) in one single-block launch
bool route_finish_small_supported(int T, int N, int k);
hipError_t launch_route_finish_small(const void* part, int ks, const float* bias, float* z, int T, int N, int k,
                                     int gating, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                                     int32_t* perm, int32_t* inv, hipStream_t s);
hipError_t launch_topk_gate(const float* z, int T, int N, int k, int gating, int32_t* idx, float* w,
                            hipStream_t s);
// Router GEMM fused with top-k and softmax (bf16, N in {64, 128, 256}): writes the logits to z
// only if z is not null, and the routing (idx, w) only if idx is not null.
bool router_fused_supported(int N, int dtype);
hipError_t launch_router_topk(const void* x, const void* wr, const float* bias, float* z, int T, int d, int N,
                              int k, int gating, int32_t* idx, float* w, hipStream_t s);
// workspace of the capacity step: ranked lists [T, capacity_ranked_stride(N)] bytes, then [T]
int capacity_ranked_stride(int N);
size_t capacity_workspace_bytes(int T, int N);
hipError_t launch_capacity(const float* z, uint8_t* ranked, int T, int N, int k, int C, int gating,
                           int32_t* idx, float* w, hipStream_t s);
hipError_t launch_permute(const int32_t* idx, int T, int k, int N, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t s);
// the same grouping over many blocks (for large T * k): per-block counts in ws, [ceil(T*k/1024), N]
// int32 (permute_multi_workspace_bytes), then a scan and the placement; bit-identical results
size_t permute_multi_workspace_bytes(int T, int k, int N);
hipError_t launch_permute_multi(const int32_t* idx, int T, int k, int N, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* ws, hipStream_t s);
hipError_t launch_gather_rows(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                              int k, int N, int row_bytes, void* x_perm, hipStream_t s);

// Int4 expert weights (codes [mats, rows, K/8] uint32, scales [mats, K/128, rows] fp32).
struct FfnQ4Weights {
    const uint32_t *gate, *up, *down, *sh_gate, *sh_up, *sh_down;
    const float *gate_scales, *up_scales, *down_scales, *sh_gate_scales, *sh_up_scales, *sh_down_scales;
};

// Grouped expert FFN.  Segment e < N: rows offsets[e] .. offsets[e+1]-1, weights of expert e;
// segment N (has_shared): rows T*k .. T*k+T-1, the shared expert's weights.
struct FfnLaunch {
    int T, d, N, k, d_ff, dtype, ffn, has_shared;
    const void* x;            // [T, d]
    const int32_t* perm;      // [T*k]
    const int32_t* offsets;   // [N+1]
    const void* w_gate;       // [N, d, d_ff] or null (x W orientation: K-major)
    const void* w_up;         // [N, d, d_ff]
    const void* w_down;       // [N, d_ff, d]
    const void* sh_gate;      // [d, d_ff] or null
    const void* sh_up;
    const void* sh_down;
    const float* row_scale;   // [T*k] or null
    void* h;                  // [T*k + T, d_ff] hidden state
    void* y_perm;             // [ksplit][T*k + T, d] fp32 (ksplit partial sums); with routed
                              // rows in bf16 (ffn_out_routed_bf16), row r < T*k is bf16 at element
                              // r*d of the buffer viewed as bf16, the shared rows stay fp32
    int ksplit;               // K parts of the out-projection (1 = y_perm holds the result)
    int routed_bf16_ok;       // the caller reads routed rows in bf16 where ffn_out_routed_bf16 says so
    unsigned int* ctr;        // the tiled GEMMs' schedule memory (claim counters, then a tile
    size_t sched_bytes;       // table), sched_bytes >= ffn_sched_bytes(); set up by the launches
    FfnQ4Weights q4;          // int4 weights (the q4 launchers only)
};
int ffn_out_ksplit(int T, int k, int N, int d, int d_ff, int has_shared, int dtype);
int ffn_out_routed_bf16(const FfnLaunch& f);   // 1: launch_ffn_out stores routed rows in bf16
#define FFN_CTR_BYTES 256
size_t ffn_sched_bytes(int T, int k, int N, int d, int d_ff, int has_shared, int ksplit);
hipError_t launch_ffn_in(const FfnLaunch& a, hipStream_t s);   // H = act(x W_in)
hipError_t launch_ffn_out(const FfnLaunch& a, hipStream_t s);  // y_perm = scale * H W_out
hipError_t launch_combine(const void* y_perm, const int32_t* inv, const float* w, void* y, int T,
                          int k, int d, int has_shared, int dtype, int nparts, int routed_bf16, hipStream_t s);

// Routing statistics: workspace of per-block partial sums, then the two-kernel launch.
size_t stats_workspace_bytes(int T, int N);
hipError_t launch_routing_stats(const float* z, const int32_t* idx, const int32_t* counts, int T, int N, int k,
                                double alpha, void* ws, double* stats, int32_t* top3, double* prob_mean,
                                hipStream_t s);

// Expert parallelism: send layout keyed by (owner rank, expert) (owner: host array [N], values in
// [0, G)); receive layout over the sources' count vectors; unpack of the grouped expert outputs
// into receive order.
hipError_t launch_ep_dispatch(const int32_t* idx, int T, int k, int N, const int32_t* owner, int G,
                              int32_t* counts, int32_t* expert_offsets, int32_t* send_counts,
                              int32_t* send_offsets, int32_t* perm, int32_t* inv, hipStream_t s);
hipError_t launch_ep_receive_layout(const int32_t* recv_counts, int N, int G, const int32_t* owner, int rank,
                                    int max_rows, int32_t* recv_offsets, int32_t* local_offsets,
                                    int32_t* recv_perm, int32_t* recv_inv, hipStream_t s);
hipError_t launch_ep_unpack(const void* y_grouped, const int32_t* recv_inv, const int32_t* recv_offsets, int G,
                            int max_rows, int row_bytes, void* ret, hipStream_t s);

// Int4 expert weights: quantisation of n_mats bf16 matrices [K, rows] (K % 128 == 0), and the
// weight-streaming expert FFN on int4 weights (f.q4; the out-projection always in one K part).
hipError_t launch_q4_quantize(const void* w, long long n_mats, int rows, int K, uint32_t* codes, float* scales,
                              hipStream_t s);
hipError_t launch_ffn_in_q4(const FfnLaunch& f, hipStream_t s);
hipError_t launch_ffn_out_q4(const FfnLaunch& f, hipStream_t s);
