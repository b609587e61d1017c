// Expert-parallel receive side, on the rank that owns a set of experts (page "MoE 分片：混合專家
// 模型的平行化策略", sections 專家平行化詳解 and 動態 token 路由: tokens reach the GPUs that own their
// experts by one all-to-all, the expert outputs return by a second one).
//
// The receive buffer is source-major: source s's block holds, for each expert this rank owns in
// ascending expert id, that source's rows for the expert (in the source's slot order).  The
// grouped FFN wants every local expert's rows together, so the layout kernel gives the grouped
// order (local expert, then source, then the source's order) as a row list into the receive
// buffer, the per-expert offsets of that order and its inverse.  Both orders cut the rows into
// (source, local expert) pairs of consecutive rows, so their starts are exclusive scans of the
// count matrix taken in two orders.  After the FFN, the unpack kernel
// puts the expert outputs back into receive order, which is the order the return exchange
// carries them in.
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int RL_THREADS = 1024;

// This rank's experts in ascending id (built on the host, passed by value).
struct LocalExperts {
    int e[MOE_MAX_EXPERTS];
    int n;
};

constexpr int RL_ROWS = 4 * RL_THREADS;   // grouped rows per block

// In-place exclusive scan of v[0..n) (n <= MOE_EP_MAX_BLOCKS) by the whole block, 4 values per
// thread; returns the total.  `tmp` holds one value per wave.
__device__ int block_exclusive_scan(int* v, int n, int* tmp) {
    const int tid = threadIdx.x, lane = tid & (WAVE - 1), wv = tid / WAVE;
    int loc[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * 4 + q;
        loc[q] = i < n ? v[i] : 0;
        sum += loc[q];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        const int u = __shfl_up(incl, o, WAVE);
        if (lane >= o) incl += u;
    }
    if (lane == WAVE - 1) tmp[wv] = incl;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < RL_THREADS / WAVE; ++w) {
            const int t = tmp[w];
            tmp[w] = run;
            run += t;
        }
        tmp[RL_THREADS / WAVE] = run;
    }
    __syncthreads();
    int run = tmp[wv] + incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int i = tid * 4 + q;
        if (i < n) v[i] = run;
        run += loc[q];
    }
    const int total = tmp[RL_THREADS / WAVE];
    __syncthreads();
    return total;
}

// recv_counts [G][N]: the full per-expert counts of every source (the count exchange).
// Pair (s, le) = source s, local expert le.  Receive order lists the pairs source-major, the
// grouped order expert-major; each block rebuilds both start tables (two exclusive scans of the
// G x n_local counts) and then places its RL_ROWS grouped rows.
__global__ __launch_bounds__(RL_THREADS) void ep_receive_layout_kernel(
    const int32_t* __restrict__ recv_counts, int N, int G, const LocalExperts loc, int max_rows,
    int32_t* __restrict__ recv_offsets, int32_t* __restrict__ local_offsets, int32_t* __restrict__ recv_perm,
    int32_t* __restrict__ recv_inv) {
    __shared__ int s_rs[MOE_EP_MAX_BLOCKS];   // receive-order start of pair (s, le), index s * NL + le
    __shared__ int s_gs[MOE_EP_MAX_BLOCKS];   // grouped start of pair (s, le), index le * G + s
    __shared__ int s_tmp[RL_THREADS / WAVE + 1];
    const int tid = threadIdx.x;
    const int NL = loc.n;
    const int nb = NL * G;
    for (int i = tid; i < nb; i += RL_THREADS) {
        const int s = i / NL, le = i % NL;
        const int c = recv_counts[(size_t)s * N + loc.e[le]];
        s_rs[i] = c;
        s_gs[le * G + s] = c;
    }
    __syncthreads();
    const int total = block_exclusive_scan(s_rs, nb, s_tmp);
    block_exclusive_scan(s_gs, nb, s_tmp);
    if (blockIdx.x == 0) {
        for (int s = tid; s <= G; s += RL_THREADS) recv_offsets[s] = (s < G && NL > 0) ? s_rs[s * NL] : (s < G ? 0 : total);
        for (int le = tid; le <= NL; le += RL_THREADS) local_offsets[le] = le < NL ? s_gs[le * G] : total;
    }
    const int R = min(total, max_rows);
    const int g0 = blockIdx.x * RL_ROWS;
#pragma unroll
    for (int q = 0; q < RL_ROWS / RL_THREADS; ++q) {
        const int g = g0 + q * RL_THREADS + tid;
        if (g >= R) break;
        // the pair holding grouped row g: the last one (in grouped order) starting at or before g
        int lo = 0, hi = nb - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_gs[mid] <= g) lo = mid; else hi = mid - 1;
        }
        const int le = lo / G, s = lo % G;
        const int r = s_rs[s * NL + le] + (g - s_gs[lo]);
        recv_perm[g] = r;
        if (r < max_rows) recv_inv[r] = g;
    }
}

// ret[r] = y_grouped[recv_inv[r]] for r < min(recv_offsets[G], max_rows); 16-byte rows.
__global__ __launch_bounds__(256) void ep_unpack_kernel(const uint8_t* __restrict__ yg,
                                                        const int32_t* __restrict__ recv_inv,
                                                        const int32_t* __restrict__ recv_offsets, int G,
                                                        int max_rows, int row_bytes, uint8_t* __restrict__ ret) {
    const int r = blockIdx.x;
    const int R = min(recv_offsets[G], max_rows);
    if (r >= R) return;
    const int g = recv_inv[r];
    if (g < 0 || g >= R) return;   // only when the layout was cut at max_rows
    const u32x4* src = (const u32x4*)(yg + (size_t)g * row_bytes);
    u32x4* dst = (u32x4*)(ret + (size_t)r * row_bytes);
    for (int i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

}  // namespace

hipError_t launch_ep_receive_layout(const int32_t* recv_counts, int N, int G, const int32_t* owner, int rank,
                                    int max_rows, int32_t* recv_offsets, int32_t* local_offsets,
                                    int32_t* recv_perm, int32_t* recv_inv, hipStream_t s) {
    LocalExperts loc{};
    for (int e = 0; e < N; ++e)
        if (owner[e] == rank) loc.e[loc.n++] = e;
    const int blocks = max_rows > 0 ? (max_rows + RL_ROWS - 1) / RL_ROWS : 1;
    ep_receive_layout_kernel<<<blocks, RL_THREADS, 0, s>>>(recv_counts, N, G, loc, max_rows, recv_offsets,
                                                           local_offsets, recv_perm, recv_inv);
    return hipGetLastError();
}

hipError_t launch_ep_unpack(const void* y_grouped, const int32_t* recv_inv, const int32_t* recv_offsets, int G,
                            int max_rows, int row_bytes, void* ret, hipStream_t s) {
    if (max_rows == 0) return hipSuccess;
    ep_unpack_kernel<<<max_rows, 256, 0, s>>>((const uint8_t*)y_grouped, recv_inv, recv_offsets, G, max_rows,
                                              row_bytes, (uint8_t*)ret);
    return hipGetLastError();
}
