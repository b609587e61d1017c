// Steps 1-3 of the MoE layer: router logits, ranking + gating, expert capacity.
//
// Router: a learned linear layer scoring every expert per token (page "MoE 分片：混合專家模型的
// 平行化策略", section 什麼是 MoE 模型; page "MoE稀疏激活原理与工程实践", section 2.2).
// Gating: top-k with softmax over the kept logits (page "MoE 推理：激活参数 vs 总参数与专家路由",
// section 代码) or softmax over all logits then top-k without renormalisation (page
// "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析", section MoE核心机制).
// Capacity: a full expert passes the token on to its next-best expert (page "MoE稀疏激活原理与
// 工程实践", section 2.2).
#include "moe_common.h"
#include "moe_kernels.h"

// ------------------------------------------------------------------ router logits, bf16 (MFMA)
// Block = 4 waves; block tile = 128 tokens x 64 experts; wave w owns tokens [32w, 32w+32) of the
// tile and all 64 experts (4 MFMA column tiles of 16, 2 row tiles of 16).  Products are summed
// by v_mfma_f32_16x16x32_bf16 into fp32 over chunks of 256 inputs, and the chunk sums are added
// in fp64, which keeps the logit error far below the gaps that decide the ranking.  The final
// logit (plus bias, in fp64) is rounded once to fp32.
#define RL_BM 128
#define RL_BN 64
#define RL_CHUNK 256

__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ z, int T, int d, int N) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t0 = blockIdx.x * RL_BM + wave * 32;
    const int e0 = blockIdx.y * RL_BN;
    const int nct = min(4, (N - e0 + 15) >> 4);  // valid 16-wide column tiles (uniform)
    const int koff = (lane >> 4) * 8;
    const int rowA0 = t0 + (lane & 15), rowA1 = rowA0 + 16;
    const bool okA0 = rowA0 < T, okA1 = rowA1 < T;
    const bf16* pa0 = x + (size_t)(okA0 ? rowA0 : 0) * d + koff;
    const bf16* pa1 = x + (size_t)(okA1 ? rowA1 : 0) * d + koff;
    const bf16* pb[4];
    bool okB[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        int e = e0 + c * 16 + (lane & 15);
        okB[c] = (c < nct) && (e < N);
        pb[c] = wr + (size_t)(okB[c] ? e : 0) * d + koff;
    }
    double acc64[4][2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[c][r][i] = 0.0;

    const bf16x8 zero8 = {};
    for (int kc = 0; kc < d; kc += RL_CHUNK) {
        f32x4 acc[4][2];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c][0] = acc[c][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
        const int kend = min(kc + RL_CHUNK, d);
        for (int kk = kc; kk < kend; kk += 32) {
            bf16x8 a0 = okA0 ? *(const bf16x8*)(pa0 + kk) : zero8;
            bf16x8 a1 = okA1 ? *(const bf16x8*)(pa1 + kk) : zero8;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (c < nct) {
                    bf16x8 b = okB[c] ? *(const bf16x8*)(pb[c] + kk) : zero8;
                    acc[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[c][0], 0, 0, 0);
                    acc[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[c][1], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[c][r][i] += (double)acc[c][r][i];
    }
    // C layout of 16x16 MFMA: lane holds column (lane & 15), rows 4*(lane >> 4) + i.
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int e = e0 + c * 16 + (lane & 15);
        if (c >= nct || e >= N) continue;
        const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + r * 16 + 4 * (lane >> 4) + i;
                if (t < T) z[(size_t)t * N + e] = (float)(acc64[c][r][i] + b);
            }
    }
}

// ------------------------------------------------------------------ router logits, fp32
// One thread per (token, expert): fp32 FMA over chunks of 256 inputs, chunk sums added in fp64.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ z, int T, int d, int N) {
    const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= (long long)T * N) return;
    const int t = (int)(o / N), e = (int)(o % N);
    const float* xr = x + (size_t)t * d;
    const float* wv = wr + (size_t)e * d;
    double acc = 0.0;
    for (int kc = 0; kc < d; kc += RL_CHUNK) {
        float s = 0.f;
        const int kend = min(kc + RL_CHUNK, d);
        for (int i = kc; i < kend; ++i) s = fmaf(xr[i], wv[i], s);
        acc += (double)s;
    }
    if (bias) acc += (double)bias[e];
    z[o] = (float)acc;
}

// ------------------------------------------------------------------ top-k + gate weights
// One wave per token.  Each lane holds up to 4 logits (N <= 256) as 64-bit ranking keys
// (descending logit, then ascending expert id).  k rounds of a wave-wide max pick the slots in
// rank order.  Softmax in fp32 with the max subtracted.
__global__ __launch_bounds__(256) void topk_gate_kernel(
    const float* __restrict__ z, int T, int N, int k, int gating,
    int32_t* __restrict__ idx, float* __restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // whole wave leaves together; no block barrier below
    const float* zr = z + (size_t)t * N;
    uint64_t key[4];
    float zl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        zl[q] = e < N ? zr[e] : 0.f;
        key[q] = e < N ? rank_key(zl[q], e) : 0ull;
    }
    float zs[4] = {0.f, 0.f, 0.f, 0.f};  // the selected logits this lane records (slot j: lane j%64)
    int es[4] = {0, 0, 0, 0};
    float zmax = 0.f, sum_sel = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t m = key[0];
#pragma unroll
        for (int q = 1; q < 4; ++q) m = key[q] > m ? key[q] : m;
        const uint64_t best = wave_max_u64(m);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (key[q] == best) key[q] = 0ull;  // keys are unique: only the owner matches
        const float zb = key_logit(best);
        const int eb = key_expert(best);
        if (j == 0) zmax = zb;
        sum_sel += __expf(zb - zmax);
        if ((j & 63) == lane) {
            const int q = j >> 6;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                if (qq == q) { zs[qq] = zb; es[qq] = eb; }
        }
    }
    float denom = sum_sel;
    if (gating == 1) {  // softmax over all N logits
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (lane + 64 * q < N) s += __expf(zl[q] - zmax);
        denom = wave_sum_f32(s);
    }
    const float inv = 1.0f / denom;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = lane + 64 * q;
        if (j < k) {
            idx[(size_t)t * k + j] = es[q];
            w[(size_t)t * k + j] = __expf(zs[q] - zmax) * inv;
        }
    }
}

// ------------------------------------------------------------------ full ranking (capacity)
// One token per 64-thread block: bitonic sort of the N ranking keys in LDS, descending.
// ranked[t, r] = expert of rank r (uint8, N <= 256).
__global__ __launch_bounds__(64) void rank_sort_kernel(const float* __restrict__ z, int T, int N,
                                                       uint8_t* __restrict__ ranked) {
    __shared__ uint64_t key[MOE_MAX_EXPERTS];
    const int t = blockIdx.x, lane = threadIdx.x;
    int P = 2;
    while (P < N) P <<= 1;
    const float* zr = z + (size_t)t * N;
    for (int i = lane; i < P; i += 64) key[i] = i < N ? rank_key(zr[i], i) : 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int p = lane; p < (P >> 1); p += 64) {
                const int i = 2 * stride * (p / stride) + (p % stride);
                const int j = i + stride;
                const uint64_t a = key[i], b = key[j];
                const bool first_block = (i & size) == 0;
                if (first_block ? (a < b) : (a > b)) { key[i] = b; key[j] = a; }
            }
            __syncthreads();
        }
    }
    for (int r = lane; r < N; r += 64) ranked[(size_t)t * N + r] = (uint8_t)key_expert(key[r]);
}

// ------------------------------------------------------------------ capacity routing
// One block of 1024 threads.  Slots are placed pass by pass (all slot-0s in token order, then
// all slot-1s, ...).  Within a pass, tokens are taken in chunks of 1024 (one per thread); the
// chunk is resolved in parallel by deferred acceptance with token order as every expert's
// priority: each token proposes to its best expert that it does not hold, that had room at the
// start of the chunk and whose current cut-off tau[e] is not below the token; an expert keeps
// its (room)-th first proposers in token order and moves tau[e] to the last one kept.  tau only
// moves down, so a token never returns to an expert that turned it away, and the fixed point
// is the token-by-token first-come assignment.
#define CAP_THREADS 1024
#define CAP_WAVES (CAP_THREADS / 64)

__global__ __launch_bounds__(CAP_THREADS) void capacity_kernel(
    const uint8_t* __restrict__ ranked, const float* __restrict__ z, int T, int N, int k, int C,
    int gating, int32_t* __restrict__ idx, float* __restrict__ w) {
    __shared__ int fill[MOE_MAX_EXPERTS];
    __shared__ int tau[MOE_MAX_EXPERTS];
    __shared__ int wcnt[CAP_WAVES][MOE_MAX_EXPERTS];
    __shared__ uint32_t held[MOE_MAX_EXPERTS / 32][CAP_THREADS];  // experts the token already holds
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int e = tid; e < N; e += CAP_THREADS) fill[e] = 0;
    __syncthreads();

    for (int j = 0; j < k; ++j) {
        for (int c0 = 0; c0 < T; c0 += CAP_THREADS) {
            const int t = c0 + tid;
            const bool active = t < T;
#pragma unroll
            for (int q = 0; q < MOE_MAX_EXPERTS / 32; ++q) held[q][tid] = 0u;
            if (active)
                for (int jj = 0; jj < j; ++jj) {
                    const int e = idx[(size_t)t * k + jj];
                    if (e >= 0) held[e >> 5][tid] |= 1u << (e & 31);
                }
            for (int e = tid; e < N; e += CAP_THREADS) tau[e] = 0x7FFFFFFF;
            __syncthreads();
            int ptr = 0, choice = -1;
            bool choose = active;
            int total_e = 0;  // thread e < N: proposers of e in the last round
            while (true) {
                if (choose) {
                    choice = -1;
                    const uint8_t* rk = ranked + (size_t)t * N;
                    while (ptr < N) {
                        const int e = rk[ptr];
                        if (!((held[e >> 5][tid] >> (e & 31)) & 1u) && fill[e] < C && t <= tau[e]) {
                            choice = e;
                            break;
                        }
                        ++ptr;
                    }
                    choose = false;
                }
                for (int i = tid; i < CAP_WAVES * MOE_MAX_EXPERTS; i += CAP_THREADS)
                    (&wcnt[0][0])[i] = 0;
                __syncthreads();
                // rank of this proposal among the wave's proposals to the same expert
                const uint32_t v = (uint32_t)(choice + 1);  // 0 = no proposal
                const uint64_t eq = match_lanes<9>(v);
                const int rin = __popcll(eq & lanemask_lt());
                if (choice >= 0 && rin == 0) wcnt[wave][choice] = __popcll(eq);
                __syncthreads();
                if (tid < N) {  // exclusive prefix over waves, per expert
                    int s = 0;
                    for (int ww = 0; ww < CAP_WAVES; ++ww) {
                        const int c = wcnt[ww][tid];
                        wcnt[ww][tid] = s;
                        s += c;
                    }
                    total_e = s;
                }
                __syncthreads();
                bool rejected = false;
                if (choice >= 0) {
                    const int rank = wcnt[wave][choice] + rin;
                    const int room = C - fill[choice];
                    if (rank == room - 1) tau[choice] = t;
                    if (rank >= room) {
                        rejected = true;
                        ++ptr;
                        choose = true;
                    }
                }
                if (!__syncthreads_or(rejected)) break;
            }
            if (active) idx[(size_t)t * k + j] = choice;
            if (tid < N) fill[tid] += total_e;  // at the fixed point every proposal is kept
            __syncthreads();
        }
    }
    // gate weights over the final experts
    for (int t = tid; t < T; t += CAP_THREADS) {
        const float* zr = z + (size_t)t * N;
        int32_t* ir = idx + (size_t)t * k;
        float* wrow = w + (size_t)t * k;
        float zmax = -INFINITY;
        if (gating == 1) {
            for (int e = 0; e < N; ++e) zmax = fmaxf(zmax, zr[e]);
        } else {
            for (int j = 0; j < k; ++j)
                if (ir[j] >= 0) zmax = fmaxf(zmax, zr[ir[j]]);
        }
        float denom = 0.f;
        if (gating == 1) {
            for (int e = 0; e < N; ++e) denom += __expf(zr[e] - zmax);
        } else {
            for (int j = 0; j < k; ++j)
                if (ir[j] >= 0) denom += __expf(zr[ir[j]] - zmax);
        }
        for (int j = 0; j < k; ++j)
            wrow[j] = ir[j] >= 0 ? __expf(zr[ir[j]] - zmax) / denom : 0.f;
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_router_logits(const void* x, const void* wr, const float* bias, float* z, int T,
                                int d, int N, int dtype, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (dtype == 1) {
        dim3 grid((T + RL_BM - 1) / RL_BM, (N + RL_BN - 1) / RL_BN);
        hipLaunchKernelGGL(router_logits_bf16_kernel, grid, dim3(256), 0, s, (const bf16*)x,
                           (const bf16*)wr, bias, z, T, d, N);
    } else {
        const long long n = (long long)T * N;
        hipLaunchKernelGGL(router_logits_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                           s, (const float*)x, (const float*)wr, bias, z, T, d, N);
    }
    return hipGetLastError();
}

hipError_t launch_topk_gate(const float* z, int T, int N, int k, int gating, int32_t* idx, float* w,
                            hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, T, N, k, gating, idx, w);
    return hipGetLastError();
}

hipError_t launch_capacity(const float* z, uint8_t* ranked, int T, int N, int k, int C, int gating,
                           int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(rank_sort_kernel, dim3(T), dim3(64), 0, s, z, T, N, ranked);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(capacity_kernel, dim3(1), dim3(CAP_THREADS), 0, s, ranked, z, T, N, k, C,
                       gating, idx, w);
    return hipGetLastError();
}
