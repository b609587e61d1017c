// Routing health statistics of one layer call: the experts' load shares and their entropy, the
// three most used experts, the spread of the per-expert counts, the value of the load-balancing
// loss and the share of slots that did not get their own ranked choice.
//   entropy and top-3 share: page "MoE稀疏激活原理与工程实践：揭秘大模型参数幻觉", section 4.2
//     (routing diagnosis), which also uses std/mean of the counts in its online calibration;
//   balance loss alpha * N * sum_i f_i p_i: page "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析",
//     section MoE核心机制;
//   re-route share: page "MoE稀疏激活原理与工程实践", section 2.2 (a full expert passes the token
//     on to its next choice) and section 3.3 (the re-route rate it monitors).
// Two kernels, both deterministic (fixed summation order, no atomics):
//   stats_tokens: a group of lanes per token (several tokens per wave when N <= 32); fp64 softmax over the token's N logits accumulated per
//     expert, and per slot whether idx[t, j] is one of the token's k best-ranked experts.  Each block writes
//     its partial sums (fp64 per expert, int64 re-route count) to the workspace.
//   stats_finish: one block of 1024 threads sums the partials in block order and derives the
//     eight statistics and the top-3 ids from the counts.
#include <math.h>

#include "moe_common.h"
#include "moe_kernels.h"

namespace {

constexpr int ST_THREADS = 1024;         // token pass: 16 waves
constexpr int ST_WAVES = ST_THREADS / WAVE;
constexpr int ST_MAX_BLOCKS = 256;
constexpr int ST_BATCH = 2;              // token passes whose inputs a wave loads before using them
constexpr int FIN_THREADS = 1024;
constexpr int FIN_GROUPS = FIN_THREADS / MOE_MAX_EXPERTS;
constexpr int FIN_UNROLL = 8;            // partial sums in flight per thread

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = __shfl_xor((uint32_t)u, m, WAVE);
    const uint32_t hi = __shfl_xor((uint32_t)(u >> 32), m, WAVE);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
// Reductions over the G lanes of one group (G a power of two dividing 64), fixed order.
template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v += shfl_xor_f64(v, m);
    return v;
}
template <int G>
__device__ __forceinline__ float group_max_f32(float v) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
    return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) { return group_sum_f64<WAVE>(v); }

// Per-block partials: prob[b][e] (fp64, stride N) then rerouted[b] (int64).
struct StatsWs {
    double* prob;
    long long* rerouted;
};
__host__ __device__ inline StatsWs stats_ws(void* ws, int B, int N) {
    StatsWs w;
    w.prob = (double*)ws;
    const size_t off = (((size_t)B * N * sizeof(double)) + 255) & ~(size_t)255;
    w.rerouted = (long long*)((char*)ws + off);
    return w;
}

// Lanes per token: the power of two >= N up to 32 experts (several tokens per wave), else the
// whole wave with ceil(N / 64) experts per lane.
int stats_group(int N) {
    if (N > 32) return WAVE;
    int g = 1;
    while (g < N) g <<= 1;
    return g;
}
int stats_blocks(int T, int N) {
    const int per_block = ST_WAVES * ST_BATCH * (WAVE / stats_group(N));   // tokens of one pass
    const int b = (T + per_block - 1) / per_block;
    return b < 1 ? 1 : (b > ST_MAX_BLOCKS ? ST_MAX_BLOCKS : b);
}

// Lane l of a wave works on token group l / G; it holds experts (l % G) + G * j, j < J (those
// below N), and slots (l % G) + G * j of that token's k slots.
template <int J, int G>
__global__ __launch_bounds__(ST_THREADS) void stats_tokens(const float* __restrict__ z,
                                                           const int32_t* __restrict__ idx, int T, int N,
                                                           int k, void* ws) {
    constexpr int TPW = WAVE / G;                // tokens per wave and pass
    constexpr int PER_WAVE = ST_BATCH * TPW;     // tokens per wave and batch
    __shared__ double s_prob[ST_WAVES][MOE_MAX_EXPERTS];
    __shared__ long long s_rr[ST_WAVES];
    const int lane = threadIdx.x & (WAVE - 1);
    const int wv = threadIdx.x / WAVE;
    const int gi = lane / G, li = lane % G;
    const int gbase = gi * G;
    const uint64_t gmask = (G == WAVE) ? ~0ull : (((1ull << G) - 1ull) << gbase);
    const int B = gridDim.x;
    // contiguous token range of this block
    const int t0 = (int)(((long long)T * blockIdx.x) / B);
    const int t1 = (int)(((long long)T * (blockIdx.x + 1)) / B);

    double acc[J];
#pragma unroll
    for (int j = 0; j < J; ++j) acc[j] = 0.0;
    long long rr = 0;

    for (int tb = t0 + wv * PER_WAVE; tb < t1; tb += ST_WAVES * PER_WAVE) {
        float v[ST_BATCH][J];
        int iv[ST_BATCH][J];
#pragma unroll
        for (int u = 0; u < ST_BATCH; ++u) {
            const int t = tb + u * TPW + gi;
            const bool tv = t < t1;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = li + G * j;
                // a lane past the block's tokens holds 0 (its group's max stays finite)
                v[u][j] = tv ? (e < N ? z[(size_t)t * N + e] : -INFINITY) : 0.0f;
                iv[u][j] = (tv && e < k) ? idx[(size_t)t * k + e] : -1;
            }
        }
#pragma unroll
        for (int u = 0; u < ST_BATCH; ++u) {
            const bool tv = tb + u * TPW + gi < t1;
            if (!__any(tv)) break;                    // wave-uniform
            float m = v[u][0];
#pragma unroll
            for (int j = 1; j < J; ++j) m = fmaxf(m, v[u][j]);
            m = group_max_f32<G>(m);
            double ex[J];
            double s = 0.0;
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = li + G * j;
                ex[j] = e < N ? exp((double)v[u][j] - (double)m) : 0.0;
                s += ex[j];
            }
            s = group_sum_f64<G>(s);
            const double inv = 1.0 / s;
            if (tv) {
#pragma unroll
                for (int j = 0; j < J; ++j) acc[j] += ex[j] * inv;
            }

            // a slot keeps an own choice iff idx[t, j] is a valid expert ranked among the token's
            // k best: rank(e) = number of experts ahead of e (larger logit, or equal logit and
            // lower id) < k.  Its position j does not matter (capacity fills slots in passes).
            uint64_t key[J];
#pragma unroll
            for (int j = 0; j < J; ++j) {
                const int e = li + G * j;
                key[j] = e < N ? rank_key(v[u][j], e) : 0ull;
            }
            for (int sl = 0; sl < k; ++sl) {
                const int src = gbase + (sl % G);
                int e = -1;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const int ej = __shfl(iv[u][j], src, WAVE);
                    if (sl / G == j) e = ej;
                }
                const bool valid = e >= 0 && e < N;
                const int ec = valid ? e : 0;
                float ze = 0.0f;
#pragma unroll
                for (int j = 0; j < J; ++j) {
                    const float zj = __shfl(v[u][j], gbase + (ec % G), WAVE);
                    if (ec / G == j) ze = zj;
                }
                const uint64_t ke = rank_key(ze, ec);
                int ahead = 0;
#pragma unroll
                for (int j = 0; j < J; ++j) ahead += __popcll(__ballot(key[j] > ke) & gmask);
                const bool own = valid && ahead < k;
                rr += (tv && li == 0 && !own) ? 1 : 0;
            }
        }
    }
    // experts are held by the same lane index in every group: fold the groups, fixed order
#pragma unroll
    for (int j = 0; j < J; ++j) {
#pragma unroll
        for (int m = WAVE / 2; m >= G; m >>= 1) acc[j] += shfl_xor_f64(acc[j], m);
    }
#pragma unroll
    for (int m = WAVE / 2; m >= 1; m >>= 1) rr += __shfl_xor(rr, m, WAVE);
    if (gi == 0) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int e = li + G * j;
            if (e < N) s_prob[wv][e] = acc[j];
        }
    }
    if (lane == 0) s_rr[wv] = rr;
    __syncthreads();
    const StatsWs w = stats_ws(ws, B, N);
    for (int e = threadIdx.x; e < N; e += ST_THREADS) {
        double p = s_prob[0][e];
#pragma unroll
        for (int q = 1; q < ST_WAVES; ++q) p += s_prob[q][e];
        w.prob[(size_t)blockIdx.x * N + e] = p;
    }
    if (threadIdx.x == 0) {
        long long r = 0;
        for (int q = 0; q < ST_WAVES; ++q) r += s_rr[q];
        w.rerouted[blockIdx.x] = r;
    }
}

// Sum of s[0..255] (double) by wave 0, fixed order; valid in wave 0's lanes.
__device__ __forceinline__ double wave0_sum256(const double* s, int lane) {
    return wave_sum_f64((s[lane] + s[lane + 64]) + (s[lane + 128] + s[lane + 192]));
}

__global__ __launch_bounds__(FIN_THREADS) void stats_finish(const int32_t* __restrict__ counts, int T, int N,
                                                            int k, int B, double alpha, const void* ws,
                                                            double* __restrict__ stats,
                                                            int32_t* __restrict__ top3,
                                                            double* __restrict__ prob_mean) {
    __shared__ double s_part[FIN_GROUPS][MOE_MAX_EXPERTS];
    __shared__ double s_a[MOE_MAX_EXPERTS], s_b[MOE_MAX_EXPERTS], s_c[MOE_MAX_EXPERTS];
    __shared__ long long s_cnt[MOE_MAX_EXPERTS];
    __shared__ unsigned long long s_key[MOE_MAX_EXPERTS];
    __shared__ long long s_S, s_rr;
    const int tid = threadIdx.x;
    const int lane = tid & (WAVE - 1);
    const int e = tid % MOE_MAX_EXPERTS;
    const int g = tid / MOE_MAX_EXPERTS;
    const StatsWs w = stats_ws(const_cast<void*>(ws), B, N);

    // 1. probability sums: group g takes blocks g, g + 4, ... in order
    double p = 0.0;
    if (e < N) {
        // blocks g, g + 4, ... in order, FIN_UNROLL loads in flight (an absent block adds 0.0)
        for (int b0 = g; b0 < B; b0 += FIN_GROUPS * FIN_UNROLL) {
            double part[FIN_UNROLL];
#pragma unroll
            for (int q = 0; q < FIN_UNROLL; ++q) {
                const int b = b0 + FIN_GROUPS * q;
                part[q] = b < B ? w.prob[(size_t)b * N + e] : 0.0;
            }
#pragma unroll
            for (int q = 0; q < FIN_UNROLL; ++q) p += part[q];
        }
    }
    s_part[g][e] = p;
    if (tid < MOE_MAX_EXPERTS) s_cnt[tid] = tid < N ? (long long)counts[tid] : 0;
    __syncthreads();

    // 2. totals: slots kept (S) and re-routed slots
    if (tid < WAVE) {
        long long c = (s_cnt[lane] + s_cnt[lane + 64]) + (s_cnt[lane + 128] + s_cnt[lane + 192]);
        long long r = 0;
        for (int b = lane; b < B; b += WAVE) r += w.rerouted[b];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            c += __shfl_xor(c, m, WAVE);
            r += __shfl_xor(r, m, WAVE);
        }
        if (lane == 0) { s_S = c; s_rr = r; }
    }
    __syncthreads();

    // 3. per-expert terms: entropy, squared deviation of the count, f_i * p_i
    const long long S = s_S;
    const double Sd = (double)S;
    const double mean = Sd / N;
    if (tid < MOE_MAX_EXPERTS) {
        double ent = 0.0, dev = 0.0, fp = 0.0;
        if (tid < N) {
            const double pm = (((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid]) / T;
            if (prob_mean) prob_mean[tid] = pm;
            const long long c = s_cnt[tid];
            const double share = (double)c / Sd;
            if (c > 0) ent = -share * log2(share);
            const double dc = (double)c - mean;
            dev = dc * dc;
            fp = share * pm;
        }
        s_a[tid] = ent;
        s_b[tid] = dev;
        s_c[tid] = fp;
        // top-3 key: count descending, then id ascending
        s_key[tid] = tid < N ? (((unsigned long long)s_cnt[tid] << 16) | (0xFFFFu - (unsigned)tid)) : 0ull;
    }
    __syncthreads();
    if (tid < WAVE) {
        const double ent = wave0_sum256(s_a, lane);
        const double dev = wave0_sum256(s_b, lane);
        const double fp = wave0_sum256(s_c, lane);
        // top 3 by three rounds of a wave-wide maximum over the 256 keys
        unsigned long long kq[4] = {s_key[lane], s_key[lane + 64], s_key[lane + 128], s_key[lane + 192]};
        long long topc = 0;
        int ids[3];
        for (int r = 0; r < 3; ++r) {
            unsigned long long mx = kq[0];
#pragma unroll
            for (int q = 1; q < 4; ++q) mx = kq[q] > mx ? kq[q] : mx;
            mx = wave_max_u64(mx);
            const bool valid = r < N;                 // keys of experts >= N are 0 and never win
            ids[r] = valid ? (int)(0xFFFFu - (unsigned)(mx & 0xFFFFu)) : -1;
            if (valid) topc += (long long)(mx >> 16);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (valid && kq[q] == mx) kq[q] = 0ull;
        }
        int touched = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) touched += __popcll(__ballot(s_cnt[lane + 64 * q] > 0));
        long long cmax = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) cmax = s_cnt[lane + 64 * q] > cmax ? s_cnt[lane + 64 * q] : cmax;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const long long o = __shfl_xor(cmax, m, WAVE);
            cmax = o > cmax ? o : cmax;
        }
        if (lane == 0) {
            // no kept slot: every share is undefined
            stats[0] = S > 0 ? ent : __builtin_nan("");
            stats[1] = log2((double)N);
            stats[2] = (double)topc / Sd;
            stats[3] = (double)cmax / Sd;
            stats[4] = sqrt(dev / N) / mean;
            stats[5] = alpha * N * fp;
            stats[6] = (double)s_rr / ((double)T * (double)k);
            stats[7] = (double)touched;
            top3[0] = ids[0];
            top3[1] = ids[1];
            top3[2] = ids[2];
        }
    }
}

}  // namespace

size_t stats_workspace_bytes(int T, int N) {
    const int B = stats_blocks(T, N);
    return ((((size_t)B * N * sizeof(double)) + 255) & ~(size_t)255) + (size_t)B * sizeof(long long);
}

hipError_t launch_routing_stats(const float* z, const int32_t* idx, const int32_t* counts, int T, int N, int k,
                                double alpha, void* ws, double* stats, int32_t* top3, double* prob_mean,
                                hipStream_t s) {
    const int B = stats_blocks(T, N);
    const int G = stats_group(N);
    switch (G) {
        case 1: stats_tokens<1, 1><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        case 2: stats_tokens<1, 2><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        case 4: stats_tokens<1, 4><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        case 8: stats_tokens<1, 8><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        case 16: stats_tokens<1, 16><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        case 32: stats_tokens<1, 32><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
        default:
            switch ((N + WAVE - 1) / WAVE) {
                case 1: stats_tokens<1, WAVE><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
                case 2: stats_tokens<2, WAVE><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
                case 3: stats_tokens<3, WAVE><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
                default: stats_tokens<4, WAVE><<<B, ST_THREADS, 0, s>>>(z, idx, T, N, k, ws); break;
            }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    stats_finish<<<1, FIN_THREADS, 0, s>>>(counts, T, N, k, B, alpha, ws, stats, top3, prob_mean);
    return hipGetLastError();
}
