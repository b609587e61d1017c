// Steps 1-3 of the MoE layer: router logits, ranking + gating, expert capacity.
//
// Router: a learned linear layer scoring every expert per token (page "MoE 分片：混合專家模型的
// 平行化策略", section 什麼是 MoE 模型; page "MoE稀疏激活原理与工程实践", section 2.2).
// Gating: top-k with softmax over the kept logits (page "MoE 推理：激活参数 vs 总参数与专家路由",
// section 代码) or softmax over all logits then top-k without renormalisation (page
// "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析", section MoE核心机制).
// Capacity: a full expert passes the token on to its next-best expert (page "MoE稀疏激活原理与
// 工程实践", section 2.2).
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

// ------------------------------------------------------------------ router logits, bf16 (MFMA)
// Work unit = one wave: 32 tokens (2 MFMA row tiles of 16) x 64 experts (4 column tiles of 16) x
// one range of K.  Products are summed by v_mfma_f32_16x16x32_bf16 into fp32 over chunks of 256
// inputs and the chunk sums are added in fp64, which keeps the logit error far below the gaps
// that decide the ranking.  When the grid would be too small to fill the chip (few tokens or
// experts) K is split into parts: each part's fp64 sum goes to the workspace and a second kernel
// adds the parts in part order plus the bias; otherwise the unit adds the bias and writes the
// logit, rounded once to fp32.  Units are numbered expert tile fastest, so the waves of one block
// share their token rows through the cache.
#define RL_BM 32
#define RL_BN 64
#define RL_CHUNK 256
#define RL_TARGET_WAVES 2048

struct RouterSplit {
    int n_tt, n_et, nchunks, ks, cpp;   // token tiles, expert tiles, chunks, K parts, chunks per part
};
static RouterSplit router_split(int T, int d, int N) {
    RouterSplit r;
    r.n_tt = (T + RL_BM - 1) / RL_BM;
    r.n_et = (N + RL_BN - 1) / RL_BN;
    r.nchunks = (d + RL_CHUNK - 1) / RL_CHUNK;
    const long long per_part = (long long)r.n_tt * r.n_et;
    long long ks = (RL_TARGET_WAVES + per_part - 1) / per_part;
    if (ks > r.nchunks) ks = r.nchunks;
    if (ks < 1) ks = 1;
    r.cpp = (int)((r.nchunks + ks - 1) / ks);
    r.ks = (r.nchunks + r.cpp - 1) / r.cpp;
    return r;
}

size_t router_workspace_bytes(int T, int d, int N, int dtype) {
    if (dtype != 1 || T == 0) return 0;
    const RouterSplit r = router_split(T, d, N);
    return r.ks > 1 ? (size_t)r.ks * T * N * sizeof(double) : 0;
}

// One wave: NCT column tiles of 16 experts (NCT = 4 except on a partial last expert tile) of
// its expert tile, for tokens t0 .. t0 + 31, over its K part.  Rows past T and experts past N
// load clamped (valid) addresses and their results are never stored, so every load is
// unconditional and the wait counts stay exact: the fragments of the next 32-input step are
// loaded while the current step's MFMAs run.
template <int NCT>
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ z, double* __restrict__ part, int T, int d, int N, RouterSplit sp, int et_beg,
    int n_et) {
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int et = et_beg + u % n_et, rest = u / n_et;
    const int kp = rest % sp.ks, tt = rest / sp.ks;
    if (tt >= sp.n_tt) return;
    const int t0 = tt * RL_BM, e0 = et * RL_BN;
    const int koff = (lane >> 4) * 8;
    const int rowA0 = t0 + (lane & 15), rowA1 = rowA0 + 16;
    const bf16* pa0 = x + (size_t)(rowA0 < T ? rowA0 : 0) * d + koff;
    const bf16* pa1 = x + (size_t)(rowA1 < T ? rowA1 : 0) * d + koff;
    const bf16* pb[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int e = e0 + c * 16 + (lane & 15);
        pb[c] = wr + (size_t)(e < N ? e : 0) * d + koff;
    }
    double acc64[NCT][2][4];
    f32x4 acc[NCT][2];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            acc[c][r] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[c][r][i] = 0.0;
        }
    struct Frag {
        bf16x8 a0, a1, b[NCT];
    };
    auto load = [&](Frag& f, int k) {
        f.a0 = *(const bf16x8*)(pa0 + k);
        f.a1 = *(const bf16x8*)(pa1 + k);
#pragma unroll
        for (int c = 0; c < NCT; ++c) f.b[c] = *(const bf16x8*)(pb[c] + k);
    };
    auto mma = [&](const Frag& f) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) {
            acc[c][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a0, f.b[c], acc[c][0], 0, 0, 0);
            acc[c][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a1, f.b[c], acc[c][1], 0, 0, 0);
        }
    };
    // the fp32 sum of a chunk of RL_CHUNK inputs goes into the fp64 sum, in chunk order
    auto fold = [&]() {
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[c][r][i] += (double)acc[c][r][i];
                acc[c][r] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
    };
    constexpr int SPC = RL_CHUNK / 32;            // 32-input steps per chunk
    const int kbeg = kp * sp.cpp * RL_CHUNK;
    const int kend = min(kbeg + sp.cpp * RL_CHUNK, d);
    const int nsteps = (kend - kbeg) / 32;        // d % 64 == 0 for bf16 layers
    Frag f0, f1;
    load(f0, kbeg);
    int st = 0;
    for (; st + 2 <= nsteps; st += 2) {
        load(f1, kbeg + 32 * (st + 1));
        mma(f0);
        if ((st + 1) % SPC == 0) fold();
        if (st + 2 < nsteps) load(f0, kbeg + 32 * (st + 2));
        mma(f1);
        if ((st + 2) % SPC == 0) fold();
    }
    if (st < nsteps) {
        mma(f0);
        ++st;
    }
    if (st % SPC != 0) fold();                   // a last, shorter chunk
    // C layout of 16x16 MFMA: lane holds column (lane & 15), rows 4*(lane >> 4) + i.
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
        const int e = e0 + c * 16 + (lane & 15);
        if (e >= N) continue;
        const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + r * 16 + 4 * (lane >> 4) + i;
                if (t >= T) continue;
                if (sp.ks == 1) z[(size_t)t * N + e] = (float)(acc64[c][r][i] + b);
                else part[((size_t)kp * T + t) * N + e] = acc64[c][r][i];
            }
    }
}

// Sum of the K parts in part order, plus the bias, rounded once to fp32.
__global__ __launch_bounds__(256) void router_reduce_kernel(const double* __restrict__ part,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ z, int T, int N, int ks) {
    const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long TN = (long long)T * N;
    if (o >= TN) return;
    double acc = 0.0;
    for (int p = 0; p < ks; ++p) acc += part[p * TN + o];
    if (bias) acc += (double)bias[o % N];
    z[o] = (float)acc;
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
// ranked[t * NP + r] = expert of rank r (uint8, N <= 256); rows are padded to NP = N rounded up
// to 16 bytes with 0xFF, which is never a valid expert when padding exists (N < 256).
__global__ __launch_bounds__(64) void rank_sort_kernel(const float* __restrict__ z, int T, int N, int NP,
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
    for (int r = lane; r < NP; r += 64)
        ranked[(size_t)t * NP + r] = r < N ? (uint8_t)key_expert(key[r]) : (uint8_t)0xFF;
}

// ------------------------------------------------------------------ capacity routing
// One block of 1024 threads.  Slots are placed pass by pass (all slot-0s in token order, then
// all slot-1s, ...).  Within a pass, tokens are taken in chunks of CT (one per thread); a chunk
// is resolved in parallel by deferred acceptance with token order as every expert's priority:
// each token proposes to its best-ranked expert that it does not hold, that had room at the
// start of the chunk and whose cut-off tau[e] is not below the token; an expert keeps its
// (room)-th first proposers in token order and moves tau[e] to the last one kept.  tau only moves
// down, so a token never returns to an expert that turned it away, and the fixed point is the
// token-by-token first-come assignment.
//
// A 64-rank window of each chunk token's ranked list sits in LDS (4 ranks per dword,
// rank-major, so a wave's lanes read neighbouring words), starting at the 16-rank boundary at
// or before the rank the token resumes from; picks are shallow (on the skewed layer every pick
// is within 41 ranks), and a scan that runs past the window reads the list from memory.  The
// window keeps a chunk at one token per thread.  "Room at chunk start" is a byte table in LDS
// and "already held" is in registers; a scan takes 16 ranks at a time, so a token steps over
// full experts cheaply.  Proposal
// counts are per wave, stamped with the round number, so no round has to clear them.
#define CAP_THREADS 1024
#define CAP_WIN 4                   // 16-byte pieces (16 ranks each) in a token's window

template <int THREADS>
__global__ __launch_bounds__(THREADS) void capacity_kernel(
    const uint8_t* __restrict__ ranked, uint8_t* __restrict__ rpos, int T, int N, int NP, int CT, int k,
    int C, int32_t* __restrict__ idx) {
    constexpr int CAP_THREADS_ = THREADS;
    constexpr int CAP_WAVES_ = THREADS / 64;
    constexpr int WW = 4 * CAP_WIN;                     // window words
    __shared__ uint32_t rk4[WW * THREADS];              // [WW][CT]
    __shared__ uint32_t cnt[CAP_WAVES_][MOE_MAX_EXPERTS]; // (round << 16) | proposals of the wave
    __shared__ int fill[MOE_MAX_EXPERTS];
    __shared__ int tau[MOE_MAX_EXPERTS];
    __shared__ uint8_t roomb[MOE_MAX_EXPERTS];          // 1: expert had room at chunk start
    const int tid = threadIdx.x, lane = tid & 63;
    (void)lane;
    const int wave = tid >> 6;
    const int NQ = NP >> 2;               // words per ranked row (multiple of 4)
    for (int e = tid; e < MOE_MAX_EXPERTS; e += CAP_THREADS_) fill[e] = 0;
    for (int i = tid; i < CAP_WAVES_ * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&cnt[0][0])[i] = 0u;
    uint32_t round = 0;                   // stamps of cnt; never reused without clearing

    // next chunk's state of this thread's token, fetched during the current chunk: the window
    // of its ranked row, the first four experts it already holds and the rank after its
    // previous slot's pick
    u32x4 pre[CAP_WIN];
    int ph0 = -1, ph1 = -1, ph2 = -1, ph3 = -1, pstart = 0, pq0 = 0;
    auto prefetch = [&](int t_next, int j_next) {
        if (tid >= CT || t_next >= T) return;
        const int32_t* ir = idx + (size_t)t_next * k;
        ph0 = j_next > 0 ? ir[0] : -1;
        ph1 = j_next > 1 ? ir[1] : -1;
        ph2 = j_next > 2 ? ir[2] : -1;
        ph3 = j_next > 3 ? ir[3] : -1;
        pstart = j_next > 0 ? rpos[t_next] : 0;
        pq0 = (pstart >> 4) << 2;                           // window start (words), 16-rank aligned
        const u32x4* row = (const u32x4*)(ranked + (size_t)t_next * NP) + (pq0 >> 2);
        const int npieces = (NQ - pq0) >> 2;                // pieces left in the row
#pragma unroll
        for (int i = 0; i < CAP_WIN; ++i)
            if (i < npieces) pre[i] = row[i];
    };
    const int nchunks = (T + CT - 1) / CT;
    prefetch(tid, 0);
    __syncthreads();

    for (int j = 0; j < k; ++j) {
        for (int ci = 0; ci < nchunks; ++ci) {
            const int c0 = ci * CT;
            const int t = c0 + tid;
            const bool active = tid < CT && t < T;
            const int wq0 = pq0;                            // this chunk token's window start
            if (active) {
                const int npieces = (NQ - wq0) >> 2;
#pragma unroll
                for (int i = 0; i < CAP_WIN; ++i)
                    if (i < npieces) {
                        rk4[(4 * i + 0) * CT + tid] = pre[i][0];
                        rk4[(4 * i + 1) * CT + tid] = pre[i][1];
                        rk4[(4 * i + 2) * CT + tid] = pre[i][2];
                        rk4[(4 * i + 3) * CT + tid] = pre[i][3];
                    }
            }
            const int h0 = ph0, h1 = ph1, h2 = ph2, h3 = ph3;
            // the rank after the previous slot's pick: everything ranked above it was held or
            // full then, and fills never go down
            const int start = pstart;
            for (int e = tid; e < MOE_MAX_EXPERTS; e += CAP_THREADS_) {
                tau[e] = 0x7FFFFFFF;
                roomb[e] = (e < N && fill[e] < C) ? 1 : 0;
            }
            __syncthreads();
            // next: the following chunk of this pass (the first chunk of the next pass is fetched
            // once this chunk's picks are written: with a single chunk they are its own tokens)
            if (ci + 1 < nchunks) prefetch(t + CT, j);
            int q = start >> 2, bpos = start & 3, choice = -1;
            bool choose = active;
            while (true) {
                ++round;
                if (choose) {                             // next candidate from (q, bpos) on
                    choice = -1;
                    // one aligned piece of four words (16 ranks) at a time: the words, then the
                    // room flags of their 16 experts, each read at once, so a scan over full
                    // experts waits for two LDS reads per 16 ranks
                    auto piece = [&](const uint32_t (&wd)[4], int q0) {
                        // all 16 reads unconditional (any byte indexes the table), so that they go
                        // out together; words past the row's end are masked afterwards
                        uint32_t rf = 0;                    // bit 4 i + b: word i, byte b had room
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                rf |= (uint32_t)roomb[(wd[i] >> (8 * b)) & 0xFF] << (4 * i + b);
                        if (NQ - q0 < 4) rf &= (1u << (4 * (NQ - q0))) - 1u;
                        rf &= ~0u << (4 * (q - q0) + bpos);    // ranks before the resume point
                        while (rf) {
                            const int p = __builtin_ctz(rf);
                            rf &= rf - 1;
                            const uint32_t w = (p >> 2) == 0 ? wd[0] : (p >> 2) == 1 ? wd[1]
                                             : (p >> 2) == 2 ? wd[2] : wd[3];
                            const int e = (w >> (8 * (p & 3))) & 0xFF;
                            if (t > tau[e]) continue;                         // turned away this chunk
                            bool held = e == h0 || e == h1 || e == h2 || e == h3;
                            for (int jj = 4; jj < j && !held; ++jj) held = idx[(size_t)t * k + jj] == e;
                            if (held) continue;
                            choice = e;
                            q = q0 + (p >> 2);
                            bpos = p & 3;
                            return true;
                        }
                        q = q0 + 4;
                        bpos = 0;
                        return false;
                    };
                    // inside the window (it starts on a piece boundary): LDS reads only, so no
                    // wait for the next chunk's loads still in flight
                    while (q < NQ && (q & ~3) - wq0 < WW) {
                        const int q0 = q & ~3;
                        uint32_t wd[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) wd[i] = rk4[(q0 + i - wq0) * CT + tid];   // in the window array
                        if (piece(wd, q0)) break;
                    }
                    // past the window (rare): the rest of the ranked row from memory
                    while (choice < 0 && q < NQ) {
                        const int q0 = q & ~3;
                        uint32_t wd[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            wd[i] = q0 + i < NQ ? *(const uint32_t*)(ranked + (size_t)t * NP + 4 * (q0 + i)) : 0u;
                        if (piece(wd, q0)) break;
                    }
                    choose = false;
                }
                // per-wave proposal counts (ballot matching), written once per expert and wave
                const uint32_t v = (uint32_t)(choice + 1);
                const uint64_t eq = match_lanes<9>(v);
                const int rin = __popcll(eq & lanemask_lt());
                if (choice >= 0 && rin == 0) cnt[wave][choice] = (round << 16) | (uint32_t)__popcll(eq);
                __syncthreads();
                bool rejected = false;
                if (choice >= 0) {
                    // proposals to the same expert from earlier waves: every wave's count read at
                    // once, then the earlier ones added
                    uint32_t cw[CAP_WAVES_];
#pragma unroll
                    for (int ww = 0; ww < CAP_WAVES_; ++ww) cw[ww] = cnt[ww][choice];
                    int rank = rin;
#pragma unroll
                    for (int ww = 0; ww < CAP_WAVES_; ++ww)
                        rank += (ww < wave && (cw[ww] >> 16) == round) ? (int)(cw[ww] & 0xFFFF) : 0;
                    const int room = C - fill[choice];
                    if (rank == room - 1) tau[choice] = t;
                    if (rank >= room) {
                        rejected = true;
                        if (++bpos == 4) { bpos = 0; ++q; }
                        choose = true;
                    }
                }
                if (!__syncthreads_or(rejected)) break;
            }
            if (active) {
                idx[(size_t)t * k + j] = choice;
                rpos[t] = (uint8_t)(choice >= 0 ? (q * 4 + bpos + 1 < 256 ? q * 4 + bpos + 1 : 255) : 255);
            }
            if (ci + 1 == nchunks && j + 1 < k) prefetch(tid, j + 1);
            if (tid < N) {                                // at the fixed point every proposal is kept
                int s = 0;
                for (int ww = 0; ww < CAP_WAVES_; ++ww) {
                    const uint32_t c = cnt[ww][tid];
                    s += (c >> 16) == round ? (int)(c & 0xFFFF) : 0;
                }
                fill[tid] += s;
            }
            if (round >= 0xFFF0) {                        // keep stamps unique: clear and restart
                __syncthreads();
                for (int i = tid; i < CAP_WAVES_ * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&cnt[0][0])[i] = 0u;
                round = 0;
            }
            __syncthreads();
        }
    }
}

// Gate weights of routed slots (idx -1 = dropped, weight 0), one wave per token.  Mode 0:
// softmax over the kept slots' logits; mode 1: softmax over all N logits taken at the slots.
__global__ __launch_bounds__(256) void slot_gate_kernel(const float* __restrict__ z,
                                                        const int32_t* __restrict__ idx, int T, int N,
                                                        int k, int gating, float* __restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;
    const float* zr = z + (size_t)t * N;
    const int32_t* ir = idx + (size_t)t * k;
    float zmax = -INFINITY, denom = 0.f;
    if (gating == 1) {
        for (int e = lane; e < N; e += 64) zmax = fmaxf(zmax, zr[e]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, m, 64));
        float s = 0.f;
        for (int e = lane; e < N; e += 64) s += __expf(zr[e] - zmax);
        denom = wave_sum_f32(s);
    } else {
        for (int j = lane; j < k; j += 64)
            if (ir[j] >= 0) zmax = fmaxf(zmax, zr[ir[j]]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) zmax = fmaxf(zmax, __shfl_xor(zmax, m, 64));
        float s = 0.f;
        for (int j = lane; j < k; j += 64)
            if (ir[j] >= 0) s += __expf(zr[ir[j]] - zmax);
        denom = wave_sum_f32(s);
    }
    for (int j = lane; j < k; j += 64) {
        const int e = ir[j];
        w[(size_t)t * k + j] = e >= 0 ? __expf(zr[e] - zmax) / denom : 0.f;
    }
}

// ------------------------------------------------------------------ launchers
hipError_t launch_router_logits(const void* x, const void* wr, const float* bias, float* z, void* ws,
                                int T, int d, int N, int dtype, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (dtype == 1) {
        const RouterSplit sp = router_split(T, d, N);
        // full expert tiles (4 column tiles of 16) in one launch, a partial last tile in another
        const int n_full = N / RL_BN, last_nct = ((N % RL_BN) + 15) / 16;
        auto launch = [&](auto nct, int et_beg, int n_et) {
            const long long units = (long long)sp.n_tt * n_et * sp.ks;
            hipLaunchKernelGGL(router_logits_bf16_kernel<decltype(nct)::value>, dim3((unsigned)((units + 3) / 4)),
                               dim3(256), 0, s, (const bf16*)x, (const bf16*)wr, bias, z, (double*)ws, T, d, N,
                               sp, et_beg, n_et);
        };
        if (n_full > 0) launch(std::integral_constant<int, 4>{}, 0, n_full);
        switch (last_nct) {
            case 1: launch(std::integral_constant<int, 1>{}, n_full, 1); break;
            case 2: launch(std::integral_constant<int, 2>{}, n_full, 1); break;
            case 3: launch(std::integral_constant<int, 3>{}, n_full, 1); break;
            case 4: launch(std::integral_constant<int, 4>{}, n_full, 1); break;
            default: break;
        }
        if (sp.ks > 1) {
            const long long n = (long long)T * N;
            hipLaunchKernelGGL(router_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                               (const double*)ws, bias, z, T, N, sp.ks);
        }
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

int capacity_ranked_stride(int N) { return (N + 15) & ~15; }
size_t capacity_workspace_bytes(int T, int N) { return (size_t)T * capacity_ranked_stride(N) + (size_t)T; }

hipError_t launch_capacity(const float* z, uint8_t* ranked, int T, int N, int k, int C, int gating,
                           int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int NP = capacity_ranked_stride(N);
    hipLaunchKernelGGL(rank_sort_kernel, dim3(T), dim3(64), 0, s, z, T, N, NP, ranked);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one token per thread and chunk (the ranked-list windows of 1024 tokens take 64 KiB of LDS)
    const int CT = CAP_THREADS;
    auto kern = capacity_kernel<CAP_THREADS>;
    hipLaunchKernelGGL(kern, dim3(1), dim3(CAP_THREADS), 0, s, ranked, ranked + (size_t)T * NP, T, N, NP, CT,
                       k, C, idx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slot_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, idx, T, N, k, gating, w);
    return hipGetLastError();
}
