// Steps 1-3 of the MoE layer: router logits, ranking + gating, expert capacity.
//
// Router: a learned linear layer scoring every expert per token (page "MoE 分片：混合專家模型的
// 平行化策略", section 什麼是 MoE 模型; page "MoE稀疏激活原理与工程实践", section 2.2).
// Gating: top-k with softmax over the kept logits (page "MoE 推理：激活参数 vs 总参数与专家路由",
// section 代码) or softmax over all logits then top-k without renormalisation (page
// "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析", section MoE核心机制).
// Capacity: a full expert passes the token on to its next-best expert (page "MoE稀疏激活原理与
// 工程实践", section 2.2).
#include <cstdlib>
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
        pb[c] = wr + (size_t)koff * N + (e < N ? e : 0);     // w_router [d, N]: column e
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
        for (int c = 0; c < NCT; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) f.b[c][i] = pb[c][(size_t)(k + i) * N];
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
    // parts loaded eight at a time, then added in part order
    double acc = 0.0;
    for (int p0 = 0; p0 < ks; p0 += 8) {
        double v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p0 + i < ks ? part[(p0 + i) * TN + o] : 0.0;
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (p0 + i < ks) acc += v[i];
    }
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
    const float* wv = wr + e;                                // w_router [d, N]: column e
    double acc = 0.0;
    for (int kc = 0; kc < d; kc += RL_CHUNK) {
        float s = 0.f;
        const int kend = min(kc + RL_CHUNK, d);
        for (int i = kc; i < kend; ++i) s = fmaf(xr[i], wv[(size_t)i * N], s);
        acc += (double)s;
    }
    if (bias) acc += (double)bias[e];
    z[o] = (float)acc;
}

// ------------------------------------------------------------------ top-k + gate weights
// One wave per token.  Each lane holds up to 4 logits (N <= 256) as 64-bit ranking keys
// (descending logit, then ascending expert id).  k rounds of a wave-wide max pick the slots in
// rank order.  Softmax in fp32 with the max subtracted.  zl[q] is the logit of expert lane + 64 q
// (any value where that expert is past N).
__device__ __forceinline__ void topk_gate_wave(const float (&zl)[4], int lane, int N, int k, int gating,
                                               int32_t* __restrict__ idx_row, float* __restrict__ w_row) {
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
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
            idx_row[j] = es[q];
            w_row[j] = __expf(zs[q] - zmax) * inv;
        }
    }
}

__global__ __launch_bounds__(256) void topk_gate_kernel(
    const float* __restrict__ z, int T, int N, int k, int gating,
    int32_t* __restrict__ idx, float* __restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // whole wave leaves together; no block barrier below
    const float* zr = z + (size_t)t * N;
    float zl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        zl[q] = e < N ? zr[e] : 0.f;
    }
    topk_gate_wave(zl, lane, N, k, gating, idx + (size_t)t * k, w + (size_t)t * k);
}

// ------------------------------------------------------------------ router + top-k, fused
// For bf16 layers with N = 64, 128 or 256 experts.  One block of 4 waves takes 32 tokens, every
// expert and the whole K: per stage of 64 inputs the token tile (32 rows x 128 bytes) and the
// router's weight tile (64 k-rows x N columns, K-major as stored) come into LDS by direct loads,
// three stages in flight (three LDS arrays used in turn: the router's weight comes from L2 at
// each block's own pace, so one stage ahead does not cover its latency),
// and v_mfma_f32_16x16x32_bf16 multiplies them: token fragments by 16-byte reads (chunk c of row
// r at c ^ ((r >> 1) & 7)), weight fragments by transposed reads (ds_read_b64_tr_b16; chunk c of
// k-row r at c ^ f(r), f as in rf_woff, so that a read's 8 k-rows fall in distinct banks).  Wave w
// owns expert tiles w, w + 4, ... of 16 experts and both 16-token row tiles.  The fp32 sums of
// 256 inputs are added in fp64, as in the unfused router, and the bias is added in fp64 before
// the one rounding to fp32.  The block's logits then go to LDS (and to memory if asked for), and
// each wave ranks 8 of its tokens with the same top-k and softmax as the unfused kernel.
#define RF_BT 32

template <int NP>
__device__ __forceinline__ int rf_woff(int r, int c) {     // byte of chunk c of k-row r
    constexpr int ROWB = 2 * NP;
    if (NP == 64) return r * ROWB + ((c ^ (2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)))) << 4);
    return r * ROWB + ((c ^ (2 * ((r & 3) | (((r >> 3) & 1) << 2)))) << 4);
}

template <int NP>
__global__ __launch_bounds__(256) void router_topk_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ z_out, int T, int d, int k, int gating, int do_topk, int32_t* __restrict__ idx,
    float* __restrict__ w) {
    static_assert(NP == 64 || NP == 128 || NP == 256, "weight tile swizzle for 64, 128 or 256 experts");
    constexpr int ROWB = 2 * NP, WBYTES = 64 * ROWB, XBYTES = RF_BT * 128;
    constexpr int SBYTES = XBYTES + WBYTES;
    constexpr int NJ = NP / 64;                               // expert tiles per wave
    constexpr int W_INS = WBYTES / 4096;                      // weight loads per wave per stage
    constexpr int LPS = 1 + W_INS;                           // direct loads per wave per stage
    static_assert(RF_BT * NP * 4 <= SBYTES, "the logit tile fits in one stage buffer");
    static_assert(LPS <= 63, "vmcnt range");
    // vmcnt(LPS) with lgkmcnt and expcnt left alone (gfx9 s_waitcnt encoding)
    constexpr int WAIT_ONE_BEHIND = (LPS & 15) | ((LPS >> 4) << 14) | (7 << 4) | (15 << 8);
    __shared__ __attribute__((aligned(1024))) char st0[SBYTES];
    __shared__ __attribute__((aligned(1024))) char st1[SBYTES];
    __shared__ __attribute__((aligned(1024))) char st2[SBYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = blockIdx.x * RF_BT;
    // direct-load offsets: token rows 8 wave .. 8 wave + 7 (rows past T load row t0), and this
    // lane's weight chunks (the stage's first k-row goes in the scalar offset)
    uint32_t xoff, woff[W_INS];
    {
        const int r = 8 * wave + (lane >> 3), pos = lane & 7;
        const int t = t0 + r < T ? t0 + r : t0;
        xoff = ((uint32_t)t * (uint32_t)d + (uint32_t)(8 * (pos ^ ((r >> 1) & 7)))) * 2u;
#pragma unroll
        for (int i = 0; i < W_INS; ++i) {
            const int q = 1024 * (wave + 4 * i) + 16 * lane;
            const int kr = q / ROWB, p = (q % ROWB) >> 4;
            // chunk c sits at position p with rf_woff(kr, c) == q; the swizzle is an involution
            const int c = (rf_woff<NP>(kr, p) - kr * ROWB) >> 4;
            woff[i] = (uint32_t)(kr * NP + 8 * c) * 2u;
        }
    }
    auto issue = [&](char* st, int k0) {
        buffer_load_lds16(x, (lds_void_t*)(st + 1024 * wave), xoff, 2 * k0);
#pragma unroll
        for (int i = 0; i < W_INS; ++i)
            buffer_load_lds16(wr, (lds_void_t*)(st + XBYTES + 1024 * (wave + 4 * i)), woff[i], 2 * k0 * NP);
    };
    // fragment offsets: token rows 16 rt + (lane & 15), chunk 4 ks + (lane >> 4); weight k-rows
    // 32 ks + 8 (lane >> 4) + ((lane & 15) >> 2) (+4) of expert tile 4 j + wave
    int aoff[2], boff[NJ];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = 16 * rt + (lane & 15);
        aoff[rt] = r * 128 + ((((lane >> 4)) ^ ((r >> 1) & 7)) << 4);      // chunk (lane >> 4) of step 0
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int g = lane >> 4, L = lane & 15;
        boff[j] = XBYTES + rf_woff<NP>(8 * g + (L >> 2), 2 * (4 * j + wave) + ((L & 3) >> 1)) + (L & 1) * 8;
    }
    f32x4 acc[2][NJ];
    double acc64[2][NJ][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            acc[rt][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc64[rt][j][i] = 0.0;
        }
    auto fold = [&]() {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) acc64[rt][j][i] += (double)acc[rt][j][i];
                acc[rt][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
    };
    // two 32-input steps of one stage; step ks reads token chunks 4 ks + (lane >> 4), whose
    // swizzled position is the step-0 one XOR 4 ks (the XOR term only touches bits 0-2)
    auto compute = [&](const char* st) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[2], b[NJ];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) a[rt] = *(const bf16x8*)(st + (aoff[rt] ^ (ks << 6)));
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[j] = lds_read_tr_b16x8(st, boff[j] + 32 * ks * ROWB, 4 * ROWB);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt], b[j], acc[rt][j], 0, 0, 0);
        }
    };
    const int S = d / 64;                                     // stages (d % 64 == 0 for bf16)
    // Stage s sits in array s % 3.  Before stage s is read, this wave's loads of stage s must have
    // landed (the loads of stage s + 1, if issued, may still be in flight) and then every wave's
    // (barrier); the barrier also ends every read of stage s - 1, whose array then takes stage s + 2.
    // Every stage's loads go out unconditionally (past the last stage, that stage again, into an
    // array no compute reads), so no wait depends on a branch: before stage s is read, this wave
    // waits until at most one stage of its loads is in flight.  The barrier is s_barrier alone
    // (after this wave's LDS reads have returned): __syncthreads() would also fence memory and so
    // wait for every load in flight, stage s + 1's included.  The direct loads need no fence:
    // their data is in LDS once the issuing wave's counter says so.
    auto kst = [&](int i) { return 64 * (i < S ? i : S - 1); };
    auto wait_stage = [&]() {
        __builtin_amdgcn_s_waitcnt(WAIT_ONE_BEHIND);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    issue(st0, 0);
    issue(st1, kst(1));
    for (int s = 0; s < S; s += 3) {
        wait_stage();
        // (stage s + 2 goes out after this stage's reads: at the loop head the compiler no longer
        // tells the arrays' loads apart and would wait for all of them before the first read)
        compute(st0);
        issue(st2, kst(s + 2));
        if ((s + 1) % 4 == 0) fold();
        if (s + 1 >= S) break;
        wait_stage();
        issue(st0, kst(s + 3));
        compute(st1);
        if ((s + 2) % 4 == 0) fold();
        if (s + 2 >= S) break;
        wait_stage();
        issue(st1, kst(s + 4));
        compute(st2);
        if ((s + 3) % 4 == 0) fold();
    }
    if (S % 4 != 0) fold();                                   // a last, shorter chunk
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();                                          // every wave done with the stages
    // logits: C layout of 16x16 MFMA, lane holds expert (lane & 15) of its tile, tokens
    // 4 (lane >> 4) + i of its row tile
    float* zt = (float*)st0;                                  // [RF_BT][NP]
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = 16 * (4 * j + wave) + (lane & 15);
        const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * rt + 4 * (lane >> 4) + i;
                const float zv = (float)(acc64[rt][j][i] + b);
                zt[r * NP + e] = zv;
                if (z_out && t0 + r < T) z_out[(size_t)(t0 + r) * NP + e] = zv;
            }
    }
    if (!do_topk) return;
    __syncthreads();
    for (int rr = 0; rr < RF_BT / 4; ++rr) {
        const int r = wave * (RF_BT / 4) + rr, t = t0 + r;
        if (t >= T) break;                                    // uniform over the wave
        float zl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) zl[q] = (lane + 64 * q < NP) ? zt[r * NP + lane + 64 * q] : 0.f;
        topk_gate_wave(zl, lane, NP, k, gating, idx + (size_t)t * k, w + (size_t)t * k);
    }
}

// ------------------------------------------------------------------ full ranking (capacity)
// One wave per token, four tokens per block: bitonic sort of the N ranking keys, descending, in
// registers.  The P = max(64, N rounded up to a power of two) keys sit KPL = P / 64 to a lane,
// element i in slot i % KPL of lane i / KPL; compare-exchanges at strides below KPL stay in a
// lane, the others pair lanes by shuffles.  Keys past N are 0, below every real key (a real key's
// upper half is the order-preserving map of its logit, never 0), so they sort last.
// ranked[t * NP + r] = expert of rank r (uint8, N <= 256); rows are padded to NP = N rounded up
// to 16 bytes with 0xFF, which is never a valid expert when padding exists (N < 256).
template <int KPL>
__global__ __launch_bounds__(256) void rank_sort_kernel(const float* __restrict__ z, int T, int N, int NP,
                                                        uint8_t* __restrict__ ranked) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    constexpr int P = 64 * KPL;
    const float* zr = z + (size_t)t * N;
    uint64_t key[KPL];
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
        const int e = lane * KPL + s;
        key[s] = e < N ? rank_key(zr[e], e) : 0ull;
    }
#pragma unroll
    for (int size = 2; size <= P; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= KPL) {                  // partner in lane ^ (stride / KPL), same slot
#pragma unroll
                for (int s = 0; s < KPL; ++s) {
                    const int i = lane * KPL + s;
                    const uint64_t o = shfl_xor_u64(key[s], stride / KPL);
                    const bool keep_max = ((i & stride) == 0) == ((i & size) == 0);
                    key[s] = keep_max ? (o > key[s] ? o : key[s]) : (o < key[s] ? o : key[s]);
                }
            } else {                              // partner in the same lane
#pragma unroll
                for (int s = 0; s < KPL; ++s) {
                    if (s & stride) continue;
                    const int i = lane * KPL + s;
                    const uint64_t a = key[s], b = key[s + stride];
                    const bool desc = (i & size) == 0;
                    const bool sw = desc ? (a < b) : (a > b);
                    key[s] = sw ? b : a;
                    key[s + stride] = sw ? a : b;
                }
            }
        }
    }
    uint8_t* out = ranked + (size_t)t * NP;
#pragma unroll
    for (int s = 0; s < KPL; ++s) {
        const int r = lane * KPL + s;
        if (r < NP) out[r] = r < N ? (uint8_t)key_expert(key[s]) : (uint8_t)0xFF;
    }
}

// ------------------------------------------------------------------ capacity routing
// One block of 1024 threads.  Slots are placed pass by pass (all slot-0s in token order, then
// all slot-1s, ...).  Within a pass, tokens are taken in chunks of CT (one per thread); a chunk
// is resolved in parallel by deferred acceptance with token order as every expert's priority:
// each token proposes to its best-ranked expert that it does not hold, that had room at the
// start of the chunk and whose cut-off is not below the token; an expert keeps its (room)-th
// first proposers in token order and moves its cut-off to the last one kept.  The cut-off only
// moves down, so a token never returns to an expert that turned it away, and the fixed point is
// the token-by-token first-come assignment.
//
// Both conditions sit in one LDS table of 16-bit chunk-local limits: lim[e] = -1 when e had no
// room at the chunk's start, else the chunk index of the last token that may still propose to e
// (CT - 1 until e is cut).  A scan takes 16 ranks at a time: the four words of the ranked row
// and the 16 limits they name are read at once, and the candidate mask is built in registers,
// so stepping over full or cut experts costs no dependent LDS read.
//
// The first 64 ranks of each chunk token's ranked list sit in LDS (4 ranks per dword,
// rank-major, so a wave's lanes read neighbouring words); picks are shallow (on the skewed layer
// every pick is within 41 ranks), and a scan that runs past them reads the list from memory.
// The next chunk's ranks, held experts and resume rank are loaded while the current chunk runs;
// none of these loads depends on another.  A wave loads the first 64 ranks of its own 64 tokens
// four lanes to a row (16 rows per load), and scatters them into the rank-major layout at the
// chunk's start (rows padded by 4 words, so that the four lanes writing one row hit four bank
// groups).  The loads are unconditional (addresses clamped into the arrays), and a chunk's
// picks are stored at the start of the next chunk of the same pass (a pass's last chunk stores
// its own, before the next pass reads them): the vector memory counter counts stores too, so a
// store issued just before the next chunk's loads are needed would make them wait for it.
//
// Proposal counts are per wave (ballot matching), stamped with the round number, so no round
// has to clear them, and an LDS total per expert (the two totals alternate between rounds) lets
// the proposers of an expert with no more proposals than room accept without reading them;
// after round_limit rounds (at most 0xFFFF, the stamp's width) the counts are cleared and the
// stamps start again at 1, at the top of a round, when no earlier round's count is read any more.
// Whether another round follows needs no block reduction: each wave's "a proposal was turned
// away" flag is written after the round's first barrier and read after its second.
#define CAP_THREADS 1024
#define CAP_WIN 4                   // 16-byte pieces (16 ranks each) of a token's list in LDS

template <int THREADS, int BITS>
__global__ __launch_bounds__(THREADS) void capacity_kernel(
    const uint8_t* __restrict__ ranked, uint8_t* __restrict__ rpos, int T, int N, int NP, int CT, int k,
    int C, uint32_t round_limit, int32_t* __restrict__ idx) {
    constexpr int CAP_THREADS_ = THREADS;
    constexpr int CAP_WAVES_ = THREADS / 64;
    constexpr int WW = 4 * CAP_WIN;                     // window words
    static_assert(CAP_WAVES_ % 4 == 0, "wave flags are read four at a time");
    __shared__ uint32_t rk4[WW * (THREADS + 4)];        // [WW][CT + 4]
    __shared__ uint32_t cnt[CAP_WAVES_][MOE_MAX_EXPERTS]; // (round << 16) | proposals of the wave
    __shared__ int fill[MOE_MAX_EXPERTS];
    __shared__ int16_t lim[MOE_MAX_EXPERTS];            // chunk-local cut-off, -1: full at chunk start
    __shared__ u32x4 rejw[CAP_WAVES_ / 4];              // per wave: a proposal was turned away
    __shared__ int tot[2][MOE_MAX_EXPERTS];             // proposals per expert, rounds alternating
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = tid >> 6;
    const int NQ = NP >> 2;               // words per ranked row (multiple of 4)
    const int NPC = NQ >> 2;              // 16-rank pieces per ranked row
    for (int e = tid; e < MOE_MAX_EXPERTS; e += CAP_THREADS_) fill[e] = 0;
    for (int i = tid; i < CAP_WAVES_ * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&cnt[0][0])[i] = 0u;
    for (int i = tid; i < 2 * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&tot[0][0])[i] = 0;
    uint32_t round = 0;                   // stamp of the current round's counts, 1 .. round_limit

    // next chunk's state, fetched during the current chunk: for this thread's token the first
    // four experts it already holds and the rank after its previous slot's pick; for the wave's
    // 64 tokens the first CAP_WIN pieces of their ranked rows, piece (lane & 3) of row
    // 16 i + (lane >> 2) in pre[i] (CAP_WIN == 4: every piece of the window once)
    static_assert(CAP_WIN == 4, "one 16-byte piece per lane and load");
    u32x4 pre[4];
    int ph0 = -1, ph1 = -1, ph2 = -1, ph3 = -1, pstart = 0;
    const int wrow0 = 64 * wave;                         // the wave's first token in a chunk
    const int pc = lane & 3;                             // piece of a row this lane carries
    auto prefetch = [&](int c_next) {                   // c_next: first token of the next chunk
        const int t_next = min(c_next + tid, T - 1);     // rows past T: loaded, never used
        const int32_t* ir = idx + (size_t)t_next * k;
        if (k > 1) { ph0 = ir[0]; pstart = rpos[t_next]; }      // only what a later pass reads
        if (k > 2) ph1 = ir[1];
        if (k > 3) ph2 = ir[2];
        if (k > 4) ph3 = ir[3];                          // masked by the pass where used
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(c_next + wrow0 + 16 * i + (lane >> 2), T - 1);
            pre[i] = *((const u32x4*)(ranked + (size_t)r * NP) + min(pc, NPC - 1));
        }
    };
    const int nchunks = (T + CT - 1) / CT;
    int pend_t = -1, pend_choice = -1, pend_rpos = 0;  // pick not stored yet (same pass)
    prefetch(0);
    __syncthreads();

    for (int j = 0; j < k; ++j) {
        for (int ci = 0; ci < nchunks; ++ci) {
            const int c0 = ci * CT;
            const int t = c0 + tid;
            const bool active = tid < CT && t < T;
            // every lane writes (rows past T and pieces past the row hold junk that no scan
            // reads), so that every load of the prefetch is waited for on every path
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wrow0 + 16 * i + (lane >> 2);
                rk4[(4 * pc + 0) * (CT + 4) + r] = pre[i][0];
                rk4[(4 * pc + 1) * (CT + 4) + r] = pre[i][1];
                rk4[(4 * pc + 2) * (CT + 4) + r] = pre[i][2];
                rk4[(4 * pc + 3) * (CT + 4) + r] = pre[i][3];
            }
            if (pend_t >= 0) {                             // the previous chunk's pick
                idx[(size_t)pend_t * k + j] = pend_choice;
                rpos[pend_t] = (uint8_t)pend_rpos;
                pend_t = -1;
            }
            const int h0 = j > 0 ? ph0 : -1, h1 = j > 1 ? ph1 : -1, h2 = j > 2 ? ph2 : -1, h3 = j > 3 ? ph3 : -1;
            // the rank after the previous slot's pick: everything ranked above it was held or
            // full then, and fills never go down
            const int start = j > 0 ? pstart : 0;
            for (int e = tid; e < MOE_MAX_EXPERTS; e += CAP_THREADS_)
                lim[e] = (int16_t)((e < N && fill[e] < C) ? CT - 1 : -1);
            __syncthreads();
            // next: the following chunk of this pass (the first chunk of the next pass is fetched
            // once this chunk's picks are written: with a single chunk they are its own tokens)
            if (ci + 1 < nchunks) prefetch(c0 + CT);
            int q = start >> 2, bpos = start & 3, choice = -1;
            bool choose = active;
            while (true) {
                // round is uniform over the block (every thread runs every round), and the
                // barrier that ended the previous round follows its last read of cnt
                if (round >= round_limit) {
                    for (int i = tid; i < CAP_WAVES_ * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&cnt[0][0])[i] = 0u;
                    // the restarted stamps may give two rounds in a row the same parity
                    for (int i = tid; i < 2 * MOE_MAX_EXPERTS; i += CAP_THREADS_) (&tot[0][0])[i] = 0;
                    round = 0;
                    __syncthreads();                      // cleared before any new stamp is written
                }
                ++round;
                if (choose) {                             // next candidate from (q, bpos) on
                    choice = -1;
                    // one aligned piece of four words (16 ranks): the limits of its 16 experts,
                    // all read at once (any byte indexes the table; words past the row's end are
                    // masked afterwards), give the candidates; then only the held check is left
                    auto piece = [&](const uint32_t (&wd)[4], int q0) {
                        uint32_t rf = 0;                    // bit 4 i + b: word i, byte b may be proposed to
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                rf |= (uint32_t)(tid <= (int)lim[(wd[i] >> (8 * b)) & 0xFF]) << (4 * i + b);
                        if (NQ - q0 < 4) rf &= (1u << (4 * (NQ - q0))) - 1u;
                        rf &= ~0u << (4 * (q - q0) + bpos);    // ranks before the resume point
                        while (rf) {
                            const int p = __builtin_ctz(rf);
                            rf &= rf - 1;
                            const uint32_t w = (p >> 2) == 0 ? wd[0] : (p >> 2) == 1 ? wd[1]
                                             : (p >> 2) == 2 ? wd[2] : wd[3];
                            const int e = (w >> (8 * (p & 3))) & 0xFF;
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
                    // the first WW words from LDS: no wait for the next chunk's loads in flight
                    while (q < NQ && q < WW) {
                        const int q0 = q & ~3;
                        uint32_t wd[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) wd[i] = rk4[(q0 + i) * (CT + 4) + tid];
                        if (piece(wd, q0)) break;
                    }
                    // past them (rare): the rest of the ranked row from memory
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
                const uint64_t eq = match_lanes<BITS>(v);
                const int rin = __popcll(eq & lanemask_lt());
                if (choice >= 0 && rin == 0) {
                    cnt[wave][choice] = (round << 16) | (uint32_t)__popcll(eq);
                    atomicAdd(&tot[round & 1][choice], __popcll(eq));
                }
                __syncthreads();
                // the other round's totals start again from zero: last read before this round's
                // first barrier, next added to after its second
                for (int e = tid; e < MOE_MAX_EXPERTS; e += CAP_THREADS_) tot[(round + 1) & 1][e] = 0;
                bool rejected = false;
                // an expert with no more proposals than room keeps them all: its proposers skip
                // the per-wave counts
                if (choice >= 0 && tot[round & 1][choice] > C - fill[choice]) {
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
                    if (rank == room - 1) lim[choice] = (int16_t)tid;
                    if (rank >= room) {
                        rejected = true;
                        if (++bpos == 4) { bpos = 0; ++q; }
                        choose = true;
                    }
                }
                // another round if any wave turned a proposal away: one flag per wave, written
                // after this round's first barrier (every wave has read the previous round's
                // flags by then) and read after the second
                const bool wrej = __ballot(rejected) != 0ull;
                if (lane == 0) ((uint32_t*)rejw)[wave] = wrej ? 1u : 0u;
                __syncthreads();
                u32x4 any = rejw[0];
#pragma unroll
                for (int i = 1; i < CAP_WAVES_ / 4; ++i) any |= rejw[i];
                if ((any[0] | any[1] | any[2] | any[3]) == 0u) break;
            }
            if (active) {
                const int rp = choice >= 0 ? (q * 4 + bpos + 1 < 256 ? q * 4 + bpos + 1 : 255) : 255;
                if (ci + 1 == nchunks) {
                    idx[(size_t)t * k + j] = choice;
                    rpos[t] = (uint8_t)rp;
                } else {
                    pend_t = t;
                    pend_choice = choice;
                    pend_rpos = rp;
                }
            }
            if (ci + 1 == nchunks && j + 1 < k) prefetch(0);
            if (tid < N) {                                // at the fixed point every proposal is kept
                int s = 0;
                for (int ww = 0; ww < CAP_WAVES_; ++ww) {
                    const uint32_t c = cnt[ww][tid];
                    s += (c >> 16) == round ? (int)(c & 0xFFFF) : 0;
                }
                fill[tid] += s;
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

// The K-part sum and top-k in one launch (layers without capacity whose expert count the fused
// router does not take): one wave per token sums its N logits' fp64 parts in part order, adds
// the bias and rounds once (as router_reduce_kernel), writes the logits, and ranks them with
// topk_gate_wave (as topk_gate_kernel).
__global__ __launch_bounds__(256) void reduce_topk_kernel(const double* __restrict__ part, int ks,
                                                          const float* __restrict__ bias, float* __restrict__ z,
                                                          int T, int N, int k, int gating, int32_t* __restrict__ idx,
                                                          float* __restrict__ w) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + wave;
    if (t >= T) return;  // whole wave leaves together; no block barrier below
    const long long TN = (long long)T * N;
    float zl[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        zl[q] = 0.f;
        if (e < N) {
            const long long o = (long long)t * N + e;
            double acc = 0.0;                            // parts loaded eight at a time, added in order
            for (int p0 = 0; p0 < ks; p0 += 8) {
                double v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = p0 + i < ks ? part[(p0 + i) * TN + o] : 0.0;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (p0 + i < ks) acc += v[i];
            }
            if (bias) acc += (double)bias[e];
            zl[q] = (float)acc;
            z[o] = zl[q];
        }
    }
    topk_gate_wave(zl, lane, N, k, gating, idx + (size_t)t * k, w + (size_t)t * k);
}

// ------------------------------------------------------------------ decode-sized batch: one finishing block
// After the router's logits (or their fp64 K-part sums) for a batch of at most RF_MAX_S slots:
// the K parts summed in part order with the bias and rounded once (as router_reduce_kernel),
// top-k and the gate weights per token (topk_gate_wave, as topk_gate_kernel), and the grouping
// (slot s = t k + j to row offsets[e] + the slots before s with expert e, so an expert's rows
// are in ascending slot order, as permute_kernel) -- one launch where a 16-token decode batch had
// three of 4-5 us each.
#define RF_THREADS 512
#define RF_WAVES (RF_THREADS / 64)
#define RF_MAX_S 512                // slots (T * k)
#define RF_MAX_Z 8192               // logits (T * N)

__global__ __launch_bounds__(RF_THREADS) void route_finish_small_kernel(
    const double* __restrict__ part, int ks, const float* __restrict__ bias, float* __restrict__ z, int T, int N,
    int k, int gating, int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ float s_z[RF_MAX_Z];
    __shared__ int32_t s_idx[RF_MAX_S];
    __shared__ float s_w[RF_MAX_S];
    __shared__ int s_cnt[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int TN = T * N, S = T * k;
    for (int o = tid; o < TN; o += RF_THREADS) {
        float zf;
        if (ks > 1) {
            // parts loaded eight at a time, then added in part order
            double acc = 0.0;
            for (int p0 = 0; p0 < ks; p0 += 8) {
                double v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = p0 + i < ks ? part[(size_t)(p0 + i) * TN + o] : 0.0;
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    if (p0 + i < ks) acc += v[i];
            }
            if (bias) acc += (double)bias[o % N];
            zf = (float)acc;
            z[o] = zf;
        } else {
            zf = z[o];                                     // written by the router itself
        }
        s_z[o] = zf;
    }
    __syncthreads();
    for (int t = wave; t < T; t += RF_WAVES) {             // uniform per wave
        float zl[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = lane + 64 * q;
            zl[q] = e < N ? s_z[t * N + e] : 0.f;
        }
        topk_gate_wave(zl, lane, N, k, gating, s_idx + t * k, s_w + t * k);
    }
    __syncthreads();
    for (int e = tid; e < N; e += RF_THREADS) {
        int c = 0;
        for (int i = 0; i < S; ++i) c += s_idx[i] == e ? 1 : 0;
        s_cnt[e] = c;
        counts[e] = c;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int e = 0; e < N; ++e) {
            s_off[e] = run;
            offsets[e] = run;
            run += s_cnt[e];
        }
        s_off[N] = run;
        offsets[N] = run;
    }
    __syncthreads();
    for (int sl = tid; sl < S; sl += RF_THREADS) {
        const int e = s_idx[sl];
        int before = 0;
        for (int i = 0; i < sl; ++i) before += s_idx[i] == e ? 1 : 0;
        const int row = s_off[e] + before;
        idx[sl] = e;
        w[sl] = s_w[sl];
        perm[row] = sl;
        inv[sl] = row;
    }
}

// ------------------------------------------------------------------ launchers
int router_k_parts(int T, int d, int N, int dtype) {
    return (dtype == 1 && T > 0) ? router_split(T, d, N).ks : 1;
}

hipError_t launch_router_logits(const void* x, const void* wr, const float* bias, float* z, void* ws,
                                int T, int d, int N, int dtype, hipStream_t s, bool sum_parts) {
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
        if (sp.ks > 1 && sum_parts) {
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

bool router_fused_supported(int N, int dtype) { return dtype == 1 && (N == 64 || N == 128 || N == 256); }

bool route_finish_small_supported(int T, int N, int k) {
    return T >= 1 && k >= 1 && k <= N && N <= MOE_MAX_EXPERTS && (long long)T * k <= RF_MAX_S &&
           (long long)T * N <= RF_MAX_Z;
}

hipError_t launch_route_finish_small(const void* part, int ks, const float* bias, float* z, int T, int N, int k,
                                     int gating, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                                     int32_t* perm, int32_t* inv, hipStream_t s) {
    if (!route_finish_small_supported(T, N, k) || (ks > 1 && !part)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_finish_small_kernel, dim3(1), dim3(RF_THREADS), 0, s, (const double*)part, ks, bias, z,
                       T, N, k, gating, idx, w, counts, offsets, perm, inv);
    return hipGetLastError();
}

hipError_t launch_router_topk(const void* x, const void* wr, const float* bias, float* z, int T, int d, int N,
                              int k, int gating, int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid((unsigned)((T + RF_BT - 1) / RF_BT));
    const int do_topk = idx != nullptr;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const bf16*)x, (const bf16*)wr, bias, z, T, d, k, gating,
                           do_topk, idx, w);
    };
    if (N == 64) go(router_topk_kernel<64>);
    else if (N == 128) go(router_topk_kernel<128>);
    else if (N == 256) go(router_topk_kernel<256>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_reduce_topk(const void* part, int ks, const float* bias, float* z, int T, int N, int k,
                             int gating, int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (!part || ks < 1 || N > MOE_MAX_EXPERTS) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reduce_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, (const double*)part, ks, bias, z, T,
                       N, k, gating, idx, w);
    return hipGetLastError();
}

hipError_t launch_topk_gate(const float* z, int T, int N, int k, int gating, int32_t* idx, float* w,
                            hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, T, N, k, gating, idx, w);
    return hipGetLastError();
}

// Rounds between two clears of the capacity kernel's proposal counts: 0xFFFF (the stamp's
// width), or the value of MOE_CAPACITY_ROUND_LIMIT (1 .. 0xFFFF), a testing hook that makes the
// clears frequent so that their path is exercised; the routing does not depend on it.
static uint32_t capacity_round_limit() {
    const char* v = getenv("MOE_CAPACITY_ROUND_LIMIT");
    if (!v || !*v) return 0xFFFFu;
    const long n = strtol(v, nullptr, 10);
    return n < 1 ? 1u : n > 0xFFFF ? 0xFFFFu : (uint32_t)n;
}

int capacity_ranked_stride(int N) { return (N + 15) & ~15; }
size_t capacity_workspace_bytes(int T, int N) { return (size_t)T * capacity_ranked_stride(N) + (size_t)T; }

hipError_t launch_capacity(const float* z, uint8_t* ranked, int T, int N, int k, int C, int gating,
                           int32_t* idx, float* w, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const int NP = capacity_ranked_stride(N);
    const dim3 sgrid((unsigned)((T + 3) / 4));
    if (N <= 64) hipLaunchKernelGGL(rank_sort_kernel<1>, sgrid, dim3(256), 0, s, z, T, N, NP, ranked);
    else if (N <= 128) hipLaunchKernelGGL(rank_sort_kernel<2>, sgrid, dim3(256), 0, s, z, T, N, NP, ranked);
    else hipLaunchKernelGGL(rank_sort_kernel<4>, sgrid, dim3(256), 0, s, z, T, N, NP, ranked);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // one token per thread and chunk (the ranked-list windows of 1024 tokens take 64 KiB of LDS)
    const int CT = CAP_THREADS;
    // ballot matching on choice + 1 <= N: 8 bits below 256 experts
    auto kern = N < 256 ? capacity_kernel<CAP_THREADS, 8> : capacity_kernel<CAP_THREADS, 9>;
    hipLaunchKernelGGL(kern, dim3(1), dim3(CAP_THREADS), 0, s, ranked, ranked + (size_t)T * NP, T, N, NP, CT,
                       k, C, capacity_round_limit(), idx);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slot_gate_kernel, dim3((T + 3) / 4), dim3(256), 0, s, z, idx, T, N, k, gating, w);
    return hipGetLastError();
}
