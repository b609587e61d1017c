// Step 5 of the MoE layer: the expert FFNs, grouped over experts.
//
// An expert is two linear maps with an activation between them (page "MoE 分片：混合專家模型的
// 平行化策略", section 什麼是 MoE 模型); each expert runs only on the rows routed to it (same
// page, section 動態 token 路由, step 4).  A shared expert sees every token (page "MoE 架構科普",
// section 专家粒度) and is scheduled here as one more segment of rows.
//
// Segments: segment e < N holds rows offsets[e] .. offsets[e+1]-1 and expert e's weights;
// segment N (shared expert) holds rows T*k .. T*k+T-1.  The grid is sized on the host from the
// worst case (sum over experts of ceil(rows/BM) <= ceil(T*k/BM) + N); each block finds its
// segment and m-tile on the device from offsets, so the host never reads the routing.
//
// bf16 path: v_mfma_f32_32x32x16_bf16, block tile 128 x 128 (x2 for gate+up), K step 64,
// LDS double buffer, 4 waves each owning a 64 x 64 quarter.  The in-projection gathers its A
// rows straight from x (row = token of the slot), so the permuted copy of x is never built;
// SwiGLU (silu(g) * u) or ReLU is applied in registers and H is stored in bf16.  The
// out-projection multiplies each row by its slot's gate weight and stores the row in fp32, so the
// combine adds unrounded expert outputs.
#include "moe_common.h"
#include "moe_kernels.h"

#define FB_BM 128
#define FB_BN 128
#define FB_BK 64
#define FB_LDK (FB_BK + 8)  // padded row (elements): conflict-free 16-byte LDS reads

enum { MODE_IN_SWIGLU = 0, MODE_IN_RELU = 1, MODE_OUT = 2 };

struct FfnKArgs {
    const bf16* A;          // in: x [T, d]; out: H [rows, d_ff]
    const int32_t* perm;
    const int32_t* offsets;
    const bf16* B0;         // routed weights [N, Ncols, K] (gate for SwiGLU, else W)
    const bf16* B1;         // routed up weights (SwiGLU) or null
    const bf16* S0;         // shared expert [Ncols, K] or null
    const bf16* S1;
    const float* row_scale; // [T*k] or null (out-projection only)
    void* C;                // [rows, Ncols]: bf16 H (in-projection) or fp32 y_perm (out-projection)
    int T, k, N, has_shared, K, Ncols, mt_max, n_tiles;
};

template <int MODE>
__global__ __launch_bounds__(256) void ffn_bf16_kernel(FfnKArgs a) {
    constexpr int NB = (MODE == MODE_IN_SWIGLU) ? 2 : 1;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    bf16* sA = (bf16*)smem;                 // [2][BM][LDK]
    bf16* sB = sA + 2 * FB_BM * FB_LDK;     // [2][NB][BN][LDK]
    __shared__ int s_info[2];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // XCD-aware order: consecutive logical tiles (the m-tiles that share one weight tile) land
    // on the same XCD, whose L2 then serves the repeated weight reads.
    const int G = gridDim.x;
    const int b = blockIdx.x;
    const int L = (b & 7) * (G >> 3) + (b >> 3);
    const int n_tile = L / a.mt_max, m_tile = L % a.mt_max;
    if (n_tile >= a.n_tiles) return;

    if (wave == 0) {  // segment of this m-tile: wave-wide scan of tiles per segment
        int tl[5], loc = 0;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            const int s = lane * 5 + q;
            int rows = 0;
            if (s < a.N) rows = a.offsets[s + 1] - a.offsets[s];
            else if (s == a.N && a.has_shared) rows = a.T;
            tl[q] = (rows + FB_BM - 1) / FB_BM;
            loc += tl[q];
        }
        int incl = loc;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (lane >= o) incl += v;
        }
        int run = incl - loc;
#pragma unroll
        for (int q = 0; q < 5; ++q) {
            if (m_tile >= run && m_tile < run + tl[q]) {
                s_info[0] = lane * 5 + q;
                s_info[1] = m_tile - run;
            }
            run += tl[q];
        }
        if (lane == 63 && m_tile >= incl) s_info[0] = -1;
    }
    __syncthreads();
    const int seg = s_info[0];
    if (seg < 0) return;
    const int mt = s_info[1];
    const size_t wstride = (size_t)a.Ncols * a.K;
    int row_beg, row_end;
    const bf16 *B0, *B1 = nullptr;
    if (seg < a.N) {
        row_beg = a.offsets[seg];
        row_end = a.offsets[seg + 1];
        B0 = a.B0 + seg * wstride;
        if (NB == 2) B1 = a.B1 + seg * wstride;
    } else {
        row_beg = a.T * a.k;
        row_end = row_beg + a.T;
        B0 = a.S0;
        if (NB == 2) B1 = a.S1;
    }
    const int m0 = row_beg + mt * FB_BM;
    const int n0 = n_tile * FB_BN;

    // global -> register assignment: 8 threads per 64-element row, 32 rows per pass, 4 passes
    const int kc = (tid & 7) * 8;
    const bf16* pA[4];
    const bf16* pB0[4];
    const bf16* pB1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rl = (tid >> 3) + 32 * i;
        const int r = (m0 + rl < row_end) ? m0 + rl : m0;
        int src;
        if (MODE == MODE_OUT) src = r;
        else src = (seg < a.N) ? a.perm[r] / a.k : r - a.T * a.k;
        pA[i] = a.A + (size_t)src * a.K + kc;
        const int n = (n0 + rl < a.Ncols) ? n0 + rl : n0;
        pB0[i] = B0 + (size_t)n * a.K + kc;
        pB1[i] = (NB == 2) ? B1 + (size_t)n * a.K + kc : nullptr;
    }
    bf16x8 ra[4], rb0[4], rb1[4];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *(const bf16x8*)(pA[i] + k0);
            rb0[i] = *(const bf16x8*)(pB0[i] + k0);
            if (NB == 2) rb1[i] = *(const bf16x8*)(pB1[i] + k0);
        }
    };
    auto sstore = [&](int buf) {
        bf16* dA = sA + buf * FB_BM * FB_LDK;
        bf16* dB = sB + buf * NB * FB_BN * FB_LDK;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rl = (tid >> 3) + 32 * i;
            *(bf16x8*)(dA + rl * FB_LDK + kc) = ra[i];
            *(bf16x8*)(dB + rl * FB_LDK + kc) = rb0[i];
            if (NB == 2) *(bf16x8*)(dB + FB_BN * FB_LDK + rl * FB_LDK + kc) = rb1[i];
        }
    };

    const int wm = wave >> 1, wn = wave & 1;
    f32x16 acc[NB][2][2];
#pragma unroll
    for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;

    gload(0);
    sstore(0);
    __syncthreads();
    const int KT = a.K / FB_BK;
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload((kt + 1) * FB_BK);
        const bf16* cA = sA + buf * FB_BM * FB_LDK + (wm * 64 + fr) * FB_LDK + fk;
        const bf16* cB = sB + buf * NB * FB_BN * FB_LDK + (wn * 64 + fr) * FB_LDK + fk;
#pragma unroll
        for (int kk = 0; kk < FB_BK; kk += 16) {
            bf16x8 af[2], bfr[NB][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)(cA + i * 32 * FB_LDK + kk);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    bfr[m][j] = *(const bf16x8*)(cB + m * FB_BN * FB_LDK + j * 32 * FB_LDK + kk);
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[m][j],
                                                                              acc[m][i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }

    // epilogue.  32x32 C layout: lane holds column (lane & 31); register r holds row
    // 8*(r >> 2) + 4*(lane >> 5) + (r & 3).
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (row >= row_end) continue;
            float scale = 1.0f;
            if (MODE == MODE_OUT && a.row_scale && seg < a.N) scale = a.row_scale[a.perm[row]];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = n0 + wn * 64 + j * 32 + (lane & 31);
                if (col >= a.Ncols) continue;
                float v;
                if (MODE == MODE_IN_SWIGLU) v = silu_f32(acc[0][i][j][r]) * acc[NB - 1][i][j][r];
                else if (MODE == MODE_IN_RELU) v = fmaxf(acc[0][i][j][r], 0.f);
                else v = acc[0][i][j][r] * scale;
                if (MODE == MODE_OUT) ((float*)a.C)[(size_t)row * a.Ncols + col] = v;
                else ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)v;
            }
        }
    }
}

// ------------------------------------------------------------------ fp32 path
// One thread per output element, fp32 FMA in input order.  Used for fp32 layers.
__device__ __forceinline__ int segment_of_row(const int32_t* offsets, int N, int r) {
    int lo = 0, hi = N;  // largest e with offsets[e] <= r (rows of an empty expert are skipped)
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (offsets[mid] <= r) lo = mid;
        else hi = mid;
    }
    return lo;
}

template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(const float* __restrict__ A, const int32_t* __restrict__ perm,
                                                      const int32_t* __restrict__ offsets,
                                                      const float* __restrict__ B0, const float* __restrict__ B1,
                                                      const float* __restrict__ S0, const float* __restrict__ S1,
                                                      const float* __restrict__ row_scale, float* __restrict__ C,
                                                      int T, int k, int N, int has_shared, int K, int Ncols) {
    const long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long rows_total = (long long)T * k + (has_shared ? T : 0);
    if (o >= rows_total * Ncols) return;
    const int r = (int)(o / Ncols), c = (int)(o % Ncols);
    int seg;
    if (r < T * k) {
        if (r >= offsets[N]) return;
        seg = segment_of_row(offsets, N, r);
    } else {
        seg = N;
    }
    const size_t wstride = (size_t)Ncols * K;
    const float* w0 = (seg < N) ? B0 + seg * wstride : S0;
    const float* w1 = (seg < N) ? (B1 ? B1 + seg * wstride : nullptr) : S1;
    const float* ar;
    if (MODE == MODE_OUT) ar = A + (size_t)r * K;
    else ar = A + (size_t)((seg < N) ? perm[r] / k : r - T * k) * K;
    const float* wr0 = w0 + (size_t)c * K;
    float s0 = 0.f;
    for (int i = 0; i < K; ++i) s0 = fmaf(ar[i], wr0[i], s0);
    float v;
    if (MODE == MODE_IN_SWIGLU) {
        const float* wr1 = w1 + (size_t)c * K;
        float s1 = 0.f;
        for (int i = 0; i < K; ++i) s1 = fmaf(ar[i], wr1[i], s1);
        v = s0 / (1.0f + expf(-s0)) * s1;
    } else if (MODE == MODE_IN_RELU) {
        v = fmaxf(s0, 0.f);
    } else {
        v = s0 * ((row_scale && seg < N) ? row_scale[perm[r]] : 1.0f);
    }
    C[(size_t)r * Ncols + c] = v;
}

// ------------------------------------------------------------------ launchers
static size_t ffn_smem_bytes(int mode) {
    const int nb = (mode == MODE_IN_SWIGLU) ? 2 : 1;
    return (size_t)(2 * FB_BM * FB_LDK + 2 * nb * FB_BN * FB_LDK) * sizeof(bf16);
}

template <int MODE>
static hipError_t launch_bf16(const FfnKArgs& ka, int T, int k, int N, int has_shared, hipStream_t s) {
    // the LDS limit above 64 KiB is a per-function, per-device attribute; set it once per device
    static bool attr_set[64] = {};
    const size_t smem = ffn_smem_bytes(MODE);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64 || !attr_set[dev]) {
        e = hipFuncSetAttribute((const void*)ffn_bf16_kernel<MODE>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < 64) attr_set[dev] = true;
    }
    FfnKArgs a = ka;
    a.mt_max = (T * k + FB_BM - 1) / FB_BM + N + (has_shared ? (T + FB_BM - 1) / FB_BM : 0);
    a.n_tiles = (a.Ncols + FB_BN - 1) / FB_BN;
    long long G = (long long)a.mt_max * a.n_tiles;
    G = (G + 7) / 8 * 8;
    hipLaunchKernelGGL(ffn_bf16_kernel<MODE>, dim3((unsigned)G), dim3(256), smem, s, a);
    return hipGetLastError();
}

hipError_t launch_ffn_in(const FfnLaunch& f, hipStream_t s) {
    if (f.T == 0) return hipSuccess;
    const long long rows_total = (long long)f.T * f.k + (f.has_shared ? f.T : 0);
    if (f.dtype == 1) {
        FfnKArgs a{};
        a.A = (const bf16*)f.x;
        a.perm = f.perm;
        a.offsets = f.offsets;
        a.C = f.h;
        a.T = f.T; a.k = f.k; a.N = f.N; a.has_shared = f.has_shared;
        a.K = f.d; a.Ncols = f.d_ff;
        if (f.ffn == 1) {
            a.B0 = (const bf16*)f.w_gate; a.B1 = (const bf16*)f.w_up;
            a.S0 = (const bf16*)f.sh_gate; a.S1 = (const bf16*)f.sh_up;
            return launch_bf16<MODE_IN_SWIGLU>(a, f.T, f.k, f.N, f.has_shared, s);
        }
        a.B0 = (const bf16*)f.w_up;
        a.S0 = (const bf16*)f.sh_up;
        return launch_bf16<MODE_IN_RELU>(a, f.T, f.k, f.N, f.has_shared, s);
    }
    const long long n = rows_total * f.d_ff;
    const dim3 grid((unsigned)((n + 255) / 256));
    if (f.ffn == 1)
        hipLaunchKernelGGL(ffn_f32_kernel<MODE_IN_SWIGLU>, grid, dim3(256), 0, s, (const float*)f.x, f.perm,
                           f.offsets, (const float*)f.w_gate, (const float*)f.w_up, (const float*)f.sh_gate,
                           (const float*)f.sh_up, nullptr, (float*)f.h, f.T, f.k, f.N, f.has_shared, f.d, f.d_ff);
    else
        hipLaunchKernelGGL(ffn_f32_kernel<MODE_IN_RELU>, grid, dim3(256), 0, s, (const float*)f.x, f.perm,
                           f.offsets, (const float*)f.w_up, nullptr, (const float*)f.sh_up, nullptr, nullptr,
                           (float*)f.h, f.T, f.k, f.N, f.has_shared, f.d, f.d_ff);
    return hipGetLastError();
}

hipError_t launch_ffn_out(const FfnLaunch& f, hipStream_t s) {
    if (f.T == 0) return hipSuccess;
    if (f.dtype == 1) {
        FfnKArgs a{};
        a.A = (const bf16*)f.h;
        a.perm = f.perm;
        a.offsets = f.offsets;
        a.B0 = (const bf16*)f.w_down;
        a.S0 = (const bf16*)f.sh_down;
        a.row_scale = f.row_scale;
        a.C = f.y_perm;
        a.T = f.T; a.k = f.k; a.N = f.N; a.has_shared = f.has_shared;
        a.K = f.d_ff; a.Ncols = f.d;
        return launch_bf16<MODE_OUT>(a, f.T, f.k, f.N, f.has_shared, s);
    }
    const long long rows_total = (long long)f.T * f.k + (f.has_shared ? f.T : 0);
    const long long n = rows_total * f.d;
    hipLaunchKernelGGL(ffn_f32_kernel<MODE_OUT>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)f.h, f.perm, f.offsets, (const float*)f.w_down, nullptr,
                       (const float*)f.sh_down, nullptr, f.row_scale, (float*)f.y_perm, f.T, f.k, f.N,
                       f.has_shared, f.d_ff, f.d);
    return hipGetLastError();
}
