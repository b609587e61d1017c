// Int4 expert weights: quantisation and the weight-streaming expert FFN that reads them.
//
// The pages name INT4 (GPTQ/AWQ) expert weights at a quarter of the memory (page "大模型MoE混合专家
// 架构原理与DeepSeek-V4工程实践解析", section DeepSeek-V4的MoE架构工程细节) without a format; the one
// used here:
//   per output (a column of the [K, rows] weight matrix, a row of the codes) and group of 128
//   consecutive inputs, scale = amax / 7 (fp32) and
//   q = clamp(rint(w / scale), -8, 7) (fp32 division, ties to even; an all-zero group has scale 0
//   and q = 0); the weight it stands for is scale * q.
//   codes q + 8, four bits each, eight to a uint32: within row r and group g, word a*4 + s
//   (a, s in 0..3) holds inputs k = 128 g + 32 s + 8 a + i, i = 0..7, input i at bit
//   4 (i / 2) + 16 (i % 2).  Codes [mats, rows, K / 8] uint32; scales [mats, K / 128, rows] fp32.
// With this order one 16-byte load gives a lane its codes for the four 32-input MFMA steps of a
// group, and (word >> 4j) & 0x000F000F | 0x43004300 turns two codes at once into the bf16 values
// 128 + code = 136 + q.  The MFMA sums (136 + q) x over a group; one more MFMA against a
// fragment of ones gives the group's sum of x, and scale * (sum - 136 * sum_x) is the group's
// share of the product, added in fp32.
#include "moe_common.h"
#include "moe_kernels.h"

namespace {

enum { MODE_IN_SWIGLU = 0, MODE_IN_RELU = 1, MODE_OUT = 2 };
constexpr int Q4G = 128;   // inputs per scale group

// ------------------------------------------------------------------ quantisation
// Input: n_mats bf16 matrices [K, rows] (x W orientation: column r holds output r's weights).
// One wave per 64 consecutive columns and one group of 128 inputs: lane l takes column r0 + l,
// reads its 128 inputs (each read of the wave is 128 contiguous bytes of one k-row), finds the
// group's scale and codes in fp32 and writes its 16 code words and its scale.
__global__ __launch_bounds__(256) void q4_quantize_kernel(const bf16* __restrict__ w, long long n_mats, int rows,
                                                          int K, uint32_t* __restrict__ codes,
                                                          float* __restrict__ scales) {
    const int G = K / Q4G, RB = (rows + 63) / 64;
    const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= n_mats * RB * G) return;
    const int lane = threadIdx.x & 63;
    const long long mat = wid / ((long long)RB * G);
    const int rem = (int)(wid % ((long long)RB * G));
    const int g = rem % G, r = (rem / G) * 64 + lane;
    if (r >= rows) return;
    const bf16* src = w + (size_t)mat * K * rows + (size_t)g * Q4G * rows + r;
    float v[Q4G];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < Q4G; ++i) {
        v[i] = (float)src[(size_t)i * rows];
        amax = fmaxf(amax, fabsf(v[i]));
    }
    float sc = 0.0f;
    if (amax > 0.0f) sc = __fdiv_rn(amax, 7.0f);
    // word a*4 + s of the group holds inputs 32 s + 8 a + i, input i at bit 4 (i / 2) + 16 (i % 2)
    uint32_t* out = codes + ((size_t)mat * rows + r) * (K / 8) + (size_t)g * 16;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                int q = 0;
                if (amax > 0.0f) q = (int)fminf(fmaxf(rintf(__fdiv_rn(v[32 * s + 8 * a + i], sc)), -8.0f), 7.0f);
                word |= (uint32_t)(q + 8) << (4 * (i >> 1) + 16 * (i & 1));
            }
            out[4 * a + s] = word;
        }
    scales[((size_t)mat * G + g) * rows + r] = sc;
}

// ------------------------------------------------------------------ weight-streaming FFN
struct FfnQ4Args {
    const bf16* A;              // in: x [T, d]; out: H [rows, d_ff]
    const int32_t* perm;
    const int32_t* offsets;
    const uint32_t* B0;         // routed codes [N, Ncols, K / 8] (gate for SwiGLU, else W)
    const uint32_t* B1;         // routed up codes (SwiGLU) or null
    const float* SB0;           // routed scales [N, K / 128, Ncols]
    const float* SB1;
    const uint32_t* S0;         // shared expert codes [Ncols, K / 8] or null
    const uint32_t* S1;
    const float* SS0;           // shared expert scales [K / 128, Ncols]
    const float* SS1;
    const float* row_scale;     // [T*k] or null (out-projection only)
    void* C;                    // bf16 H (in-projection) or fp32 y_perm (out-projection)
    int T, k, N, has_shared, K, Ncols;
};

__device__ __forceinline__ bf16x8 q4_to_bf16(uint32_t w) {
    u32x4 d;
    d[0] = (w & 0x000F000Fu) | 0x43004300u;
    d[1] = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    d[2] = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    d[3] = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, d);
}

// One wave owns CG 16-column groups of one segment and the whole K range, UG groups of 128
// inputs per step of its loop (their codes, scales and activations loaded before use).  Layout
// of the MFMA operands and result as in the bf16 weight-streaming kernel: activations are the A
// operand (lane: row lane & 15, inputs 8 (lane >> 4) .. + 7 of a 32-input step), weights the B
// operand (lane: column lane & 15, same inputs), result lane: column lane & 15, rows
// 4 (lane >> 4) + i.
template <int MODE, int CG, int UG>
__global__ __launch_bounds__(256) void ffn_skinny_q4_kernel(FfnQ4Args a) {
    constexpr int NB = (MODE == MODE_IN_SWIGLU) ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int ngroups = (a.Ncols + 16 * CG - 1) / (16 * CG);
    const int nseg = a.N + (a.has_shared ? 1 : 0);
    const int seg = gw / ngroups, cg = gw % ngroups;
    if (seg >= nseg) return;
    const int KG = a.K / Q4G;
    int row_beg, row_end;
    const uint32_t *B0, *B1 = nullptr;
    const float *SB0, *SB1 = nullptr;
    if (seg < a.N) {
        row_beg = a.offsets[seg];
        row_end = a.offsets[seg + 1];
        const size_t cs = (size_t)a.Ncols * (a.K / 8), ss = (size_t)KG * a.Ncols;
        B0 = a.B0 + seg * cs;
        SB0 = a.SB0 + seg * ss;
        if (NB == 2) { B1 = a.B1 + seg * cs; SB1 = a.SB1 + seg * ss; }
    } else {
        row_beg = a.T * a.k;
        row_end = row_beg + a.T;
        B0 = a.S0;
        SB0 = a.SS0;
        if (NB == 2) { B1 = a.S1; SB1 = a.SS1; }
    }
    if (row_end <= row_beg) return;                             // expert not touched
    const int kq = (lane >> 4) * 8;
    int colc[CG];
    const uint32_t* pb0[CG];
    const uint32_t* pb1[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
        const int col = (cg * CG + c) * 16 + (lane & 15);
        colc[c] = col < a.Ncols ? col : a.Ncols - 1;
        // this lane's four words of group g: 16 g + 4 (lane >> 4) .. + 3
        pb0[c] = B0 + (size_t)colc[c] * (a.K / 8) + 4 * (lane >> 4);
        pb1[c] = (NB == 2) ? B1 + (size_t)colc[c] * (a.K / 8) + 4 * (lane >> 4) : nullptr;
    }
    const bf16x8 zero8 = {};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, (u32x4){0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    for (int m0 = row_beg; m0 < row_end; m0 += 16) {
        const int r = m0 + (lane & 15);
        const bool rok = r < row_end;
        int src;
        if (MODE == MODE_OUT) src = rok ? r : m0;
        else src = (seg < a.N) ? a.perm[rok ? r : m0] / a.k : (rok ? r : m0) - a.T * a.k;
        const bf16* pa = a.A + (size_t)src * a.K + kq;
        f32x4 tot0[CG], tot1[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) { tot0[c] = zero4; tot1[c] = zero4; }
        for (int g0 = 0; g0 < KG; g0 += UG) {
            u32x4 w0[UG][CG], w1[UG][CG];
            float s0[UG][CG], s1[UG][CG];
            bf16x8 av[UG][4];
#pragma unroll
            for (int u = 0; u < UG; ++u) {
                const int g = g0 + u < KG ? g0 + u : KG - 1;      // past the end: loaded, never added
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    w0[u][c] = *(const u32x4*)(pb0[c] + 16 * g);
                    s0[u][c] = SB0[(size_t)g * a.Ncols + colc[c]];
                    if (NB == 2) {
                        w1[u][c] = *(const u32x4*)(pb1[c] + 16 * g);
                        s1[u][c] = SB1[(size_t)g * a.Ncols + colc[c]];
                    }
                }
#pragma unroll
                for (int st = 0; st < 4; ++st) av[u][st] = rok ? *(const bf16x8*)(pa + g * Q4G + 32 * st) : zero8;
            }
#pragma unroll
            for (int u = 0; u < UG; ++u) {
                if (g0 + u >= KG) break;
                f32x4 sx = zero4;
#pragma unroll
                for (int st = 0; st < 4; ++st) sx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][st], ones, sx, 0, 0, 0);
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    f32x4 p0 = zero4, p1 = zero4;
#pragma unroll
                    for (int st = 0; st < 4; ++st) {
                        p0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][st], q4_to_bf16(w0[u][c][st]), p0, 0, 0, 0);
                        if (NB == 2)
                            p1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][st], q4_to_bf16(w1[u][c][st]), p1, 0, 0, 0);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        tot0[c][i] += s0[u][c] * (p0[i] - 136.0f * sx[i]);
                        if (NB == 2) tot1[c][i] += s1[u][c] * (p1[i] - 136.0f * sx[i]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            const int col = (cg * CG + c) * 16 + (lane & 15);
            if (col >= a.Ncols) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 4 * (lane >> 4) + i;
                if (row >= row_end) continue;
                if (MODE == MODE_OUT) {
                    const float scale = (a.row_scale && seg < a.N) ? a.row_scale[a.perm[row]] : 1.0f;
                    ((float*)a.C)[(size_t)row * a.Ncols + col] = tot0[c][i] * scale;
                } else if (MODE == MODE_IN_SWIGLU) {
                    ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)(silu_f32(tot0[c][i]) * tot1[c][i]);
                } else {
                    ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)fmaxf(tot0[c][i], 0.f);
                }
            }
        }
    }
}

template <int MODE, int CG, int UG>
hipError_t launch_q4(const FfnQ4Args& a, hipStream_t s) {
    const long long waves = (long long)(a.N + (a.has_shared ? 1 : 0)) * ((a.Ncols + 16 * CG - 1) / (16 * CG));
    auto kern = ffn_skinny_q4_kernel<MODE, CG, UG>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Column groups per wave and groups of 128 inputs per loop step (measured on the Mixtral decode
// layer: in-projection 0.120 ms at 2 x 2, against 0.123-0.136 ms for 1 x 1..4 and 4 x 1;
// out-projection 0.069 ms at 2 x 4, against 0.084-0.099 ms for 1 x 2..8 and 2 x 2; a register
// double buffer of the next groups was slower for every pair, its registers halving the waves
// per SIMD).
#ifndef Q4_CG_IN
#define Q4_CG_IN 2
#endif
#ifndef Q4_UG_IN
#define Q4_UG_IN 2
#endif
#ifndef Q4_CG_OUT
#define Q4_CG_OUT 2
#endif
#ifndef Q4_UG_OUT
#define Q4_UG_OUT 4
#endif

}  // namespace

hipError_t launch_q4_quantize(const void* w, long long n_mats, int rows, int K, uint32_t* codes, float* scales,
                              hipStream_t s) {
    const long long waves = n_mats * ((rows + 63) / 64) * (K / Q4G);
    if (waves == 0) return hipSuccess;
    q4_quantize_kernel<<<(unsigned)((waves + 3) / 4), 256, 0, s>>>((const bf16*)w, n_mats, rows, K, codes, scales);
    return hipGetLastError();
}

hipError_t launch_ffn_in_q4(const FfnLaunch& f, hipStream_t s) {
    if (f.T == 0) return hipSuccess;
    FfnQ4Args a{};
    a.A = (const bf16*)f.x;
    a.perm = f.perm;
    a.offsets = f.offsets;
    a.C = f.h;
    a.T = f.T; a.k = f.k; a.N = f.N; a.has_shared = f.has_shared;
    a.K = f.d; a.Ncols = f.d_ff;
    if (f.ffn == 1) {
        a.B0 = f.q4.gate; a.SB0 = f.q4.gate_scales; a.B1 = f.q4.up; a.SB1 = f.q4.up_scales;
        a.S0 = f.q4.sh_gate; a.SS0 = f.q4.sh_gate_scales; a.S1 = f.q4.sh_up; a.SS1 = f.q4.sh_up_scales;
        return launch_q4<MODE_IN_SWIGLU, Q4_CG_IN, Q4_UG_IN>(a, s);
    }
    a.B0 = f.q4.up; a.SB0 = f.q4.up_scales;
    a.S0 = f.q4.sh_up; a.SS0 = f.q4.sh_up_scales;
    return launch_q4<MODE_IN_RELU, Q4_CG_IN, Q4_UG_IN>(a, s);
}

hipError_t launch_ffn_out_q4(const FfnLaunch& f, hipStream_t s) {
    if (f.T == 0) return hipSuccess;
    FfnQ4Args a{};
    a.A = (const bf16*)f.h;
    a.perm = f.perm;
    a.offsets = f.offsets;
    a.B0 = f.q4.down; a.SB0 = f.q4.down_scales;
    a.S0 = f.q4.sh_down; a.SS0 = f.q4.sh_down_scales;
    a.row_scale = f.row_scale;
    a.C = f.y_perm;
    a.T = f.T; a.k = f.k; a.N = f.N; a.has_shared = f.has_shared;
    a.K = f.d_ff; a.Ncols = f.d;
    return launch_q4<MODE_OUT, Q4_CG_OUT, Q4_UG_OUT>(a, s);
}
