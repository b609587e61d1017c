// Step 6 of the MoE layer: the gate-weighted combine.  Each token's output is the sum of its k
// expert outputs weighted by the router's gate weights (page "MoE 分片：混合專家模型的平行化策略",
// section 動態 token 路由, step 6; page "MoE 推理：激活参数 vs 总参数与专家路由", section 代码),
// plus the shared expert's output with weight 1 when the layer has one.
//
// One block per token; the fp32 expert rows are summed in slot order in fp32 and the result is
// rounded once to the layer dtype, so the output does not depend on scheduling.  (bf16 layers
// have d % 64 == 0, so every thread's 8 columns are whole.)
#include "moe_common.h"
#include "moe_kernels.h"

// A row's value is the sum of its nparts K-part partials (added in part order), then
// weighted; part p of row r sits at yp + p * part_stride + r * d.
__device__ __forceinline__ void row8(const float* __restrict__ yp, long long part_stride, int nparts,
                                     size_t off, float v[8]) {
    f32x4 a = *(const f32x4*)(yp + off), b = *(const f32x4*)(yp + off + 4);
    for (int p = 1; p < nparts; ++p) {
        const f32x4 c = *(const f32x4*)(yp + p * part_stride + off);
        const f32x4 e = *(const f32x4*)(yp + p * part_stride + off + 4);
        a += c;
        b += e;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[i + 4] = b[i];
    }
}

// Eight columns of routed row r stored in bf16 (row r at element r * d of the buffer).
__device__ __forceinline__ void row8_bf16(const float* __restrict__ yp, size_t off, float v[8]) {
    const bf16x8 b = *(const bf16x8*)((const bf16*)yp + off);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
}

// One block per token, one thread per 8 columns (the block is as wide as d / 8 allows), so a
// whole output row is one pass.  Slots are taken four at a time: their rows are loaded before
// any of them is added, which keeps four rows' loads in flight, and the adds still run in slot
// order.  A dropped slot (inv < 0) or a slot past k is neither loaded nor added.  With
// routed_bf16 (one K part) the routed rows are bf16 and the shared expert's rows fp32.
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const float* __restrict__ yp,
                                                            const int32_t* __restrict__ inv,
                                                            const float* __restrict__ w,
                                                            bf16* __restrict__ y, int T, int k, int d,
                                                            int has_shared, int nparts, int routed_bf16) {
    const int t = blockIdx.x;
    const int32_t* iv = inv + (size_t)t * k;
    const float* wv = w ? w + (size_t)t * k : nullptr;
    const long long part_stride = ((long long)T * k + (has_shared ? T : 0)) * d;
    for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += 4) {
            int r[4];
            float sc[4];
            bool ok[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + q;
                const int rr = j < k ? iv[j] : -1;
                ok[q] = rr >= 0;
                r[q] = rr;
                sc[q] = (ok[q] && wv) ? wv[j] : 1.0f;
            }
            float v[4][8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (!ok[q]) continue;                                                   // uniform per block
                if (routed_bf16) row8_bf16(yp, (size_t)r[q] * d + c, v[q]);
                else row8(yp, part_stride, nparts, (size_t)r[q] * d + c, v[q]);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (!ok[q]) continue;
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(sc[q], v[q][i], acc[i]);
            }
        }
        if (has_shared) {
            float v[8];
            row8(yp, part_stride, nparts, ((size_t)T * k + t) * d + c, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (bf16)acc[i];
        *(bf16x8*)(y + (size_t)t * d + c) = o;
    }
}

__global__ __launch_bounds__(256) void combine_f32_kernel(const float* __restrict__ yp,
                                                          const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ y, int T, int k, int d,
                                                          int has_shared) {
    const int t = blockIdx.x;
    const int32_t* iv = inv + (size_t)t * k;
    const float* wv = w ? w + (size_t)t * k : nullptr;
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
        float acc = 0.f;
        for (int j = 0; j < k; ++j) {
            const int r = iv[j];
            if (r < 0) continue;
            acc = fmaf(wv ? wv[j] : 1.0f, yp[(size_t)r * d + c], acc);
        }
        if (has_shared) acc += yp[((size_t)T * k + t) * d + c];
        y[(size_t)t * d + c] = acc;
    }
}

hipError_t launch_combine(const void* y_perm, const int32_t* inv, const float* w, void* y, int T,
                          int k, int d, int has_shared, int dtype, int nparts, int routed_bf16, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (dtype == 1) {
        // one thread per 8 columns, in whole waves, at most 1024
        int threads = ((d / 8 + 63) / 64) * 64;
        threads = threads < 64 ? 64 : (threads > 1024 ? 1024 : threads);
        hipLaunchKernelGGL(combine_bf16_kernel, dim3(T), dim3(threads), 0, s, (const float*)y_perm, inv, w,
                           (bf16*)y, T, k, d, has_shared, nparts < 1 ? 1 : nparts, routed_bf16);
    }
    else
        hipLaunchKernelGGL(combine_f32_kernel, dim3(T), dim3(256), 0, s, (const float*)y_perm, inv, w,
                           (float*)y, T, k, d, has_shared);
    return hipGetLastError();
}
