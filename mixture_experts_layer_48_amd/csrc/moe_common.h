// Shared device/host helpers of the MoE HIP library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_MAX_EXPERTS 256
#define MOE_EP_MAX_RANKS 64     // expert-parallel ranks of the dispatch / receive layouts
#define MOE_EP_MAX_BLOCKS 4096  // (source rank, local expert) pairs of one receive layout
#define WAVE 64

// Order-preserving map of an fp32 logit to uint32 (larger float -> larger key).
// -0.0 is first folded into +0.0 so that the two zeros compare equal, as they
// do in float arithmetic.
__device__ __forceinline__ uint32_t ordered_key32(float z) {
    z = z + 0.0f;
    uint32_t u = __float_as_uint(z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key32_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}
// 64-bit ranking key: descending logit, then ascending expert id.
__device__ __forceinline__ uint64_t rank_key(float z, int e) {
    return ((uint64_t)ordered_key32(z) << 32) | (uint32_t)(0xFFFFu - (uint32_t)e);
}
__device__ __forceinline__ int key_expert(uint64_t key) { return (int)(0xFFFFu - (uint32_t)(key & 0xFFFFu)); }
__device__ __forceinline__ float key_logit(uint64_t key) { return key32_to_float((uint32_t)(key >> 32)); }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m, WAVE);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, WAVE);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        uint64_t o = shfl_xor_u64(v, m);
        v = o > v ? o : v;
    }
    return v;
}
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
    return v;
}

// Mask of the lanes of this wave whose value equals mine (values < 2^bits).
template <int BITS>
__device__ __forceinline__ uint64_t match_lanes(uint32_t v) {
    uint64_t eq = ~0ull;
#pragma unroll
    for (int b = 0; b < BITS; ++b) {
        uint64_t m = __ballot((v >> b) & 1u);
        eq &= ((v >> b) & 1u) ? m : ~m;
    }
    return eq;
}
__device__ __forceinline__ uint64_t lanemask_lt() {
    int lane = threadIdx.x & (WAVE - 1);
    return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}

// silu(u) = u * sigmoid(u) = u / (1 + e^-u), with the hardware reciprocal (about 1 ulp); for
// u -> -inf the reciprocal of +inf is 0 and the result -0.
__device__ __forceinline__ float silu_f32(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

