// Step 4 of the MoE layer: group the (token, slot) pairs by target expert so that each expert
// sees one contiguous block of rows (page "MoE稀疏激活原理与工程实践：揭秘大模型参数幻觉",
// section 3.1: tokens routed one by one, then regrouped by expert id before the experts run).
//
// The same kernel, keyed by (owner rank, expert), gives the expert-parallel send layout: each
// destination rank's rows are one contiguous range (page "MoE 分片：混合專家模型的平行化策略",
// sections 專家平行化詳解 and 動態 token 路由, steps 3-5: tokens go to the GPUs that own their
// experts and come back for the combine).
//
// One block of 1024 threads does the whole grouping, deterministically and without atomics on
// the output order:
//   1. each wave counts its contiguous range of slots per expert (LDS histogram per wave);
//   2. counts, the exclusive scan over experts (offsets) and each wave's starting row per
//      expert (offsets[e] + counts of e in earlier waves);
//   3. each wave walks its range again in groups of 64 slots, in order and independently of the
//      other waves; a lane's row is its wave's next free row for its expert plus the number of
//      lower lanes with the same expert (ballot matching), so rows of an expert are in
//      ascending slot order.
#include "moe_common.h"
#include "moe_kernels.h"

#define PM_THREADS 1024
#define PM_WAVES (PM_THREADS / 64)
#define PM_BATCH 16   // groups of 64 slots whose expert ids one wave loads together

// Destination-major keys for the expert-parallel send layout: experts are ordered by (owner
// rank, expert id); pos[e] is expert e's place in that order, exp_at inverts it, and rank r's
// experts occupy places rank_first[r] .. rank_first[r+1]-1.  Built on the host, passed by value.
struct EpMapArg {
    int pos[MOE_MAX_EXPERTS];
    int exp_at[MOE_MAX_EXPERTS];
    int rank_first[MOE_EP_MAX_RANKS + 1];
    int G;
};
struct NoMapArg {};

// EP = false: plain grouping by expert.  EP = true: grouping by (owner rank, expert), plus the
// per-rank row counts and offsets.  In both, rows of one expert are in ascending slot order;
// slots whose index is outside [0, N) are dropped (inv -1).
template <bool EP, typename MapT>
__global__ __launch_bounds__(PM_THREADS) void permute_kernel(
    const int32_t* __restrict__ idx, int S, int N, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ inv, const MapT map,
    int32_t* __restrict__ send_counts, int32_t* __restrict__ send_offsets) {
    __shared__ int hist[PM_WAVES][MOE_MAX_EXPERTS];
    __shared__ int offs[MOE_MAX_EXPERTS + 1];
    __shared__ int s_pos[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // equal contiguous ranges per wave, a multiple of 64 slots each
    const int per_wave = ((S + PM_WAVES * 64 - 1) / (PM_WAVES * 64)) * 64;
    const int beg = wave * per_wave;
    const int end = min(S, beg + per_wave);

    for (int i = tid; i < PM_WAVES * MOE_MAX_EXPERTS; i += PM_THREADS) (&hist[0][0])[i] = 0;
    if constexpr (EP) {
        for (int e = tid; e < N; e += PM_THREADS) s_pos[e] = map.pos[e];
    }
    __syncthreads();
    // key of a slot: its expert's place in the layout, or -1 (dropped)
    auto key_of = [&](int e) -> int {
        if (e < 0 || e >= N) return -1;
        if constexpr (EP) return s_pos[e];
        return e;
    };
    // A lane's slots are beg + lane + 64 g.  Their ids are loaded PM_BATCH groups at a time, all
    // loads of a batch in flight together (one at a time, each load's latency was paid in turn).
    auto load_batch = [&](int g0, int (&ev)[PM_BATCH]) {
#pragma unroll
        for (int u = 0; u < PM_BATCH; ++u) {
            const int s = beg + g0 + u * 64 + lane;
            ev[u] = s < end ? idx[s] : -1;
        }
    };
    for (int g0 = 0; g0 < per_wave; g0 += 64 * PM_BATCH) {
        int ev[PM_BATCH];
        load_batch(g0, ev);
#pragma unroll
        for (int u = 0; u < PM_BATCH; ++u) {
            const int e = key_of(ev[u]);
            if (e >= 0) atomicAdd(&hist[wave][e], 1);  // integer counts: order-independent
        }
    }
    __syncthreads();
    if (tid < 64) {  // one wave: totals, exclusive scan over places
        int tot[4], run = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid * 4 + q;
            int c = 0;
            if (e < N)
                for (int ww = 0; ww < PM_WAVES; ++ww) c += hist[ww][e];
            tot[q] = c;
            run += c;
        }
        // inclusive scan of per-lane sums across the wave
        int incl = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (tid >= o) incl += v;
        }
        int base = incl - run;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid * 4 + q;
            if (e < N) {
                offs[e] = base;
                int ge = e;  // the expert at this place
                if constexpr (EP) ge = map.exp_at[e];
                counts[ge] = tot[q];
                offsets[ge] = base;
            }
            base += tot[q];
        }
        if (tid == 63) {
            offs[N] = incl;
            offsets[N] = incl;
        }
    }
    __syncthreads();
    if constexpr (EP) {
        for (int r = tid; r <= map.G; r += PM_THREADS) {
            send_offsets[r] = offs[map.rank_first[r]];
            if (r < map.G) send_counts[r] = offs[map.rank_first[r + 1]] - offs[map.rank_first[r]];
        }
    }
    // per-wave starting row of each place: offs[e] + counts of e in earlier waves
    for (int e = tid; e < N; e += PM_THREADS) {
        int run = offs[e];
        for (int ww = 0; ww < PM_WAVES; ++ww) {
            const int c = hist[ww][e];
            hist[ww][e] = run;
            run += c;
        }
    }
    __syncthreads();
    for (int g0 = 0; g0 < per_wave; g0 += 64 * PM_BATCH) {
      int ev[PM_BATCH];
      load_batch(g0, ev);
#pragma unroll
      for (int u = 0; u < PM_BATCH; ++u) {
        const int g = g0 + u * 64;
        if (g >= per_wave) break;                        // uniform: past the wave's range
        const int s = beg + g + lane;
        const bool valid = s < end;
        const int e = valid ? key_of(ev[u]) : -1;
        const uint64_t eq = match_lanes<9>((uint32_t)(e + 1));
        const uint64_t lt = lanemask_lt();
        if (e >= 0) {
            const int r = hist[wave][e] + __popcll(eq & lt);
            perm[r] = s;
            inv[s] = r;
        } else if (valid) {
            inv[s] = -1;
        }
        // hist[wave] is this wave's own row: its LDS reads and writes complete in program
        // order, so the group's update needs no block barrier, only the compiler kept from
        // moving LDS accesses across it
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (e >= 0 && (eq & ~(lt | (1ull << lane))) == 0)  // highest lane of its group
            hist[wave][e] += __popcll(eq);
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        __builtin_amdgcn_wave_barrier();
      }
    }
}

// The same grouping over many blocks, for large slot counts (the fused forward, which has a
// workspace for the per-block counts): one block of 1024 threads does 1024 slots' worth of it,
// where the single block above walks every slot in 64-slot groups (65536 slots of the
// DeepSeek-V3 shape: 66 us on one CU).
//   1. permute_count_kernel: block b counts its slots per expert;
//   2. permute_scan_kernel (one block): counts, the exclusive scan over experts (offsets), and in
//      place of each block's count its first row for that expert (offsets[e] + the counts of e in
//      earlier blocks);
//   3. permute_place_kernel: a slot's row is its block's first row for its expert, plus the
//      slots with that expert in earlier waves of the block, plus the lower lanes of its own wave
//      with that expert (ballot matching): rows of an expert are in ascending slot order, so the
//      result is the single-block kernel's, bit for bit.
#define PMB_SLOTS 1024
#define PMB_WAVES (PMB_SLOTS / 64)

__global__ __launch_bounds__(PMB_SLOTS) void permute_count_kernel(const int32_t* __restrict__ idx, int S, int N,
                                                                  int32_t* __restrict__ cnt) {
    __shared__ int h[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    for (int e = tid; e < N; e += PMB_SLOTS) h[e] = 0;
    __syncthreads();
    const int s = blockIdx.x * PMB_SLOTS + tid;
    const int e = s < S ? idx[s] : -1;
    if (e >= 0 && e < N) atomicAdd(&h[e], 1);              // integer counts: order-independent
    __syncthreads();
    for (int x = tid; x < N; x += PMB_SLOTS) cnt[(size_t)blockIdx.x * N + x] = h[x];
}

__global__ __launch_bounds__(MOE_MAX_EXPERTS) void permute_scan_kernel(int32_t* __restrict__ cnt, int B, int N,
                                                                       int32_t* __restrict__ counts,
                                                                       int32_t* __restrict__ offsets) {
    __shared__ int s_tot[MOE_MAX_EXPERTS];
    __shared__ int s_off[MOE_MAX_EXPERTS + 1];
    const int tid = threadIdx.x;                           // one thread per expert (N <= 256)
    auto sum_blocks = [&](int e) {                         // block counts loaded eight at a time
        int tot = 0;
        for (int b0 = 0; b0 < B; b0 += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = b0 + i < B ? cnt[(size_t)(b0 + i) * N + e] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) tot += v[i];
        }
        return tot;
    };
    if (tid < N) s_tot[tid] = sum_blocks(tid);
    __syncthreads();
    if (tid < 64) {  // one wave: exclusive scan over experts, four per lane
        int tot[4], run = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid * 4 + q;
            tot[q] = e < N ? s_tot[e] : 0;
            run += tot[q];
        }
        int incl = run;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int v = __shfl_up(incl, o, 64);
            if (tid >= o) incl += v;
        }
        int base = incl - run;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid * 4 + q;
            if (e < N) {
                s_off[e] = base;
                counts[e] = tot[q];
                offsets[e] = base;
            }
            base += tot[q];
        }
        if (tid == 63) offsets[N] = incl;
    }
    __syncthreads();
    if (tid < N) {
        int run = s_off[tid];
        for (int b0 = 0; b0 < B; b0 += 8) {
            int v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = b0 + i < B ? cnt[(size_t)(b0 + i) * N + tid] : 0;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (b0 + i < B) {
                    cnt[(size_t)(b0 + i) * N + tid] = run;
                    run += v[i];
                }
        }
    }
}

__global__ __launch_bounds__(PMB_SLOTS) void permute_place_kernel(const int32_t* __restrict__ idx, int S, int N,
                                                                  const int32_t* __restrict__ base,
                                                                  int32_t* __restrict__ perm, int32_t* __restrict__ inv) {
    __shared__ int cw[PMB_WAVES][MOE_MAX_EXPERTS];        // slots per expert in each wave
    const int tid = threadIdx.x, wave = tid >> 6;
    for (int i = tid; i < PMB_WAVES * N; i += PMB_SLOTS) cw[i / N][i % N] = 0;
    __syncthreads();
    const int s = blockIdx.x * PMB_SLOTS + tid;
    const bool valid = s < S;
    const int ev = valid ? idx[s] : -1;
    const int e = (ev >= 0 && ev < N) ? ev : -1;
    const uint64_t eq = match_lanes<9>((uint32_t)(e + 1));  // every lane takes part
    const int rin = __popcll(eq & lanemask_lt());
    if (e >= 0 && rin == 0) cw[wave][e] = __popcll(eq);
    __syncthreads();
    if (e >= 0) {
        int r = base[(size_t)blockIdx.x * N + e] + rin;
        for (int w = 0; w < wave; ++w) r += cw[w][e];
        perm[r] = s;
        inv[s] = r;
    } else if (valid) {
        inv[s] = -1;
    }
}

// Optional materialised gather: x_perm[r] = x[perm[r] / k] for r < offsets[N].
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          const int32_t* __restrict__ perm,
                                                          const int32_t* __restrict__ offsets, int N,
                                                          int k, int row_bytes, uint8_t* __restrict__ xp) {
    const int r = blockIdx.x;
    if (r >= offsets[N]) return;
    const int t = perm[r] / k;
    if ((row_bytes & 15) == 0) {  // every row starts 16-byte aligned
        const u32x4* src = (const u32x4*)(x + (size_t)t * row_bytes);
        u32x4* dst = (u32x4*)(xp + (size_t)r * row_bytes);
        for (int i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
    } else {
        for (int i = threadIdx.x; i < row_bytes; i += blockDim.x)
            xp[(size_t)r * row_bytes + i] = x[(size_t)t * row_bytes + i];
    }
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int N, int32_t* counts, int32_t* offsets,
                          int32_t* perm, int32_t* inv, hipStream_t s) {
    const int S = T * k;
    permute_kernel<false, NoMapArg><<<1, PM_THREADS, 0, s>>>(idx, S, N, counts, offsets, perm, inv, NoMapArg{},
                                                             nullptr, nullptr);
    return hipGetLastError();
}

size_t permute_multi_workspace_bytes(int T, int k, int N) {
    const long long S = (long long)T * k;
    return (size_t)((S + PMB_SLOTS - 1) / PMB_SLOTS) * N * sizeof(int32_t);
}

hipError_t launch_permute_multi(const int32_t* idx, int T, int k, int N, int32_t* counts, int32_t* offsets,
                                int32_t* perm, int32_t* inv, int32_t* ws, hipStream_t s) {
    const int S = T * k;
    if (S == 0) return hipSuccess;
    if (N > MOE_MAX_EXPERTS || !ws) return hipErrorInvalidValue;
    const int B = (S + PMB_SLOTS - 1) / PMB_SLOTS;
    permute_count_kernel<<<B, PMB_SLOTS, 0, s>>>(idx, S, N, ws);
    permute_scan_kernel<<<1, MOE_MAX_EXPERTS, 0, s>>>(ws, B, N, counts, offsets);
    permute_place_kernel<<<B, PMB_SLOTS, 0, s>>>(idx, S, N, ws, perm, inv);
    return hipGetLastError();
}

hipError_t launch_ep_dispatch(const int32_t* idx, int T, int k, int N, const int32_t* owner, int G,
                              int32_t* counts, int32_t* expert_offsets, int32_t* send_counts,
                              int32_t* send_offsets, int32_t* perm, int32_t* inv, hipStream_t s) {
    // places ordered by (owner, expert id): a counting sort over the ranks
    EpMapArg m{};
    m.G = G;
    int nper[MOE_EP_MAX_RANKS] = {0};
    for (int e = 0; e < N; ++e) nper[owner[e]]++;
    m.rank_first[0] = 0;
    for (int r = 0; r < G; ++r) m.rank_first[r + 1] = m.rank_first[r] + nper[r];
    int next[MOE_EP_MAX_RANKS];
    for (int r = 0; r < G; ++r) next[r] = m.rank_first[r];
    for (int e = 0; e < N; ++e) {
        const int p = next[owner[e]]++;
        m.pos[e] = p;
        m.exp_at[p] = e;
    }
    permute_kernel<true, EpMapArg><<<1, PM_THREADS, 0, s>>>(idx, T * k, N, counts, expert_offsets, perm, inv, m,
                                                           send_counts, send_offsets);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm, const int32_t* offsets, int T,
                              int k, int N, int row_bytes, void* x_perm, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(gather_rows_kernel, dim3(T * k), dim3(256), 0, s, (const uint8_t*)x, perm,
                       offsets, N, k, row_bytes, (uint8_t*)x_perm);
    return hipGetLastError();
}
