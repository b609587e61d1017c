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
// bf16 path: v_mfma_f32_32x32x16_bf16, block tiles of 256 or 128 rows, K step 64, LDS double
// buffer filled by direct loads, 4 waves each owning a quarter of the tile.  The in-projection gathers its A
// rows straight from x (row = token of the slot), so the permuted copy of x is never built;
// SwiGLU (silu(g) * u) or ReLU is applied in registers and H is stored in bf16.  The
// out-projection multiplies each row by its slot's gate weight and stores the row in fp32, so the
// combine adds unrounded expert outputs.
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

#define FB_BK 64

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
    int ksplit;             // K is split into ksplit equal parts (out-projection only)
    long long part_stride;  // elements between the fp32 partial outputs of the K parts
};

// Tile configuration: BM rows x BNH output columns per block, WGM x WGN waves; each wave owns a
// (BM/WGM) x (BNH/WGN) block of outputs (for SwiGLU: of both the gate and the up products).
template <int MODE, int BM, int BNH, int WGM, int WGN>
struct FfnTile {
    static constexpr int NT = 64 * WGM * WGN;
    static constexpr int NB = (MODE == MODE_IN_SWIGLU) ? 2 : 1;
    static constexpr int BROWS = NB * BNH;           // weight rows per B tile
    static constexpr int WTM = BM / WGM, WTN = BNH / WGN;
    static constexpr int TM = WTM / 32, TN = WTN / 32;
    static constexpr int ROWS_PER_PASS = NT / 8;     // 8 threads x 16 B cover one 64-wide row
    static constexpr int A_LD = BM / ROWS_PER_PASS, B_LD = BROWS / ROWS_PER_PASS;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
    static_assert(BM % ROWS_PER_PASS == 0 && BROWS % ROWS_PER_PASS == 0, "load passes");
};

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS tile layout: rows of 64 bf16 (128 B, 8 chunks of 16 B), unpadded; chunk c of row r sits at
// position c ^ ((r >> 1) & 7).  A fragment read serves 16 lanes (16 consecutive rows, one chunk,
// 256 B) per LDS cycle; with this swizzle those 16 reads land in 16 distinct 16-byte bank groups
// of the 64 banks.  One wave's direct global->LDS load (64 lanes x 16 B = 8 whole rows) stays
// contiguous in LDS: lane l writes position l & 7 of row 8g + (l >> 3) and therefore fetches
// chunk (l & 7) ^ ((4g + (l >> 4)) & 7) of that row.

// 16 bytes per lane from base + voff + soff into LDS (M0 + 16 * lane): the buffer (MUBUF) form
// of the direct load, with a raw-buffer descriptor (no range limit, 32-bit data format, the gfx9
// encoding).  The per-lane offset is 32 bits and the K offset goes in a scalar register, so no
// per-lane 64-bit address arithmetic is needed.  (A function of its own: the host pass drops a
// kernel whose lambdas use the descriptor type.)
__device__ __forceinline__ void buffer_load_lds16(const void* base, lds_void_t* dst, uint32_t voff, int soff) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, -1, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}

// Work split, computed by wave 0 of every block.  From offsets it counts the real m-tiles of
// each segment (ceil(rows / BM)); the real tiles are numbered segment by segment.  Within a
// segment they go in rectangles of at most 8 m-tiles x (32 / that) n-tiles, m fastest inside a
// rectangle: 32 blocks are what one XCD runs at once (32 CUs, one block each), so the blocks
// that run together on an XCD cover a compact rectangle and share its row tiles and weight
// tiles in that XCD's L2 (a column of 32 m-tiles against one n-tile would fetch every row tile
// again for every n-tile).  The 8 XCDs get equal contiguous ranges of the numbering; blocks are
// dealt to XCDs round-robin (block b runs on XCD b % 8 as its (b / 8)-th block), so every XCD
// gets the same amount of real work.  s_info receives segment (-1: no tile), m-tile, n-tile and
// K part.
template <int BM>
__device__ __forceinline__ void decode_tile(const FfnKArgs& a, int lane, int* s_info) {
    const int b = blockIdx.x;
    const int xcd = b & 7, j = b >> 3;
    int tl[5], loc = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        const int s = lane * 5 + q;
        int rows = 0;
        if (s < a.N) rows = a.offsets[s + 1] - a.offsets[s];
        else if (s == a.N && a.has_shared) rows = a.T;
        tl[q] = (rows + BM - 1) / BM;
        loc += tl[q];
    }
    int incl = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    const int R1 = __shfl(incl, 63, 64) * a.n_tiles;   // tiles of one K part
    const int R = R1 * a.ksplit;
    const int per_xcd = (R + 7) / 8;
    int t = (j < per_xcd) ? xcd * per_xcd + j : R;     // tile id, R = none
    const int ks = t < R ? t / R1 : 0;                  // K part (outermost)
    if (t < R) t -= ks * R1;
    else t = R1;
    int run = (incl - loc) * a.n_tiles;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        const int cnt = tl[q] * a.n_tiles;
        if (t >= run && t < run + cnt) {
            const int rem = t - run, tm = tl[q];
            const int GM = tm < 8 ? tm : 8;               // m-tiles per rectangle
            const int GN = 32 / GM;                       // n-tiles per rectangle
            const int mg = rem / (GM * a.n_tiles);        // rectangle row (GM m-tiles, all n)
            const int gm = min(GM, tm - mg * GM);         // m-tiles in this row (last may be short)
            const int r2 = rem - mg * GM * a.n_tiles;
            const int band = r2 / (gm * GN);              // rectangle within the row
            const int r3 = r2 - band * gm * GN;
            s_info[0] = lane * 5 + q;
            s_info[1] = mg * GM + r3 % gm;
            s_info[2] = band * GN + r3 / gm;
        }
        run += cnt;
    }
    if (lane == 63 && t >= R1) s_info[0] = -1;
    if (lane == 0) s_info[3] = ks;
}

template <int MODE, int BM, int BNH, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_bf16_kernel(FfnKArgs a) {
    using Cfg = FfnTile<MODE, BM, BNH, WGM, WGN>;
    constexpr int NB = Cfg::NB, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int NW = WGM * WGN;
    constexpr int ROWS = BM + Cfg::BROWS;            // rows of one stage (A rows, then B rows)
    constexpr int A_INS = BM / (8 * NW);             // load instructions per wave per stage (A)
    constexpr int B_INS = Cfg::BROWS / (8 * NW);     // (B)
    static_assert(BM % (8 * NW) == 0 && Cfg::BROWS % (8 * NW) == 0, "load split");
    // two stages in two distinct LDS objects, so the compiler can tell a fragment read of one
    // stage from the asynchronous loads into the other
    __shared__ __attribute__((aligned(1024))) bf16 st0[ROWS * 64];
    __shared__ __attribute__((aligned(1024))) bf16 st1[ROWS * 64];
    __shared__ int s_info[4];
    __shared__ float s_scale[MODE == MODE_OUT ? BM : 1];   // gate weight of each row of the tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases go to M0
    if (wave == 0) decode_tile<BM>(a, lane, s_info);
    __syncthreads();
    const int seg = s_info[0];
    if (seg < 0) return;
    const int mt = s_info[1];
    const int n_tile = s_info[2];
    const int kpart = s_info[3];
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
    const int m0 = row_beg + mt * BM;
    const int n0 = n_tile * BNH;

    // per-lane 32-bit byte offsets of this wave's load instructions from a uniform base
    // (x / H stay below 4 GiB, one expert's weight matrix too)
    const int lrow = lane >> 3;                          // row within the 8-row group
    // element offset of the chunk lane fetches for LDS row group g (8 rows)
    auto lchunk = [&](int g) { return ((lane & 7) ^ ((4 * g + (lane >> 4)) & 7)) * 8; };
    uint32_t offA[A_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int rl = 8 * (wave + NW * i) + lrow;
        const int r = (m0 + rl < row_end) ? m0 + rl : m0;
        int src;
        if (MODE == MODE_OUT) src = r;
        else src = (seg < a.N) ? a.perm[r] / a.k : r - a.T * a.k;
        offA[i] = ((uint32_t)src * (uint32_t)a.K + (uint32_t)lchunk(wave + NW * i)) * 2u;
    }
    uint32_t offB[B_INS];
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        const int br = 8 * (wave + NW * i) + lrow;       // row of the B tile
        const int n = n0 + (br % BNH);
        const int nc = n < a.Ncols ? n : n0;
        offB[i] = ((uint32_t)nc * (uint32_t)a.K + (uint32_t)lchunk((BM >> 3) + wave + NW * i)) * 2u;
    }
    const char* baseA = (const char*)a.A;
    const char* baseB0 = (const char*)B0;
    const char* baseB1 = (const char*)(NB == 2 ? B1 : B0);
    const int wm = wave / WGN, wn = wave % WGN;
    // fragment addresses: rows of one wave's fragments differ by multiples of 32, so their
    // swizzle only depends on the lane: row r, chunk c sits at r*64 + ((c ^ ((r >> 1) & 7)) << 3)
    const int fr = lane & 31, fh = lane >> 5, l7 = (fr >> 1) & 7;
    const int abase = (wm * 32 + fr) * 64;              // sub-tile i of this wave: i * WGM + wm
    const int bbase = (BM + wn * Cfg::WTN + fr) * 64;
    struct Frags { bf16x8 a[TM]; bf16x8 b[NB][TN]; };
    auto load_frags = [&](const bf16* st, int kk, Frags& f, auto nv) {
        const int xo = ((2 * kk + fh) ^ l7) << 3;
#pragma unroll
        for (int i = 0; i < decltype(nv)::value; ++i)
            f.a[i] = *(const bf16x8*)(st + abase + i * WGM * 32 * 64 + xo);
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                f.b[m][j] = *(const bf16x8*)(st + bbase + (m * BNH + j * 32) * 64 + xo);
    };
    // The tile's 32-row sub-tiles are dealt to the wave rows in turn (sub-tile s to wave row
    // s % WGM), so the rows of a short tile (an expert's last one) spread over all waves.  A tile
    // whose valid sub-tiles fit in NV per wave runs the variant with NV sub-tiles per wave and
    // skips the MFMAs and fragment reads of the rest; rows past the end were loaded as copies of
    // the first row and are never stored.
    const int rows_valid = row_end - m0;
    const int nsub = (rows_valid + 31) / 32;
    typedef f32x16 Acc[NB][TM][TN];
    auto mfmas = [&](Acc& acc, const Frags& f, auto nv) {
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int i = 0; i < decltype(nv)::value; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[m][j],
                                                                          acc[m][i][j], 0, 0, 0);
            }
    };
    constexpr int NLD = A_INS + B_INS;           // direct-to-LDS loads per stage
    constexpr int NLD0 = (NLD + 1) / 2;          // ... issued during step 0, the rest during step 1
    // Interleave one MFMA with the step's other instructions so that a single wave per SIMD keeps
    // the matrix core busy: MFMA, fragment read, MFMA, load, ...
    auto interleave = [&](int n_ds, int n_ld, auto nv) {
        constexpr int NMF = NB * decltype(nv)::value * TN;   // MFMAs per K=16 step
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);          // MFMA
            if (i < n_ds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
            if (i < n_ld) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
        }
    };
    // A variant with NV sub-tiles per wave reads rows [0, NV * WGM * 32) of the A tile only, so
    // its direct loads skip the rest (those LDS rows are never read).
    auto issue_part = [&](bf16* st, int k0, int beg, int end, auto nv) {
        constexpr int A_NEED = decltype(nv)::value * WGM * 32 / (8 * NW);
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
            if (q < beg || q >= end) continue;
            if (q < A_INS && q >= A_NEED) continue;
            if (q < A_INS) {
                buffer_load_lds16(baseA, (lds_void_t*)(st + (8 * (wave + NW * q)) * 64), offA[q], 2 * k0);
            } else {
                const int i = q - A_INS;
                const int br0 = 8 * NW * i;
                const char* bb = (NB == 2 && br0 >= BNH) ? baseB1 : baseB0;
                buffer_load_lds16(bb, (lds_void_t*)(st + (BM + 8 * (wave + NW * i)) * 64), offB[i], 2 * k0);
            }
        }
    };
    // One stage (K = 64 in four K=16 steps).  On entry f0 holds step 0's fragments and the
    // first half of the next stage's loads is in flight.  The second half goes out during step 0;
    // the barrier sits before step 3, so the next stage's first fragments are read while step 3's
    // MFMAs run, and step 3 already sends the first half of the stage after next into the slot
    // this stage has just released.  Loads past the last stage re-read K offset 0 into the idle
    // slot (in bounds, never used), which keeps the schedule free of branches.
    auto stage = [&](Acc& acc, bf16* cur, bf16* nxt, int k_next, int k_after, Frags& f0, Frags& f1, auto nv) {
        constexpr int NDS = decltype(nv)::value + NB * TN;   // fragment reads per K=16 step
        load_frags(cur, 1, f1, nv);
        issue_part(nxt, k_next, NLD0, NLD, nv);
        mfmas(acc, f0, nv);
        interleave(NDS, NLD - NLD0, nv);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 2, f0, nv);
        mfmas(acc, f1, nv);
        interleave(NDS, 0, nv);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 3, f1, nv);
        mfmas(acc, f0, nv);
        interleave(NDS, 0, nv);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070);    // vmcnt(0) lgkmcnt(0): own loads and reads done
        __syncthreads();                       // next stage visible; this stage no longer read
        load_frags(nxt, 0, f0, nv);
        issue_part(cur, k_after, 0, NLD0, nv);
        mfmas(acc, f1, nv);
        interleave(NDS, NLD0, nv);
        __builtin_amdgcn_sched_barrier(0);
    };

    const int KT = a.K / FB_BK / a.ksplit;                 // stages of this K part
    const int kbase = kpart * KT * FB_BK;
    auto kofs = [&](int t) { return kbase + (t < KT ? t : 0) * FB_BK; };
    // Epilogue.  32x32 C layout: lane holds column (lane & 31); register r holds row
    // 8*(r >> 2) + 4*(lane >> 5) + (r & 3).
    auto store = [&](const Acc& acc, auto nv) {
#pragma unroll
        for (int i = 0; i < decltype(nv)::value; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + (i * WGM + wm) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (row >= row_end) continue;
                const float scale = (MODE == MODE_OUT) ? s_scale[row - m0] : 1.0f;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + wn * Cfg::WTN + j * 32 + (lane & 31);
                    if (col >= a.Ncols) continue;
                    float v;
                    if (MODE == MODE_IN_SWIGLU) v = silu_f32(acc[0][i][j][r]) * acc[NB - 1][i][j][r];
                    else if (MODE == MODE_IN_RELU) v = fmaxf(acc[0][i][j][r], 0.f);
                    else v = acc[0][i][j][r] * scale;
                    if (MODE == MODE_OUT) ((float*)a.C)[kpart * a.part_stride + (size_t)row * a.Ncols + col] = v;
                    else ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)v;
                }
            }
        }
    };
    // Each variant owns its accumulators and epilogue, so no accumulator is live across the
    // choice of variant.
    auto run = [&](auto nv) {
        Acc acc;
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;
        Frags fa, fb;
        // the out-projection's row scales are fetched once per tile, while the first stage loads
        float sc = 1.0f;
        if (MODE == MODE_OUT && tid < BM && m0 + tid < row_end && a.row_scale && seg < a.N)
            sc = a.row_scale[a.perm[m0 + tid]];
        issue_part(st0, kbase, 0, NLD, nv);
        __builtin_amdgcn_s_waitcnt(0x0070);
        if (MODE == MODE_OUT && tid < BM) s_scale[tid] = sc;
        __syncthreads();
        load_frags(st0, 0, fa, nv);
        issue_part(st1, kofs(1), 0, NLD0, nv);
        int kt = 0;
        for (; kt + 2 <= KT; kt += 2) {
            stage(acc, st0, st1, kofs(kt + 1), kofs(kt + 2), fa, fb, nv);
            stage(acc, st1, st0, kofs(kt + 2), kofs(kt + 3), fa, fb, nv);
        }
        if (kt < KT) stage(acc, st0, st1, kbase, kbase, fa, fb, nv);
        __builtin_amdgcn_s_waitcnt(0x0070);    // no load may still be writing LDS at exit
        store(acc, nv);
    };
    if (TM >= 2 && nsub <= WGM) run(std::integral_constant<int, 1>{});
    else if (TM >= 4 && nsub <= 2 * WGM) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, TM>{});
}

// ------------------------------------------------------------------ skinny path (decode)
// For a few rows per expert the GEMMs are weight streams: every weight byte of a touched expert
// is read once and used for at most 16 rows.  One wave owns one 16-column group of one segment
// and the whole K range; its B fragments (16 weight rows x 32 K for v_mfma_f32_16x16x32_bf16)
// come straight from memory into registers, U steps at a time, and its A fragments (the <= 16
// rows, gathered through perm for the in-projection) are shared by all waves through L2.  Waves
// are numbered segment, then column group, so the waves of a block stream neighbouring weight
// rows.  Empty experts are skipped, so only touched
// experts' weights are read.  Segments with more than 16 rows loop over 16-row tiles.  (Weight
// loads stay cached: a load instruction covers half of each 128-byte line it touches and the
// next K step reads the other half; non-temporal loads measured slower.)
template <int MODE, int U>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(FfnKArgs a) {
    constexpr int NB = (MODE == MODE_IN_SWIGLU) ? 2 : 1;
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);        // global wave id
    const int ngroups = (a.Ncols + 15) / 16;
    const int nseg = a.N + (a.has_shared ? 1 : 0);
    const int seg = gw / ngroups, cg = gw % ngroups;
    if (seg >= nseg) return;
    int row_beg, row_end;
    const bf16 *B0, *B1 = nullptr;
    const size_t wstride = (size_t)a.Ncols * a.K;
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
    if (row_end <= row_beg) return;                             // expert not touched
    const int KS = a.K / 32;
    const int col = cg * 16 + (lane & 15);                      // this lane's B column
    const int colc = col < a.Ncols ? col : a.Ncols - 1;
    const int kq = (lane >> 4) * 8;                             // this lane's K offset in a step
    const bf16* pb0 = B0 + (size_t)colc * a.K + kq;
    const bf16* pb1 = (NB == 2) ? B1 + (size_t)colc * a.K + kq : nullptr;
    for (int m0 = row_beg; m0 < row_end; m0 += 16) {
        const int r = m0 + (lane & 15);                         // this lane's A row
        const bool rok = r < row_end;
        int src;
        if (MODE == MODE_OUT) src = rok ? r : m0;
        else src = (seg < a.N) ? a.perm[rok ? r : m0] / a.k : (rok ? r : m0) - a.T * a.k;
        const bf16* pa = a.A + (size_t)src * a.K + kq;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const bf16x8 zero8 = {};
        int ks = 0;
        for (; ks + U <= KS; ks += U) {
            bf16x8 b0[U], b1[U], av[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                b0[u] = *(const bf16x8*)(pb0 + (ks + u) * 32);
                if (NB == 2) b1[u] = *(const bf16x8*)(pb1 + (ks + u) * 32);
                av[u] = rok ? *(const bf16x8*)(pa + (ks + u) * 32) : zero8;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], b0[u], acc0, 0, 0, 0);
                if (NB == 2) acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], b1[u], acc1, 0, 0, 0);
            }
        }
        for (; ks < KS; ++ks) {
            const bf16x8 b0 = *(const bf16x8*)(pb0 + ks * 32);
            const bf16x8 av = rok ? *(const bf16x8*)(pa + ks * 32) : zero8;
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b0, acc0, 0, 0, 0);
            if (NB == 2) {
                const bf16x8 b1 = *(const bf16x8*)(pb1 + ks * 32);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b1, acc1, 0, 0, 0);
            }
        }
        // 16x16 C layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + i
        if (col < a.Ncols) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = m0 + 4 * (lane >> 4) + i;
                if (row >= row_end) continue;
                if (MODE == MODE_OUT) {
                    const float scale = (a.row_scale && seg < a.N) ? a.row_scale[a.perm[row]] : 1.0f;
                    ((float*)a.C)[(size_t)row * a.Ncols + col] = acc0[i] * scale;
                } else if (MODE == MODE_IN_SWIGLU) {
                    ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)(silu_f32(acc0[i]) * acc1[i]);
                } else {
                    ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)fmaxf(acc0[i], 0.f);
                }
            }
        }
    }
}

template <int MODE, int U>
static hipError_t launch_skinny(const FfnKArgs& a, hipStream_t s) {
    const long long waves = (long long)(a.N + (a.has_shared ? 1 : 0)) * ((a.Ncols + 15) / 16);
    auto kern = ffn_skinny_kernel<MODE, U>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Decode-sized batches (at most 16 rows per expert on average) take the weight-streaming path.
// Unroll depths: the in-projection's shallower unroll keeps its registers low enough that all of
// its waves are resident at once.
#define SK_U_IN 4
#define SK_U_OUT 8
static bool skinny(const FfnLaunch& f) { return (long long)f.T * f.k <= 16LL * f.N; }

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
template <int MODE, int BM, int BNH, int WGM, int WGN>
static hipError_t launch_bf16(const FfnKArgs& ka, hipStream_t s) {
    using Cfg = FfnTile<MODE, BM, BNH, WGM, WGN>;
    auto kern = ffn_bf16_kernel<MODE, BM, BNH, WGM, WGN>;
    FfnKArgs a = ka;
    if (a.ksplit < 1) a.ksplit = 1;
    a.mt_max = (a.T * a.k + BM - 1) / BM + a.N + (a.has_shared ? (a.T + BM - 1) / BM : 0);
    a.n_tiles = (a.Ncols + BNH - 1) / BNH;
    const long long G = 8 * (((long long)a.mt_max * a.n_tiles * a.ksplit + 7) / 8);
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(Cfg::NT), 0, s, a);
    return hipGetLastError();
}

// Tile choice from what the host knows (T, k, N, widths): rows per expert on average.
static bool big_tiles(const FfnLaunch& f) {
    return (long long)f.T * f.k >= 192LL * f.N;   // >= 192 rows per expert on average
}

// K parts for the out-projection: two when its K is long and one part alone would leave the
// last round of blocks on the CUs mostly empty.  The parts' fp32 outputs are summed, in order,
// by the combine.
int ffn_out_ksplit(int T, int k, int N, int d, int d_ff, int has_shared, int dtype) {
    if (dtype != 1) return 1;
    const long long rows = (long long)T * k;
    if (rows <= 16LL * N) return 1;                        // weight streaming (decode)
    if (d_ff % (2 * FB_BK) != 0 || d_ff < 8192) return 1;
    if (rows < 192LL * N) return 1;                       // small-tile path: many blocks already
    const long long tiles = ((rows + 255) / 256 + N + (has_shared ? (T + 255) / 256 : 0)) * ((d + 255) / 256);
    return tiles < 4 * 256 ? 2 : 1;
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
            if (skinny(f)) return launch_skinny<MODE_IN_SWIGLU, SK_U_IN>(a, s);
            if (big_tiles(f)) return launch_bf16<MODE_IN_SWIGLU, 256, 128, 2, 2>(a, s);
            return launch_bf16<MODE_IN_SWIGLU, 128, 128, 2, 2>(a, s);
        }
        a.B0 = (const bf16*)f.w_up;
        a.S0 = (const bf16*)f.sh_up;
        if (skinny(f)) return launch_skinny<MODE_IN_RELU, SK_U_IN>(a, s);
        if (big_tiles(f)) return launch_bf16<MODE_IN_RELU, 256, 256, 2, 2>(a, s);
        return launch_bf16<MODE_IN_RELU, 128, 128, 2, 2>(a, s);
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
        a.ksplit = f.ksplit;
        a.part_stride = (long long)((long long)f.T * f.k + (f.has_shared ? f.T : 0)) * f.d;
        if (skinny(f)) return launch_skinny<MODE_OUT, SK_U_OUT>(a, s);
        if (big_tiles(f)) return launch_bf16<MODE_OUT, 256, 256, 2, 2>(a, s);
        return launch_bf16<MODE_OUT, 128, 128, 2, 2>(a, s);
    }
    const long long rows_total = (long long)f.T * f.k + (f.has_shared ? f.T : 0);
    const long long n = rows_total * f.d;
    hipLaunchKernelGGL(ffn_f32_kernel<MODE_OUT>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)f.h, f.perm, f.offsets, (const float*)f.w_down, nullptr,
                       (const float*)f.sh_down, nullptr, f.row_scale, (float*)f.y_perm, f.T, f.k, f.N,
                       f.has_shared, f.d_ff, f.d);
    return hipGetLastError();
}
