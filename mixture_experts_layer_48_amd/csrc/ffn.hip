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
// bf16 path: v_mfma_f32_32x32x16_bf16, block tiles of 128, 256 or 320 rows, K step 64, LDS
// double buffer filled by direct loads, 4 or 8 waves each owning an equal part of the tile.  The in-projection gathers its A
// rows straight from x (row = token of the slot), so the permuted copy of x is never built;
// SwiGLU (silu(g) * u) or ReLU is applied in registers and H is stored in bf16.  The
// out-projection multiplies each row by its slot's gate weight and stores the row in fp32, so the
// combine adds unrounded expert outputs.
#include <mutex>
#include <type_traits>

#include "moe_common.h"
#include "moe_kernels.h"

#define FB_BK 64

enum { MODE_IN_SWIGLU = 0, MODE_IN_RELU = 1, MODE_OUT = 2 };

struct FfnKArgs {
    const bf16* A;          // in: x [T, d]; out: H [rows, d_ff]
    const int32_t* perm;
    const int32_t* offsets;
    const bf16* B0;         // routed weights [N, K, Ncols], K-major (gate for SwiGLU, else W)
    const bf16* B1;         // routed up weights (SwiGLU) or null
    const bf16* S0;         // shared expert [K, Ncols] or null
    const bf16* S1;
    const float* row_scale; // [T*k] or null (out-projection only)
    void* C;                // [rows, Ncols]: bf16 H (in-projection) or fp32 y_perm (out-projection)
    int T, k, N, has_shared, K, Ncols, mt_max, n_tiles;
    int ksplit;             // K is split into ksplit equal parts (out-projection only)
    long long part_stride;  // elements between the fp32 partial outputs of the K parts
    int small_rows;         // > 0: routed experts with 1 .. small_rows rows go to the weight-stream
                            // kernel, and the tiled kernels leave them out
    int routed_bf16;        // out-projection, one K part: routed rows stored in bf16 (row r at
                            // element r * Ncols of C viewed as bf16), the shared rows in fp32
    unsigned int* ctr;      // claiming GEMM: its schedule memory, 8 claim counters and from
                            // word FFN_CTR_BYTES / 4 on the tile table (ffn_tile_table)
};

__device__ __forceinline__ int4* tile_table(const FfnKArgs& a) {
    return (int4*)((char*)a.ctr + FFN_CTR_BYTES);
}

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

// Work split.  Wave 0 of every block turns offsets into a segment table in LDS: each segment's
// first tile, its m-tile count (ceil(rows / BM)) and its row range.  Real tiles are numbered
// segment by segment, K part outermost.  Within a segment they go in rectangles of at most 8
// m-tiles x (32 / that) n-tiles, m fastest inside a rectangle: one XCD works on 32 tiles at once
// (32 CUs, one block each), so the tiles it holds together cover a compact rectangle and share
// its row tiles and weight tiles in that XCD's L2 (a column of 32 m-tiles against one n-tile
// would fetch every row tile again for every n-tile).  The 8 XCDs get equal contiguous ranges
// of the numbering (block b runs on XCD b % 8).
//
// The kernel is persistent: the grid holds only as many blocks as the CUs keep resident, and
// each block runs a sequence of tiles from its XCD's range.  The in-projections (and 128-row
// tiles) deal the range: round i of it to the XCD's blocks in order, reversed on odd rounds, so
// that a pattern of period two (a full m-tile next to an expert's short last one) does not fall
// on the same blocks every round.  The out-projection with 256- and 320-row tiles claims tiles
// one at a time with an atomic counter per range (the XCD's blocks take the range in order, so
// the tiles in flight together still form the rectangles above) and, once its own range is used
// up, from the other XCDs' ranges: a block that runs faster (a shorter tile, a less contended CU)
// takes more, instead of the launch waiting for the slowest share.
#define FFN_MAX_SEG 320   // 5 segments per lane of one wave: routed experts and the shared one

// Sub-tiles per wave of the variant a tile with nsub valid 32-row sub-tiles runs: the fewest of
// 1, 2, 4 (when below TM) and TM that holds them.
template <int TM, int WGM>
__device__ __forceinline__ int variant_nv(int nsub) {
    if (TM >= 2 && nsub <= WGM) return 1;
    if (TM >= 4 && nsub <= 2 * WGM) return 2;
    if (TM >= 5 && nsub <= 4 * WGM) return 4;
    return TM;
}

// Estimated cost of a tile in 1/256 of a full tile: a short tile (an expert's last m-tile) runs
// the variant with fewer sub-tiles per wave and costs a fixed part, its weight stream, plus its
// share of the MFMAs.  The fixed part is half a tile (measured: a 64-row tile of 256 takes 0.65
// of a full one), except for a 320-row in-projection tile that is its expert's only one: no
// other m-tile shares its weight tiles through the L2, and it counts 160/256 (fitted to the
// XCDs' finishing times on the skewed layer, where such tiles of 64 rows took 0.69 of a full one
// and the two XCDs holding them finished 15% after the rest with the half-tile estimate).
template <int MODE, int TM, int WGM>
__device__ __forceinline__ int tile_cost(int rows_in_tile, bool alone) {
    const int fix = (MODE != MODE_OUT && TM >= 5 && alone) ? 160 : 128;
    return fix + (256 - fix) * variant_nv<TM, WGM>((rows_in_tile + 31) / 32) / TM;
}

template <int MODE, int BM, int TM, int WGM>
__device__ __forceinline__ void build_segments(const FfnKArgs& a, int lane, int* s_tab, int* s_R1, int* s_C1) {
    int tl[5], beg[5], rows[5], cost[5], loc = 0, cloc = 0;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        const int s = lane * 5 + q;
        beg[q] = 0;
        rows[q] = 0;
        if (s < a.N) {
            beg[q] = a.offsets[s];
            rows[q] = a.offsets[s + 1] - beg[q];
            if (rows[q] <= a.small_rows) rows[q] = 0;      // (small_rows 0: none left out)
        } else if (s == a.N && a.has_shared) {
            beg[q] = a.T * a.k;
            rows[q] = a.T;
        }
        tl[q] = (rows[q] + BM - 1) / BM;
        const int part = rows[q] % BM;
        cost[q] = a.n_tiles * ((rows[q] / BM) * 256 + (part ? tile_cost<MODE, TM, WGM>(part, rows[q] < BM) : 0));
        loc += tl[q];
        cloc += cost[q];
    }
    int incl = loc, cincl = cloc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        const int w = __shfl_up(cincl, o, 64);
        if (lane >= o) {
            incl += v;
            cincl += w;
        }
    }
    int run = incl - loc, crun = cincl - cloc;
#pragma unroll
    for (int q = 0; q < 5; ++q) {
        const int s = lane * 5 + q;
        s_tab[s] = run * a.n_tiles;
        s_tab[FFN_MAX_SEG + s] = tl[q];
        s_tab[2 * FFN_MAX_SEG + s] = beg[q];
        s_tab[3 * FFN_MAX_SEG + s] = beg[q] + rows[q];
        s_tab[4 * FFN_MAX_SEG + s] = crun;
        run += tl[q];
        crun += cost[q];
    }
    if (lane == 63) {
        *s_R1 = incl * a.n_tiles;
        *s_C1 = cincl;
    }
}

// The XCDs' shares of the tile numbering, split by estimated cost rather than by count (an
// XCD whose share holds no short tiles would otherwise finish last): lane x of wave 0 finds
// where cost x/8 of the whole starts, as the segment holding it and the tile at that fraction
// of the segment's cost.
__device__ __forceinline__ void xcd_bounds(const FfnKArgs& a, const int* s_tab, int R1, int C1, int lane, int* s_bound) {
    if (lane > 8) return;
    const int R = R1 * a.ksplit;
    if (lane == 8 || C1 == 0) {
        s_bound[lane] = lane == 8 ? R : 0;
        return;
    }
    const long long b = (long long)C1 * a.ksplit * lane / 8;
    const int kp = (int)(b / C1);
    const int rem = (int)(b - (long long)kp * C1);
    int lo = 0, hi = a.N + (a.has_shared ? 1 : 0) - 1;
    while (lo < hi) {                                  // last segment whose cost starts <= rem
        const int mid = (lo + hi + 1) >> 1;
        if (s_tab[4 * FFN_MAX_SEG + mid] <= rem) lo = mid;
        else hi = mid - 1;
    }
    const int tiles = s_tab[FFN_MAX_SEG + lo] * a.n_tiles;
    // (segments past the last one have zero cost, so lo + 1 always has a cost start)
    const int seg_c = s_tab[4 * FFN_MAX_SEG + lo + 1] - s_tab[4 * FFN_MAX_SEG + lo];
    int off = seg_c > 0 ? (int)((long long)(rem - s_tab[4 * FFN_MAX_SEG + lo]) * tiles / seg_c) : 0;
    off = off < tiles ? off : tiles;
    const int t = kp * R1 + s_tab[lo] + off;
    s_bound[lane] = t < R ? t : R;
}

// Two floats rounded to bf16 (nearest even, as a bf16 conversion) in one 32-bit word, the
// first in the low half.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// A pointer every lane holds the same value of, kept in scalar registers (a buffer descriptor
// must be uniform).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    const unsigned long long v = (unsigned long long)p;
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    return (const char*)(((unsigned long long)hi << 32) | lo);
}

struct TileInfo {
    int seg, mt, nt, kpart, row_beg, row_end;
};

// Tile t (0 <= t < R1 * ksplit) -> segment, m-tile, n-tile and K part, one tile per lane.  The
// segment is found by a binary search for the last one whose first tile is <= t (an empty
// segment starts where the next one does, so the last of equal starts is the one holding t).
__device__ __forceinline__ TileInfo decode_lane(const FfnKArgs& a, const int* s_tab, int R1, int t) {
    TileInfo ti;
    ti.kpart = t / R1;
    const int tt = t - ti.kpart * R1;
    int lo = 0, hi = a.N + (a.has_shared ? 1 : 0) - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tab[mid] <= tt) lo = mid;
        else hi = mid - 1;
    }
    ti.seg = lo;
    const int tm = s_tab[FFN_MAX_SEG + lo];
    const int rem = tt - s_tab[lo];
    const int GM = tm < 8 ? tm : 8;
    const int GN = 32 / GM;
    const int mg = rem / (GM * a.n_tiles);
    const int gm = min(GM, tm - mg * GM);
    const int r2 = rem - mg * GM * a.n_tiles;
    const int band = r2 / (gm * GN);
    const int r3 = r2 - band * gm * GN;
    ti.mt = mg * GM + r3 % gm;
    ti.nt = band * GN + r3 / gm;
    ti.row_beg = s_tab[2 * FFN_MAX_SEG + lo];
    ti.row_end = s_tab[3 * FFN_MAX_SEG + lo];
    return ti;
}

// The tile table of one tiled GEMM launch, in the numbering its blocks claim tiles by: entry t =
// {segment | K part << 16, m-tile, n-tile, 0}.  One wave per block, each with
// a segment table of its own; block 0 also clears the launch's eight claim counters.  The GEMM
// then turns a claimed tile number into a tile with one load, issued a stage before it is used,
// instead of a search and a chain of divisions inside a stage.
template <int MODE, int BM, int BNH, int WGM, int WGN>
__global__ __launch_bounds__(64) void ffn_tile_table(FfnKArgs a) {
    constexpr int TM = FfnTile<MODE, BM, BNH, WGM, WGN>::TM;
    __shared__ int s_tab[5 * FFN_MAX_SEG];
    __shared__ int s_R1, s_C1;
    const int lane = threadIdx.x;
    if (blockIdx.x == 0 && lane < 8) a.ctr[lane] = 0u;
    build_segments<MODE, BM, TM, WGM>(a, lane, s_tab, &s_R1, &s_C1);
    __syncthreads();
    const int R1 = s_R1, R = R1 * a.ksplit;
    for (int t = blockIdx.x * 64 + lane; t < R; t += gridDim.x * 64) {
        const TileInfo ti = decode_lane(a, s_tab, R1, t);
        tile_table(a)[t] = make_int4(ti.seg | (ti.kpart << 16), ti.mt, ti.nt, 0);
    }
}

// Which tiled GEMMs claim their tiles: the out-projection with 256- and 320-row tiles.  Measured
// on one box (down projection, ms, dealt -> claimed): Mixtral 0.949 -> 0.924, DeepSeek-V3 2.615
// -> 2.53, shared + top-7 of 256 2.43 -> 2.40, top-1 of 16 0.651 -> 0.638, skewed 0.83 -> 0.82;
// but top-1 of 128 (32 rows per expert, 128-row tiles, a weight stream) 2.53 -> 2.59.  The
// gate/up projection claiming its tiles was no faster, and its larger register footprint put
// spill reloads into its main loops.
constexpr bool claims_tiles(int mode, int bm) { return mode == MODE_OUT && bm >= 256; }
template <int MODE, int BM, int BNH, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_bf16_kernel(FfnKArgs a) {
    using Cfg = FfnTile<MODE, BM, BNH, WGM, WGN>;
    constexpr int NB = Cfg::NB, TM = Cfg::TM, TN = Cfg::TN;
    constexpr int NW = WGM * WGN;
    constexpr int ROWS = BM + Cfg::BROWS;            // rows of one stage (A rows, then B rows)
    constexpr int A_INS = BM / (8 * NW);             // load instructions per wave per stage (A)
    constexpr int B_INS = Cfg::BROWS / (8 * NW);     // (B)
    static_assert(BM % (8 * NW) == 0 && Cfg::BROWS % (8 * NW) == 0, "load split");
    // Weight tiles are stored K-major, as the weights are: per matrix 64 k-rows of BNH columns
    constexpr int BROWB = 2 * BNH;                   // bytes of one k-row of a weight tile
    constexpr int BMATB = 64 * BROWB;                // bytes of one matrix's tile per stage
    static_assert(BMATB % (1024 * NW) == 0, "every B load instruction stays inside one matrix");
    static_assert(BM <= 64 * NW, "one thread per row of the A tile");
    // two stages in two distinct LDS objects, so the compiler can tell a fragment read of one
    // stage from the asynchronous loads into the other
    __shared__ __attribute__((aligned(1024))) bf16 st0[ROWS * 64];
    __shared__ __attribute__((aligned(1024))) bf16 st1[ROWS * 64];
    __shared__ int s_tab[5 * FFN_MAX_SEG];
    __shared__ int s_R1, s_C1;
    __shared__ int s_bound[9];                                 // the XCDs' shares of the tiles
    __shared__ int s_tiles[64 * 6];                            // dealt tiles, or the ring of claimed ones
    __shared__ int s_src[MODE == MODE_OUT ? 1 : BM];          // next tile's x row of each A row
    __shared__ float s_scale[MODE == MODE_OUT ? 2 * BM : 1];  // gate weight of each row, 2 tiles

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases go to M0
    static_assert(FFN_MAX_SEG > MOE_MAX_EXPERTS + 1, "a zero-cost entry follows the last segment");
    if (wave == 0) build_segments<MODE, BM, TM, WGM>(a, lane, s_tab, &s_R1, &s_C1);
    __syncthreads();
    if (wave == 0) xcd_bounds(a, s_tab, s_R1, s_C1, lane, s_bound);
    __syncthreads();
    const int R1 = __builtin_amdgcn_readfirstlane(s_R1);
    const int xcd = blockIdx.x & 7;
    int it = 0;                                          // tiles done by this block
    // A block's tiles are claimed (DYN) or dealt.  Dealt: round i of the XCD's range goes to its
    // blocks in order, reversed on odd rounds, and wave 0 decodes the block's tiles 64 at a time,
    // one per lane, into s_tiles.  Claimed, by wave 0: the XCD's own range first, then the others
    // in turn, each by an add on the range's counter; a claimed tile's entry comes from the tile
    // table into a ring of four slots.  `first` is the result of an add already issued on this
    // XCD's counter (~0u: none).  A counter past its range's end stays so (claims only add), so a
    // range found used up is not asked again.
    constexpr bool DYN = claims_tiles(MODE, BM);
    const int lo = __builtin_amdgcn_readfirstlane(s_bound[xcd]), hi = __builtin_amdgcn_readfirstlane(s_bound[xcd + 1]);
    const int nbx = gridDim.x >> 3, jb = blockIdx.x >> 3;
    auto tile_id = [&](int i) { return lo + i * nbx + ((i & 1) ? nbx - 1 - jb : jb); };
    auto decode_chunk = [&](int c) {                     // wave 0, dealt tiles 64c .. 64c + 63
        const int t = tile_id(c * 64 + lane);
        if (t < hi) {
            const TileInfo ti = decode_lane(a, s_tab, R1, t);
            int* p = s_tiles + lane * 6;
            p[0] = ti.seg; p[1] = ti.mt; p[2] = ti.nt; p[3] = ti.kpart; p[4] = ti.row_beg; p[5] = ti.row_end;
        }
    };
    unsigned int spent = 0;                              // ranges found used up
    auto claim = [&](unsigned int first) -> int {
#pragma unroll 1
        for (int v = 0; v < 8; ++v) {
            const int x = (xcd + v) & 7;
            if (spent & (1u << x)) continue;
            unsigned int c = first;
            if (v != 0 || first == ~0u) {
                if (lane == 0) c = atomicAdd(a.ctr + x, 1u);
                c = __builtin_amdgcn_readfirstlane(c);
            }
            const int t = s_bound[x] + (int)c;
            if (t < s_bound[x + 1]) return t;
            spent |= 1u << x;
        }
        return -1;
    };
    // Ring slot i & 3 (claimed tiles): the table entry of the block's tile i (word w from lane w
    // of wave 0) and whether one was found (tile number t >= 0).
    auto fetch = [&](int t) -> int {                     // wave 0: this lane's word of entry t
        return (t >= 0 && lane < 4) ? ((const int*)tile_table(a))[4 * t + lane] : 0;
    };
    auto put = [&](int i, int t, int e) {                // wave 0
        int* p = s_tiles + (i & 3) * 5;
        if (lane < 4) p[lane] = e;
        if (lane == 4) p[4] = t >= 0 ? 1 : 0;
    };
    auto found = [&](int i) { return __builtin_amdgcn_readfirstlane(s_tiles[(i & 3) * 5 + 4]) != 0; };
    auto read_tile = [&](int i) {
        TileInfo ti;
        if constexpr (DYN) {
            const int* p = s_tiles + (i & 3) * 5;
            const int w0 = __builtin_amdgcn_readfirstlane(p[0]);
            ti.seg = w0 & 0xffff;
            ti.kpart = w0 >> 16;
            ti.mt = __builtin_amdgcn_readfirstlane(p[1]);
            ti.nt = __builtin_amdgcn_readfirstlane(p[2]);
            ti.row_beg = __builtin_amdgcn_readfirstlane(s_tab[2 * FFN_MAX_SEG + ti.seg]);
            ti.row_end = __builtin_amdgcn_readfirstlane(s_tab[3 * FFN_MAX_SEG + ti.seg]);
        } else {
            const int* p = s_tiles + (i & 63) * 6;
            ti.seg = __builtin_amdgcn_readfirstlane(p[0]);
            ti.mt = __builtin_amdgcn_readfirstlane(p[1]);
            ti.nt = __builtin_amdgcn_readfirstlane(p[2]);
            ti.kpart = __builtin_amdgcn_readfirstlane(p[3]);
            ti.row_beg = __builtin_amdgcn_readfirstlane(p[4]);
            ti.row_end = __builtin_amdgcn_readfirstlane(p[5]);
        }
        return ti;
    };
    if constexpr (DYN) {
        if (wave == 0) {
            const int t0 = claim(~0u);
            put(0, t0, fetch(t0));
            const int t1 = claim(~0u);
            put(1, t1, fetch(t1));
        }
        __syncthreads();
        if (!found(0)) return;                           // every range used up already
    } else {
        if (tile_id(0) >= hi) return;
        if (wave == 0) decode_chunk(0);
        __syncthreads();
    }
    TileInfo cur = read_tile(0);
    // Tile it + 2 of the block: claimed with an add issued at the start of tile it, its table
    // entry loaded after the tile's first stage and put in its slot after the second (whose
    // wait for its own loads covers it).  The stages that follow end in barriers, so the slot
    // is visible when tile it + 1 starts; it was last read when tile it - 2 started.
    unsigned int pend = ~0u;
    bool claim_next = false;
    auto fetch_next = [&](int& t, int& e) {
        t = -1;
        e = 0;
        if (DYN && claim_next && wave == 0) {
            t = claim(pend);
            e = fetch(t);
        }
    };
    auto put_next = [&](int t, int e) {
        if (DYN && claim_next && wave == 0) put(it + 2, t, e);
    };

    const int KT = a.K / FB_BK / a.ksplit;               // stages of one tile
    // A tile's last two stages load the next tile's first stage (and half of its second) into
    // the LDS slots they free, when the next tile starts in slot 0 (an even stage count).
    const bool chain = (KT % 2 == 0) && KT >= 4;
    const size_t wstride = (size_t)a.Ncols * a.K;
    // Base of the A loads: x for the in-projection, whose gathered rows may sit anywhere in it;
    // the tile's first row of H for the out-projection, whose rows are contiguous per tile, so
    // that H may exceed the 4 GiB of a 32-bit offset.
    auto base_a = [&](const TileInfo& ti) -> const char* {
        if (MODE != MODE_OUT) return (const char*)a.A;
        return uniform_ptr((const char*)(a.A + (size_t)(ti.row_beg + ti.mt * BM) * a.K));
    };
    const char* baseA = base_a(cur);

    // per-lane 32-bit byte offsets of this wave's load instructions from a uniform base
    // (x stays below 4 GiB, which the host checks; one tile of H and one expert's weight
    // matrix do too)
    // Lane-derived values are recomputed where a tile's offsets are set (an empty asm hides the
    // lane id from the optimiser there), instead of being precomputed once per row group and
    // held in registers for the whole kernel.
    auto fresh_lane = [&]() {
        int l = lane;
        asm volatile("" : "+v"(l));
        return l;
    };
    // element offset of the chunk lane fetches for LDS row group g (8 rows): ((lane & 7) ^
    // ((4g + (lane >> 4)) & 7)) * 8.  Every group this wave loads (A: g = wave + NW*i, B: g =
    // BM/8 + wave + NW*i) has 4g = 4*wave (mod 8), so one value serves all of its loads.
    static_assert((4 * NW) % 8 == 0 && (4 * (BM / 8)) % 8 == 0, "one chunk offset per lane");
    auto a_row = [&](const TileInfo& ti, int i, int l) {  // row of A load i (rows past the end: row 0)
        const int m0 = ti.row_beg + ti.mt * BM, rl = 8 * (wave + NW * i) + (l >> 3);
        return (m0 + rl < ti.row_end) ? m0 + rl : m0;
    };
    // in-projection: x row of slot row r; out-projection: r's place in its tile
    auto a_src = [&](const TileInfo& ti, int r) {
        if (MODE == MODE_OUT) return r - (ti.row_beg + ti.mt * BM);
        return (ti.seg < a.N) ? a.perm[r] / a.k : r - a.T * a.k;
    };
    uint32_t offA[A_INS], offB[B_INS];
    const char *baseB0, *baseB1;
    // B load instruction i of this wave fills bytes 1024 (wave + NW i) .. +1023 of the B region:
    // lane l the 16 bytes at 1024 (wave + NW i) + 16 l, i.e. k-row kr and chunk position p of one
    // matrix's tile.  Position p of k-row kr holds the weight chunk (8 columns) p ^ 4 (kr & 3), so
    // that a transposed fragment read (4 k-rows x 32 bytes per 16 lanes) finds the four rows in
    // four different quarters of the banks.  Columns past the matrix (a partial last n-tile) load
    // the tile's first chunk instead; their outputs are never stored.  The per-lane offset is
    // (kr * Ncols + column) * 2 bytes from the expert's matrix (a matrix stays below 4 GiB, which
    // the host checks); the stage's first k-row goes in the scalar offset.
    auto set_b = [&](const TileInfo& ti) {
        const int n0 = ti.nt * BNH;
        const int l = fresh_lane();
#pragma unroll
        for (int i = 0; i < B_INS; ++i) {
            const int qm = (1024 * (wave + NW * i) + 16 * l) % BMATB;
            const int kr = qm / BROWB, pos = (qm % BROWB) >> 4;
            const int n = n0 + 8 * (pos ^ (4 * (kr & 3)));
            const int nc = n < a.Ncols ? n : n0;
            offB[i] = ((uint32_t)kr * (uint32_t)a.Ncols + (uint32_t)nc) * 2u;
        }
        const bf16* B0 = (ti.seg < a.N) ? a.B0 + ti.seg * wstride : a.S0;
        const bf16* B1 = (NB == 2) ? ((ti.seg < a.N) ? a.B1 + ti.seg * wstride : a.S1) : B0;
        baseB0 = uniform_ptr((const char*)B0);
        baseB1 = uniform_ptr((const char*)B1);
    };
    auto set_a_direct = [&](const TileInfo& ti) {
        const int l = fresh_lane();
        const uint32_t lc = (uint32_t)(((l & 7) ^ ((4 * wave + (l >> 4)) & 7)) * 8);
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            offA[i] = ((uint32_t)a_src(ti, a_row(ti, i, l)) * (uint32_t)a.K + lc) * 2u;
        baseA = base_a(ti);
    };
    auto scale_of = [&](const TileInfo& ti) {            // gate weight of this thread's row
        const int r = ti.row_beg + ti.mt * BM + tid;
        return (tid < BM && r < ti.row_end && a.row_scale && ti.seg < a.N) ? a.row_scale[a.perm[r]] : 1.0f;
    };

    const int wm = wave / WGN, wn = wave % WGN;
    // fragment addresses: rows of one wave's fragments differ by multiples of 32, so their
    // swizzle only depends on the lane: row r, chunk c sits at r*64 + ((c ^ ((r >> 1) & 7)) << 3)
    const int fr = lane & 31, fh = lane >> 5, l7 = (fr >> 1) & 7;
    const int abase = (wm * 32 + fr) * 64;              // sub-tile i of this wave: i * WGM + wm
    // Weight fragment (32 columns x 16 k, lane l: column l & 31, k 8 (l >> 5) .. +7) from the
    // K-major tile by two transposed reads: in each 16-lane group g = l >> 4, lane L = l & 15
    // addresses k-row 8 (g >> 1) + (L >> 2) (+4 for the second read) at column
    // 16 (g & 1) + 4 (L & 3) of the fragment's block, and receives column 16 (g & 1) + L of the
    // four rows.  Bytes from the stage's B region: (16 kk + 4 half) BROWB + brow + bcol[j].
    // this lane's weight-fragment byte offset within a k-step of matrix 0, per 32-column block:
    // one register each (so that a read's address is the stage array, one lane offset and
    // constants, which lets the compiler keep track of the LDS array it reads)
    int boff[TN];
    {
        const int gq = lane >> 4, lq = lane & 15;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int ncol = wn * Cfg::WTN + j * 32 + 16 * (gq & 1) + 4 * (lq & 3);
            boff[j] = (8 * (gq >> 1) + (lq >> 2)) * BROWB + (((ncol >> 3) ^ (4 * (lq >> 2))) << 4) +
                      ((ncol & 7) << 1);
        }
    }
    struct Frags { bf16x8 a[TM]; bf16x8 b[NB][TN]; };
    auto load_frags = [&](const bf16* st, int kk, Frags& f, auto nv) {
        const int xo = ((2 * kk + fh) ^ l7) << 3;
#pragma unroll
        for (int i = 0; i < decltype(nv)::value; ++i)
            f.a[i] = *(const bf16x8*)(st + abase + i * WGM * 32 * 64 + xo);
        // lane-derived parts recomputed here (a few integer operations) rather than held in
        // registers through the whole kernel
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int m = 0; m < NB; ++m)
                f.b[m][j] = lds_read_tr_b16x8(st, BM * 128 + 16 * kk * BROWB + m * BMATB + boff[j], 4 * BROWB);
    };
    // The weight fragment is the MFMA's first operand and the row fragment its second, so each
    // accumulator holds the transposed 32x32 block: lane l has tile row (l & 31), register r
    // has output column 8*(r >> 2) + 4*(l >> 5) + (r & 3) -- four adjacent columns per lane and
    // register group, stored with one vector store.  The first K step of a tile starts from zero
    // instead of from the accumulators (no separate clearing).
    typedef f32x16 Acc[NB][TM][TN];
    auto mfmas = [&](Acc& acc, const Frags& f, auto nv, auto first) {
        const f32x16 zero = {};
#pragma unroll
        for (int m = 0; m < NB; ++m)
#pragma unroll
            for (int i = 0; i < decltype(nv)::value; ++i) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[m][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        f.b[m][j], f.a[i], decltype(first)::value ? zero : acc[m][i][j], 0, 0, 0);
            }
    };
    const std::integral_constant<bool, true> first_step{};
    const std::integral_constant<bool, false> later_step{};
    constexpr int NLD = A_INS + B_INS;           // direct-to-LDS loads per stage
    // the first part of a stage's loads goes out during step 3 of the stage before, the rest
    // during step 0; the first part holds A rows only, so that a tile's last two stages can
    // switch the A offsets to the next tile before the B offsets
    constexpr int NLD0 = (NLD + 1) / 2 < A_INS ? (NLD + 1) / 2 : A_INS;
    static_assert(NLD0 == A_INS, "the second part of a stage's loads holds B rows only");
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
    // Loads of stage kidx of the current tile; kidx >= KT means stage kidx - KT of the next tile
    // (the offsets and weight bases have been switched to it by then; without a chain these are
    // in-bounds loads of the current tile into the idle slot, never used).  A variant with NV
    // sub-tiles per wave reads rows [0, NV * WGM * 32) of its own A tile only, so its loads skip
    // the rest; the next tile's loads take every row.
    int kbase_c = cur.kpart * KT * FB_BK, kbase_n = kbase_c;
    auto issue_part = [&](bf16* st, int kidx, int beg, int end, auto nv) {
        constexpr int A_NEED = decltype(nv)::value * WGM * 32 / (8 * NW);
        const bool nxs = kidx >= KT;
        const int k0 = nxs ? kbase_n + (chain ? (kidx - KT) * FB_BK : 0) : kbase_c + kidx * FB_BK;
        const int a_need = nxs ? A_INS : A_NEED;
#pragma unroll
        for (int q = 0; q < NLD; ++q) {
            if (q < beg || q >= end) continue;
            if (q < A_INS) {
                if (q >= a_need) continue;
                buffer_load_lds16(baseA, (lds_void_t*)(st + (8 * (wave + NW * q)) * 64), offA[q], 2 * k0);
            } else {
                const int i = q - A_INS;
                const bool second = NB == 2 && (1024 * NW * i) / BMATB == 1;   // the up matrix
                const char* bb = uniform_ptr(second ? baseB1 : baseB0);
                buffer_load_lds16(bb, (lds_void_t*)((char*)st + BM * 128 + 1024 * (wave + NW * i)), offB[i],
                                  2 * k0 * a.Ncols);
            }
        }
    };
    // One stage (K = 64 in four K=16 steps).  On entry f0 holds step 0's fragments and the
    // first half of the next stage's loads is in flight.  The second half goes out during step 0;
    // the barrier sits before step 3, so the next stage's first fragments are read while step 3's
    // MFMAs run, and step 3 already sends the first half of the stage after next into the slot
    // this stage has just released.
    auto stage = [&](Acc& acc, bf16* cur_st, bf16* nxt_st, int k_next, int k_after, Frags& f0, Frags& f1, auto nv,
                     auto first) {
        constexpr int NDS = decltype(nv)::value + 2 * NB * TN;   // fragment reads per K=16 step
        load_frags(cur_st, 1, f1, nv);
        issue_part(nxt_st, k_next, NLD0, NLD, nv);
        mfmas(acc, f0, nv, first);
        interleave(NDS, NLD - NLD0, nv);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur_st, 2, f0, nv);
        mfmas(acc, f1, nv, later_step);
        interleave(NDS, 0, nv);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur_st, 3, f1, nv);
        mfmas(acc, f0, nv, later_step);
        interleave(NDS, 0, nv);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070);    // vmcnt(0) lgkmcnt(0): own loads and reads done
        __syncthreads();                       // next stage visible; this stage no longer read
        load_frags(nxt_st, 0, f0, nv);
        issue_part(cur_st, k_after, 0, NLD0, nv);
        mfmas(acc, f1, nv, later_step);
        interleave(NDS, NLD0, nv);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The next tile's A sources (in-projection: x rows through perm) and row scales
    // (out-projection: gate weights through perm) are loaded at the start of a tile and put in
    // place after its first stage, so no load latency is waited for at a tile boundary.
    TileInfo nx = cur;
    int praw = 0;
    float sc_next = 1.0f;
    auto prefetch_next = [&]() {
        const int r = nx.row_beg + nx.mt * BM + tid;
        if (MODE == MODE_OUT) {
            praw = (tid < BM && r < nx.row_end && a.row_scale && nx.seg < a.N) ? a.perm[r] : -1;
        } else if (tid < BM) {
            const int rc = r < nx.row_end ? r : nx.row_beg + nx.mt * BM;
            praw = (nx.seg < a.N) ? a.perm[rc] : rc;
        }
    };
    auto after_first_stage = [&]() {
        if (MODE == MODE_OUT) sc_next = praw >= 0 ? a.row_scale[praw] : 1.0f;
        else if (tid < BM) s_src[tid] = (nx.seg < a.N) ? praw / a.k : praw - a.T * a.k;
    };
    auto switch_a = [&]() {                              // A offsets of the next tile
        const int l = fresh_lane();
        const uint32_t lc = (uint32_t)(((l & 7) ^ ((4 * wave + (l >> 4)) & 7)) * 8);
#pragma unroll
        for (int i = 0; i < A_INS; ++i) {
            const int src = (MODE == MODE_OUT) ? a_src(nx, a_row(nx, i, l)) : s_src[8 * (wave + NW * i) + (l >> 3)];
            offA[i] = ((uint32_t)src * (uint32_t)a.K + lc) * 2u;
        }
        baseA = base_a(nx);
    };

    // Epilogue (transposed accumulator layout, see mfmas): per sub-tile one row per lane and
    // four groups of four adjacent columns, each written with one 8-byte (bf16) or 16-byte
    // (fp32) store.  Ncols is a multiple of 64, so a group is either inside or past the end.
    auto store = [&](const Acc& acc, auto nv) {
        const int m0 = cur.row_beg + cur.mt * BM, n0 = cur.nt * BNH;
        const float* scl = s_scale + (MODE == MODE_OUT ? (it & 1) * BM : 0);
        const bool row_b16 = MODE == MODE_OUT && a.routed_bf16 && cur.seg < a.N;   // uniform
        // computed here, not hoisted above the K loop where they would hold registers
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int c0 = n0 + wn * Cfg::WTN;             // this wave's first column
#pragma unroll
        for (int i = 0; i < decltype(nv)::value; ++i) {
            const int rl = (i * WGM + wm) * 32 + (ln & 31);
            const int row = m0 + rl;
            if (row >= cur.row_end) continue;
            const float scale = (MODE == MODE_OUT) ? scl[rl] : 1.0f;
            // this lane's row at its first group of four columns; the groups follow at constant
            // offsets (immediate offsets of the stores)
            const size_t base = (size_t)row * a.Ncols + c0 + 4 * (ln >> 5);
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (c0 + j * 32 >= a.Ncols) continue;   // whole 32-column blocks (Ncols % 64 == 0)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = acc[0][i][j][4 * g + e];
                        if (MODE == MODE_IN_SWIGLU) v[e] = silu_f32(x) * acc[NB - 1][i][j][4 * g + e];
                        else if (MODE == MODE_IN_RELU) v[e] = fmaxf(x, 0.f);
                        else v[e] = x * scale;
                    }
                    if (MODE == MODE_OUT && !row_b16) {
                        float4 o = {v[0], v[1], v[2], v[3]};
                        *(float4*)((float*)a.C + cur.kpart * a.part_stride + base + j * 32 + 8 * g) = o;
                    } else {
                        uint2 o;
                        o.x = pack_bf16x2(v[0], v[1]);
                        o.y = pack_bf16x2(v[2], v[3]);
                        *(uint2*)((bf16*)a.C + base + j * 32 + 8 * g) = o;
                    }
                }
                // one 32x32 block at a time keeps the epilogue's registers few
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // One tile.  The tile's 32-row sub-tiles are dealt to the wave rows in turn (sub-tile s to
    // wave row s % WGM), so the rows of a short tile (an expert's last one) spread over all
    // waves; a tile whose valid sub-tiles fit in NV per wave runs the variant with NV sub-tiles
    // per wave and skips the MFMAs and fragment reads of the rest (rows past the end were loaded
    // as copies of the first row and are never stored).  Each variant owns its accumulators and
    // epilogue, so no accumulator is live across the choice of variant.  On entry the tile's
    // first stage and half of its second are loaded or in flight.
    auto run = [&](auto nv) {
        Acc acc;
        Frags fa, fb;
        __builtin_amdgcn_s_waitcnt(0x0070);
        __syncthreads();
        if (chain) prefetch_next();
        load_frags(st0, 0, fa, nv);
        if (chain) {
            stage(acc, st0, st1, 1, 2, fa, fb, nv, first_step);
            after_first_stage();
            int tn, en;
            fetch_next(tn, en);
            stage(acc, st1, st0, 2, 3, fa, fb, nv, later_step);
            put_next(tn, en);
            for (int kt = 2; kt + 4 <= KT; kt += 2) {
                stage(acc, st0, st1, kt + 1, kt + 2, fa, fb, nv, later_step);
                stage(acc, st1, st0, kt + 2, kt + 3, fa, fb, nv, later_step);
            }
            // the last two stages send out the next tile's first stage and half of its second
            switch_a();
            stage(acc, st0, st1, KT - 1, KT, fa, fb, nv, later_step);
            set_b(nx);
            stage(acc, st1, st0, KT, KT + 1, fa, fb, nv, later_step);
        } else {
#pragma unroll
            for (int m = 0; m < NB; ++m)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int r = 0; r < 16; ++r) acc[m][i][j][r] = 0.f;
            // (no chain: the next tile starts after a barrier, which makes the slot visible)
            int tn, en;
            fetch_next(tn, en);
            put_next(tn, en);
            int kt = 0;
            for (; kt + 2 <= KT; kt += 2) {
                stage(acc, st0, st1, kt + 1, kt + 2, fa, fb, nv, later_step);
                stage(acc, st1, st0, kt + 2, kt + 3, fa, fb, nv, later_step);
            }
            if (kt < KT) stage(acc, st0, st1, KT, KT + 1, fa, fb, nv, later_step);
        }
        store(acc, nv);
        // the next tile's offsets again (cheap), so that none is held through the epilogue
        if (chain) {
            switch_a();
            set_b(nx);
        }
    };
    auto run_tile = [&]() {
        const int nv = variant_nv<TM, WGM>((cur.row_end - (cur.row_beg + cur.mt * BM) + 31) / 32);
        if (TM >= 2 && nv == 1) run(std::integral_constant<int, 1>{});
        else if (TM >= 4 && nv == 2) run(std::integral_constant<int, 2>{});
        else if (TM >= 5 && nv == 4) run(std::integral_constant<int, (TM >= 5 ? 4 : TM)>{});
        else run(std::integral_constant<int, TM>{});
    };

    // first tile: everything loaded here
    set_a_direct(cur);
    set_b(cur);
    if (MODE == MODE_OUT && tid < BM) s_scale[tid] = scale_of(cur);
    issue_part(st0, 0, 0, NLD, std::integral_constant<int, TM>{});
    issue_part(st1, 1, 0, NLD0, std::integral_constant<int, TM>{});
    for (;;) {
        bool has_next;
        if constexpr (DYN) {
            has_next = found(it + 1);
            // without a next tile every range is used up: no claim (it could only fail)
            claim_next = has_next;
            pend = ~0u;
            if (has_next && wave == 0 && !(spent & (1u << xcd))) {
                if (lane == 0) pend = atomicAdd(a.ctr + xcd, 1u);
                pend = __builtin_amdgcn_readfirstlane(pend);
            }
        } else {
            has_next = tile_id(it + 1) < hi;
            if (has_next && ((it + 1) & 63) == 0) {
                // every wave has taken its tiles of the previous 64 from s_tiles (one tile back)
                if (wave == 0) decode_chunk((it + 1) >> 6);
                __syncthreads();
            }
        }
        nx = has_next ? read_tile(it + 1) : cur;
        kbase_n = nx.kpart * KT * FB_BK;
        run_tile();
        if (!has_next) break;
        if (!chain) {
            // no chain: the next tile's first loads go out after every wave is done with this one
            __builtin_amdgcn_s_waitcnt(0x0070);
            __syncthreads();
            set_a_direct(nx);
            set_b(nx);
            sc_next = (MODE == MODE_OUT) ? scale_of(nx) : 1.0f;
            kbase_c = kbase_n;
            issue_part(st0, 0, 0, NLD, std::integral_constant<int, TM>{});
            issue_part(st1, 1, 0, NLD0, std::integral_constant<int, TM>{});
        }
        // the next tile's epilogue comes after at least one more barrier
        if (MODE == MODE_OUT && tid < BM) s_scale[((it + 1) & 1) * BM + tid] = sc_next;
        cur = nx;
        kbase_c = kbase_n;
        ++it;
    }
    __builtin_amdgcn_s_waitcnt(0x0070);    // no load may still be writing LDS at exit
}

// ------------------------------------------------------------------ skinny path (decode)
// For a few rows per expert the GEMMs are weight streams: every weight byte of a touched expert
// is read once and used for at most 16 rows.  One wave owns CG 16-column groups of one segment
// and the whole K range.  Per K step of 32, its weight block (32 k-rows x 16 CG columns, K-major
// as stored) comes from memory into registers U steps ahead, 16 bytes per lane (so the wave reads
// whole 32 CG-byte segments of k-rows), is written to a small LDS tile of the wave's own and read
// back as v_mfma_f32_16x16x32_bf16 B fragments (lane: column lane & 15, k 8 (lane >> 4) .. +7) by
// transposed reads.  The A fragments (the <= 16 rows, gathered through perm for the
// in-projection) serve all CG groups and are shared by all waves through L2.  Waves are numbered
// segment, then column group, so the waves of a block stream neighbouring weight columns.
// Empty experts are skipped, so only touched experts' weights are read.  Segments with more than
// 16 rows loop over 16-row tiles.
//
// The wave's LDS tile holds 32 k-rows of 32 CG bytes.  A transposed read takes rows 8g .. 8g+3
// (+4) of one 16-column block in lane group g = lane >> 4, and groups 0-1 (and 2-3) share an LDS
// cycle.  So that the 8 rows of a cycle fall in distinct banks: with CG = 1 the blocks of 8 rows
// (256 bytes) start 384 bytes apart (rows of blocks 1 and 3 in banks 32-63, of blocks 0 and 2 in
// banks 0-31); with CG = 2 the 16-byte chunks of rows 8-15 and 24-31 are swapped in pairs (chunk
// c at c ^ 2); with CG = 4 chunk c of row r sits at c ^ 2 (((r >> 1) & 1) | ((r >> 3) & 1) << 1).
// Steps alternate between two tiles; a wave's LDS operations are performed in order, so a step's
// writes into a tile follow the reads of the step two before.
template <int CG>
struct SkinnyTile {
    static constexpr int ROWB = 32 * CG;                         // bytes of one k-row
    static constexpr int BYTES = CG == 1 ? 3 * 384 + 256 : 32 * ROWB;
    static constexpr int CPR = ROWB / 16;                        // 16-byte chunks per k-row
    static constexpr int RPI = 64 / CPR;                         // k-rows per wave load
    static_assert(CG == 1 || CG == 2 || CG == 4, "tile layouts for 1, 2 or 4 16-column groups");
    __device__ static int off(int r, int c) {
        if (CG == 1) return (r >> 3) * 384 + (r & 7) * ROWB + c * 16;
        if (CG == 2) return r * ROWB + ((c ^ (2 * ((r >> 3) & 1))) << 4);
        return r * ROWB + ((c ^ (2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)))) << 4);
    }
};

// Weight loads are non-temporal when a wave's k-row piece is a whole 128-byte line (four
// 16-column groups): each weight byte is read once per call, and both streams of the Mixtral
// decode layer then run at 6.7 TB/s (gate/up 0.281 vs 0.312 ms with ordinary loads).  With two
// groups per wave the neighbouring wave reads the other half of each line, which the L2 then
// no longer holds (down projection 0.234 vs 0.185 ms).
#ifndef SK_NT_MIN_CG
#define SK_NT_MIN_CG 4
#endif
// SMALL: the launch beside a tiled GEMM, which runs only the routed experts of 1 .. small_rows
// rows.  The check sits in that instantiation alone: compiled into the decode kernels as well (where
// small_rows is 0 and it never returns), it slowed the Mixtral decode down projection from 0.139 to
// 0.163 ms with an identical main loop (three interleaved pairs; a uniform form of the check and
// 64-byte loop alignment did not recover it).
template <int MODE, int U, int CG, int RT, bool SMALL>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(FfnKArgs a) {
    using Tile = SkinnyTile<CG>;
    constexpr int NB = (MODE == MODE_IN_SWIGLU) ? 2 : 1;
    __shared__ __attribute__((aligned(16))) char s_tile[4][2][NB][Tile::BYTES];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int gw = blockIdx.x * 4 + wv;                        // global wave id
    const int ngroups = (a.Ncols + 16 * CG - 1) / (16 * CG);
    const int nseg = a.N + (a.has_shared ? 1 : 0);
    // K parts (out-projection): part kp of a segment takes K steps [kp KS, (kp + 1) KS) and
    // writes its partial sums to part kp of the output, which the combine adds in order
    const int nkp = (MODE == MODE_OUT && a.ksplit > 1) ? a.ksplit : 1;
    const int seg = gw / (ngroups * nkp), kp = (gw / ngroups) % nkp, cg = gw % ngroups;
    if (seg >= nseg) return;                                   // no block barrier below
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
    // beside a tiled GEMM: only the routed experts it leaves out
    if (SMALL && (seg >= a.N || row_end - row_beg > a.small_rows)) return;
    const int KS = a.K / 32 / nkp;                              // K steps of this wave
    const size_t step = (size_t)32 * a.Ncols;                   // elements between K steps
    B0 += (size_t)kp * KS * step;
    if (NB == 2) B1 += (size_t)kp * KS * step;
    // this lane's weight loads (CG per matrix and step): k-row q RPI + lane / CPR, chunk lane % CPR
    // of the wave's columns (Ncols is a multiple of 64, so every column group is whole); where they
    // go in the tile; and where its transposed reads start
    const bf16* pw0[CG];
    const bf16* pw1[CG];
    int woff[CG], roff[CG];
#pragma unroll
    for (int q = 0; q < CG; ++q) {
        const int r = q * Tile::RPI + lane / Tile::CPR, c = lane % Tile::CPR;
        const size_t o = (size_t)r * a.Ncols + (size_t)cg * 16 * CG + 8 * c;
        pw0[q] = B0 + o;
        pw1[q] = (NB == 2) ? B1 + o : nullptr;
        woff[q] = Tile::off(r, c);
        const int g = lane >> 4, L = lane & 15;
        roff[q] = Tile::off(8 * g + (L >> 2), 2 * q + ((L & 3) >> 1)) + (L & 1) * 8;
    }

    auto wload = [](const u32x4* p) -> u32x4 {
        if constexpr (CG >= SK_NT_MIN_CG) return __builtin_nontemporal_load(p);
        else return *p;
    };
    const int kq = (lane >> 4) * 8;                             // this lane's K offset in a step
    // RT tiles of 16 rows per pass over the weights: row tile t's lane row m0 + 16 t + (lane & 15)
    for (int m0 = row_beg; m0 < row_end; m0 += 16 * RT) {
        bool rok[RT];
        const bf16* pa[RT];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            const int r = m0 + 16 * t + (lane & 15);            // this lane's A row
            rok[t] = r < row_end;
            int src;
            if (MODE == MODE_OUT) src = rok[t] ? r : m0;
            else src = (seg < a.N) ? a.perm[rok[t] ? r : m0] / a.k : (rok[t] ? r : m0) - a.T * a.k;
            pa[t] = a.A + (size_t)src * a.K + kq + kp * KS * 32;
        }
        f32x4 acc0[RT][CG], acc1[RT][CG];
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                acc0[t][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
                acc1[t][c] = (f32x4){0.f, 0.f, 0.f, 0.f};
            }
        const bf16x8 zero8 = {};
        // a K step's weight pieces into tile t, and back as B fragments
        struct Frag { bf16x8 b0[CG], b1[CG]; };
        auto to_tile = [&](int t, const u32x4 (&w0)[CG], const u32x4 (&w1)[CG]) {
#pragma unroll
            for (int q = 0; q < CG; ++q) {
                *(u32x4*)(s_tile[wv][t][0] + woff[q]) = w0[q];
                if (NB == 2) *(u32x4*)(s_tile[wv][t][NB - 1] + woff[q]) = w1[q];
            }
        };
        auto from_tile = [&](int t, Frag& f) {
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                f.b0[c] = lds_read_tr_b16x8(s_tile, ((wv * 2 + t) * NB) * Tile::BYTES + roff[c], 4 * Tile::ROWB);
                if (NB == 2)
                    f.b1[c] = lds_read_tr_b16x8(s_tile, ((wv * 2 + t) * NB + 1) * Tile::BYTES + roff[c],
                                                4 * Tile::ROWB);
            }
        };
        auto mfmas = [&](const Frag& f, const bf16x8 (&av)[RT]) {
#pragma unroll
            for (int t = 0; t < RT; ++t)
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    acc0[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t], f.b0[c], acc0[t][c], 0, 0, 0);
                    if (NB == 2)
                        acc1[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t], f.b1[c], acc1[t][c], 0, 0, 0);
                }
        };
        int ks = 0;
        for (; ks + U <= KS; ks += U) {
            u32x4 w0[U][CG], w1[U][CG];
            bf16x8 av[U][RT];
#pragma unroll
            for (int u = 0; u < U; ++u) {
#pragma unroll
                for (int q = 0; q < CG; ++q) {
                    w0[u][q] = wload((const u32x4*)(pw0[q] + (ks + u) * step));
                    if (NB == 2) w1[u][q] = wload((const u32x4*)(pw1[q] + (ks + u) * step));
                }
#pragma unroll
                for (int t = 0; t < RT; ++t) av[u][t] = rok[t] ? *(const bf16x8*)(pa[t] + (ks + u) * 32) : zero8;
            }
            // every step's tile write and read go out before the MFMAs (steps alternate tiles)
            Frag f[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                to_tile(u & 1, w0[u], w1[u]);
                from_tile(u & 1, f[u]);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) mfmas(f[u], av[u]);
        }
        for (; ks < KS; ++ks) {
            u32x4 w0[CG], w1[CG];
#pragma unroll
            for (int q = 0; q < CG; ++q) {
                w0[q] = wload((const u32x4*)(pw0[q] + ks * step));
                if (NB == 2) w1[q] = wload((const u32x4*)(pw1[q] + ks * step));
            }
            bf16x8 av[RT];
#pragma unroll
            for (int t = 0; t < RT; ++t) av[t] = rok[t] ? *(const bf16x8*)(pa[t] + ks * 32) : zero8;
            Frag f;
            to_tile(ks & 1, w0, w1);
            from_tile(ks & 1, f);
            mfmas(f, av);
        }
        // 16x16 C layout: lane holds column (lane & 15), rows 4 * (lane >> 4) + i of each row tile
#pragma unroll
        for (int t = 0; t < RT; ++t)
#pragma unroll
            for (int c = 0; c < CG; ++c) {
                const int col = (cg * CG + c) * 16 + (lane & 15);
                if (col >= a.Ncols) continue;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = m0 + 16 * t + 4 * (lane >> 4) + i;
                    if (row >= row_end) continue;
                    if (MODE == MODE_OUT) {
                        const float scale = (a.row_scale && seg < a.N) ? a.row_scale[a.perm[row]] : 1.0f;
                        ((float*)a.C)[kp * a.part_stride + (size_t)row * a.Ncols + col] = acc0[t][c][i] * scale;
                    } else if (MODE == MODE_IN_SWIGLU) {
                        ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)(silu_f32(acc0[t][c][i]) * acc1[t][c][i]);
                    } else {
                        ((bf16*)a.C)[(size_t)row * a.Ncols + col] = (bf16)fmaxf(acc0[t][c][i], 0.f);
                    }
                }
            }
    }
}

template <int MODE, int U, int CG, int RT = 1, bool SMALL = false>
static hipError_t launch_skinny(const FfnKArgs& a, hipStream_t s) {
    const int nkp = (MODE == MODE_OUT && a.ksplit > 1) ? a.ksplit : 1;
    const long long waves = (long long)(a.N + (a.has_shared ? 1 : 0)) * ((a.Ncols + 16 * CG - 1) / (16 * CG)) * nkp;
    auto kern = ffn_skinny_kernel<MODE, U, CG, RT, SMALL>;
    hipLaunchKernelGGL(kern, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

// Decode-sized batches (at most 16 rows per expert on average) take the weight-streaming path.
// 16-column groups per wave and unroll depths, measured on the Mixtral decode layer (one box,
// 200 calls each): the in-projection takes four groups (whole 128-byte k-row pieces) two steps
// at a time, 0.281 ms with non-temporal loads (four steps: 0.280; two groups: 0.407).  The
// out-projection takes four groups two steps at a time, in two K parts (so that its
// 8 x 64 column groups still give every SIMD a wave): 0.141 ms, against 0.185 ms with two
// groups, four steps and one part, 0.186 ms with four groups in one part, and 0.193 ms with
// two groups in two parts.  Batches double-buffered in registers were no faster.
#ifndef SK_U_IN
#define SK_U_IN 2
#endif
#ifndef SK_CG_IN
#define SK_CG_IN 4
#endif
#ifndef SK_U_OUT
#define SK_U_OUT 2
#endif
#ifndef SK_CG_OUT
#define SK_CG_OUT 4
#endif
static bool skinny(const FfnLaunch& f) { return (long long)f.T * f.k <= 16LL * f.N; }
// Next to the tiled SwiGLU gate/up GEMM, routed experts with at most FFN_SMALL_ROWS rows run as
// weight streams, FFN_SMALL_RT tiles of 16 rows per pass over their weights (0: all in the tiled
// GEMM): a tile of such an expert streams a whole weight slice through the tiled kernel's LDS
// loads for a few rows, which the weight-stream kernel's register loads do faster.  Measured on
// one box (gate/up, ms, tiled -> split): skewed with capacity 1.53 -> 1.46, top-1 of 128 SwiGLU
// 5.55 -> 4.93, the other shapes unchanged.  The down projection and the ReLU in-projection were
// slower split (skewed down 0.80 -> 0.86, top-1 of 128 ReLU 2.71 -> 2.89 and 2.54 -> 2.78): a
// weight-stream wave re-reads its rows' activations for its own 64 columns, which against one
// weight matrix (not the two of SwiGLU) costs as much as the weights themselves.
#ifndef FFN_SMALL_ROWS
#define FFN_SMALL_ROWS 64
#endif
#ifndef FFN_SMALL_RT
#define FFN_SMALL_RT 4
#endif

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
    // weights K-major: column c of a [K, Ncols] matrix
    float s0 = 0.f;
    for (int i = 0; i < K; ++i) s0 = fmaf(ar[i], w0[(size_t)i * Ncols + c], s0);
    float v;
    if (MODE == MODE_IN_SWIGLU) {
        float s1 = 0.f;
        for (int i = 0; i < K; ++i) s1 = fmaf(ar[i], w1[(size_t)i * Ncols + c], s1);
        v = s0 / (1.0f + expf(-s0)) * s1;
    } else if (MODE == MODE_IN_RELU) {
        v = fmaxf(s0, 0.f);
    } else {
        v = s0 * ((row_scale && seg < N) ? row_scale[perm[r]] : 1.0f);
    }
    C[(size_t)r * Ncols + c] = v;
}

// ------------------------------------------------------------------ launchers
// Blocks of one kernel that the device keeps resident at once (a multiple of 8, one share per
// XCD), found once per (kernel, device).  Every instantiation has the same function-pointer type,
// so the cache is keyed on the kernel's address as well as the device.
template <typename K>
static int resident_blocks(K kern, int threads) {
    struct Entry {
        const void* kern;
        int dev, blocks;
    };
    static Entry cache[64];
    static int n_cached = 0;
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n_cached; ++i)
        if (cache[i].kern == (const void*)kern && cache[i].dev == dev) return cache[i].blocks;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, threads, 0) != hipSuccess) return 0;
    int v = (cus * (per_cu > 0 ? per_cu : 1)) / 8 * 8;
    if (v < 8) v = 8;
    if (n_cached < 64) cache[n_cached++] = Entry{(const void*)kern, dev, v};
    return v;
}

// Tiles of a tiled GEMM launch at most: m-tiles (an expert's rows in tiles of BM, the shared
// expert's T rows too) x n-tiles x K parts.
static long long tile_bound(int T, int k, int N, int has_shared, int Ncols, int ksplit, int BM, int BNH) {
    const long long mt = ((long long)T * k + BM - 1) / BM + N + (has_shared ? (T + BM - 1) / BM : 0);
    return mt * ((Ncols + BNH - 1) / BNH) * (ksplit < 1 ? 1 : ksplit);
}

// Schedule memory of the tiled GEMMs: eight claim counters, then one tile table; a claiming
// GEMM's launch writes both (ffn_tile_table) just before the GEMM, so successive launches on one
// stream can share them.  Sized for the smallest tiles (128 x 128) and either projection.
size_t ffn_sched_bytes(int T, int k, int N, int d, int d_ff, int has_shared, int ksplit) {
    const long long in = tile_bound(T, k, N, has_shared, d_ff, 1, 128, 128);
    const long long out = tile_bound(T, k, N, has_shared, d, ksplit, 128, 128);
    return FFN_CTR_BYTES + 16 * (size_t)(in > out ? in : out);
}

template <int MODE, int BM, int BNH, int WGM, int WGN>
static hipError_t launch_bf16(const FfnKArgs& ka, size_t sched_bytes, hipStream_t s) {
    using Cfg = FfnTile<MODE, BM, BNH, WGM, WGN>;
    auto kern = ffn_bf16_kernel<MODE, BM, BNH, WGM, WGN>;
    FfnKArgs a = ka;
    if (a.ksplit < 1) a.ksplit = 1;
    a.mt_max = (a.T * a.k + BM - 1) / BM + a.N + (a.has_shared ? (a.T + BM - 1) / BM : 0);
    a.n_tiles = (a.Ncols + BNH - 1) / BNH;
    const int resident = resident_blocks(kern, Cfg::NT);
    if (resident <= 0) return hipErrorInvalidDevice;
    const long long tiles = (long long)a.mt_max * a.n_tiles * a.ksplit;
    if (claims_tiles(MODE, BM)) {
        if (!a.ctr || FFN_CTR_BYTES + 16 * (size_t)tiles > sched_bytes) return hipErrorInvalidValue;
        const long long GT = (tiles + 63) / 64;         // table: one entry per lane, <= 256 blocks
        hipLaunchKernelGGL((ffn_tile_table<MODE, BM, BNH, WGM, WGN>), dim3((unsigned)(GT < 256 ? GT : 256)), dim3(64),
                           0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    long long G = 8 * ((tiles + 7) / 8);                // one tile per block at most
    if (G > resident) G = resident;
    hipLaunchKernelGGL(kern, dim3((unsigned)G), dim3(Cfg::NT), 0, s, a);
    return hipGetLastError();
}

// Tile choice from what the host knows (T, k, N, widths): rows per expert on average.
static bool big_tiles(const FfnLaunch& f) {
    return (long long)f.T * f.k >= 192LL * f.N;   // >= 192 rows per expert on average
}

// 320-row in-projection tiles (eight waves, 2 x 4) when experts hold 224 to 288 rows on
// average: an expert of 257 to 320 rows is then one m-tile instead of a full 256-row tile plus a
// short one that streams the expert's whole weight matrix a second time.  Measured on one box
// against 256-row tiles, gate/up projection: DeepSeek-V3 shape 4.22 vs 5.10 ms, top-1 over 16
// experts 1.05 vs 1.17, shared + top-7 of 256 3.94 vs 4.09, skewed with capacity 1.50 vs 1.53.
// (320 x 128 with four waves needs 320 accumulator registers per lane and spills; 320 x 64
// with four waves fits but was slower than 256-row tiles on all four.)
static bool tiles_320(const FfnLaunch& f) {
    const long long rows = (long long)f.T * f.k;
    return rows >= 224LL * f.N && rows <= 288LL * f.N;
}
// The out-projection takes 320 x 256 tiles (eight waves) from 240 rows per expert on average,
// with no upper limit: a 320-row tile moves 10% fewer bytes per flop through the CU's load path
// than a 256-row one.  Measured on one box against 256-row tiles, down projection: DeepSeek-V3
// shape 2.55 vs 2.84 ms, top-1 over 16 experts 0.65 vs 0.72, skewed layer 0.85 vs 0.89, Mixtral
// prefill (about 1024 rows per expert) 0.874 vs 0.912 (two interleaved pairs); at 224 rows per
// expert (shared + top-7 of 256), where few experts pass 256 rows, 2.48 vs 2.44.  The gate/up
// projection keeps 256-row tiles above 288 rows per expert (Mixtral 1.59 vs 1.77 ms).
static bool tiles_320_out(const FfnLaunch& f) {
    return (long long)f.T * f.k >= 240LL * f.N;
}

// K parts for the out-projection: for the tiled GEMM two when its K is long and one part alone
// would leave the last round of blocks on the CUs mostly empty; for the weight stream two when
// one part would run at most one wave per SIMD.  The parts' fp32 outputs are summed, in order,
// by the combine.
int ffn_out_ksplit(int T, int k, int N, int d, int d_ff, int has_shared, int dtype) {
    if (dtype != 1) return 1;
    const long long rows = (long long)T * k;
    if (rows <= 16LL * N) {                                // weight streaming (decode)
        // two parts when one would give the stream at most one wave per SIMD
        const long long waves = (long long)(N + (has_shared ? 1 : 0)) * ((d + 16 * SK_CG_OUT - 1) / (16 * SK_CG_OUT));
        return (waves <= 1024 && (d_ff / 32) % 2 == 0) ? 2 : 1;
    }
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
        a.ctr = f.ctr;
        if (f.ffn == 1) {
            a.B0 = (const bf16*)f.w_gate; a.B1 = (const bf16*)f.w_up;
            a.S0 = (const bf16*)f.sh_gate; a.S1 = (const bf16*)f.sh_up;
            if (skinny(f)) return launch_skinny<MODE_IN_SWIGLU, SK_U_IN, SK_CG_IN>(a, s);
            // (at 512 rows per expert on average, as on Mixtral, the launch would only cost time)
            a.small_rows = (long long)f.T * f.k < 512LL * f.N ? FFN_SMALL_ROWS : 0;
            const hipError_t e = tiles_320(f) ? launch_bf16<MODE_IN_SWIGLU, 320, 128, 2, 4>(a, f.sched_bytes, s)
                               : big_tiles(f) ? launch_bf16<MODE_IN_SWIGLU, 256, 128, 2, 2>(a, f.sched_bytes, s)
                                              : launch_bf16<MODE_IN_SWIGLU, 128, 128, 2, 2>(a, f.sched_bytes, s);
            if (e != hipSuccess || a.small_rows == 0) return e;
            return launch_skinny<MODE_IN_SWIGLU, SK_U_IN, SK_CG_IN, FFN_SMALL_RT, true>(a, s);
        }
        a.B0 = (const bf16*)f.w_up;
        a.S0 = (const bf16*)f.sh_up;
        if (skinny(f)) return launch_skinny<MODE_IN_RELU, SK_U_IN, SK_CG_IN>(a, s);
        if (big_tiles(f)) return launch_bf16<MODE_IN_RELU, 256, 256, 2, 2>(a, f.sched_bytes, s);
        return launch_bf16<MODE_IN_RELU, 128, 128, 2, 2>(a, f.sched_bytes, s);
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

// Routed rows of the out-projection in bf16: on bf16 layers with a shared expert, in one K part,
// on the tiled path, when the caller reads that format.  The fused forward allows it for
// fine-grained layers (k <= N / 8) whose gate weights are probabilities of a softmax over all N
// experts.  The shared expert's row carries weight 1 and stays fp32; a routed row is already
// scaled by its gate weight, and rounding it moves y by at most 2^-8 of that row's value (bf16's
// unit roundoff), so the routed rows add at most 2^-8 * sum_j w_j |f_j|, sum_j w_j being the mass of
// the k picks (about 0.2 for 8 of 256 experts).  Measured on one box: DeepSeek-V3 shape
// 7.35-7.39 -> 7.17 ms per layer (combine 0.43 -> 0.25 ms, down projection 2.52 -> 2.44), shared +
// top-7 of 256 6.99 -> 6.77-6.84, max|err|/RMS against the oracle unchanged (1.902e-2).  Where
// the picks hold most of the mass (1 of 2 or 2 of 4 experts) the routed rows carry as much of y
// as the shared one, and small layers of that kind measured 1.43e-2 -> 1.89e-2 with bf16 rows;
// they, and layers with renormalised top-k weights, keep fp32 rows.
int ffn_out_routed_bf16(const FfnLaunch& f) {
    return f.routed_bf16_ok && f.dtype == 1 && f.has_shared && f.ksplit <= 1 && !skinny(f) &&
           f.row_scale != nullptr;
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
        a.ctr = f.ctr;
        a.routed_bf16 = ffn_out_routed_bf16(f);
        if (skinny(f)) return launch_skinny<MODE_OUT, SK_U_OUT, SK_CG_OUT>(a, s);
        // eight waves (2 x 4, two per SIMD) for the out-projection: measured on the same box,
        // Mixtral down projection 0.94 vs 1.01 ms with four, skewed 0.89 vs 0.93, DeepSeek-V3
        // 2.72 vs 2.71; four stay faster for the SwiGLU in-projection (1.70 vs 1.59 ms)
        if (tiles_320_out(f)) return launch_bf16<MODE_OUT, 320, 256, 2, 4>(a, f.sched_bytes, s);
        if (big_tiles(f)) return launch_bf16<MODE_OUT, 256, 256, 2, 4>(a, f.sched_bytes, s);
        return launch_bf16<MODE_OUT, 128, 128, 2, 2>(a, f.sched_bytes, s);
    }
    const long long rows_total = (long long)f.T * f.k + (f.has_shared ? f.T : 0);
    const long long n = rows_total * f.d;
    hipLaunchKernelGGL(ffn_f32_kernel<MODE_OUT>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       (const float*)f.h, f.perm, f.offsets, (const float*)f.w_down, nullptr,
                       (const float*)f.sh_down, nullptr, f.row_scale, (float*)f.y_perm, f.T, f.k, f.N,
                       f.has_shared, f.d_ff, f.d);
    return hipGetLastError();
}
