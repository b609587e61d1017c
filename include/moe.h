/*
 * moe.h -- C ABI of the sparse mixture-of-experts layer forward on MI355X (gfx950).
 *
 * One call computes, for one GPU holding every expert of the layer:
 *   1. router logits      z = x W_r (+ b)
 *   2. ranking + gating   top-k experts per token and their gate weights
 *   3. expert capacity    optional per-expert cap with re-routing to the next-best expert
 *   4. grouping by expert the (token, slot) pairs sorted into contiguous per-expert rows
 *   5. expert FFNs        grouped over experts (SwiGLU or two-layer ReLU), plus an
 *                         optional shared expert applied to every token
 *   6. combine            gate-weighted sum of each token's k expert outputs
 *
 * Sources (web pages on MoE layers, cited by title and section):
 *   [P1] "MoE 分片：混合專家模型的平行化策略" -- sections 什麼是 MoE 模型 (router is a learned
 *        linear layer, only the top-k experts run, outputs weighted by the router's scores;
 *        an expert is two linear maps around an activation) and 動態 token 路由 (steps 2
 *        and 6: scoring, softmax, top-k; weighted combine on the token's own device).
 *   [P2] "MoE 推理：激活参数 vs 总参数与专家路由" -- sections 深入原理 and 代码 (router linear,
 *        top-k, softmax over the picked logits, weighted sum; decode reads the weights of the
 *        distinct experts a batch touches).
 *   [P3] "大模型MoE混合专家架构原理与DeepSeek-V4工程实践解析" -- section MoE核心机制 (softmax
 *        over all experts, then top-K, outputs weighted by the un-renormalised probabilities).
 *   [P4] "MoE 架构科普：为什么大模型要「混合专家」" -- section 专家粒度 (shared experts that
 *        every token passes through).
 *   [P5] "MoE稀疏激活原理与工程实践：揭秘大模型参数幻觉" -- section 2.2 (expert capacity:
 *        a full expert sends the token to its next-best expert; capacity_factor 2.0) and
 *        section 3.1 (tokens regrouped by target expert id before the experts run).
 *
 * Conventions
 *  - All tensors are row-major and contiguous, on the device unless stated otherwise.
 *  - Weights are in the x W orientation of the pages' toy ([P2] 代码: router_W [d, N],
 *    x @ experts_W[e]), row-major with the output index fastest:
 *      w_router [d, N]; w_gate, w_up [N, d, d_ff]; w_down [N, d_ff, d];
 *      shared expert: sh_gate, sh_up [d, d_ff], sh_down [d_ff, d].
 *    For MOE_FFN_RELU2, w_up holds W1 and w_down holds W2 (y = relu(x W1) W2); w_gate unused.
 *  - Activations and weights share one dtype (MOE_F32 or MOE_BF16).  Logits, gate weights
 *    and every accumulation are fp32; the router accumulates fp32 partial sums of 256
 *    products each into fp64.  The FFN hidden state H is stored in the layer dtype (bf16
 *    rounding to nearest even); the per-row expert outputs (y_perm) that moe_expert_ffn and
 *    moe_combine exchange are fp32 for every layer dtype, and the output y is rounded once, in
 *    the combine, to the layer dtype.  Inside the fused forward (workspace only), a bf16 layer
 *    with a shared expert, MOE_GATE_SOFTMAX_TOPK and k <= N / 8 keeps its routed rows, already
 *    scaled by their gate weights, in bf16 (the shared expert's rows stay fp32); each of those
 *    roundings moves y by at most 2^-8 of that row's value (bf16 unit roundoff).
 *  - Ownership: the caller owns every buffer, including the workspace sized by
 *    moe_workspace_size().  The library allocates no device memory, keeps no pointer after a
 *    call returns and holds no state across calls beyond the thread-local error text.
 *  - Asynchrony: every compute call validates its arguments on the host, then only enqueues
 *    kernels on `stream` (a hipStream_t; NULL = the default stream) and returns.  The host is
 *    never synchronised.  On any error status nothing has been enqueued, except MOE_ERR_HIP,
 *    which reports a failed launch (earlier kernels of that call may have been enqueued).
 *  - Determinism: no floating-point atomics; every reduction has a fixed order, so equal
 *    inputs give bit-identical outputs.
 *  - Thread safety: calls may run concurrently if each uses its own workspace and outputs.
 *  - NaN/Inf inputs are not checked; results are then undefined.
 *
 * Routing semantics (fixed readings where the pages are silent)
 *  - Ranking: descending logit; equal logits rank the lower expert id first.
 *  - idx[t, j] is the expert of token t's slot j; slot 0 is the best-ranked kept expert.
 *  - MOE_GATE_TOPK_SOFTMAX: w = softmax over the logits of the k kept experts [P2].
 *    MOE_GATE_SOFTMAX_TOPK: w_j = softmax over all N logits, taken at idx_j, no renormalisation [P3].
 *  - Capacity (capacity_factor > 0): C = ceil(capacity_factor * T * k / N).  Slots are placed
 *    in priority order: every token's slot 0 in token order, then every token's slot 1, ...
 *    A slot takes the highest-ranked expert that the token does not already hold and whose
 *    fill is still below C [P5 2.2].  A slot with no room anywhere is dropped: idx = -1,
 *    w = 0, and it appears in no expert's rows.  Gate weights use the final experts' logits.
 *  - The logit bias b (optional) is part of the logit for ranking and for the weights.
 *  - Grouping: counts[e] = number of slots routed to e; offsets = exclusive prefix sum
 *    (offsets[N] = kept slots); perm[r] = slot s = t*k + j held by row r, rows of expert e
 *    ordered by ascending slot; inv[s] = row of slot s, or -1 if the slot was dropped.
 *  - Shared expert (has_shared): applied to every token with weight 1; it is not counted in
 *    counts.  In y_perm its output for token t sits at row T*k + t.
 *
 * Limits: 1 <= k <= N <= 256; T >= 0 (T = 0 is a no-op); d, d_ff >= 1.  For MOE_BF16:
 *   d % 64 == 0 and d_ff % 64 == 0, x below 4 GiB (T * d * 2 < 2^32 bytes) and one expert
 *   matrix below 4 GiB (d * d_ff * 2 < 2^32 bytes), else MOE_ERR_UNSUPPORTED.  MOE_F32 has no divisibility requirement.  T * k must fit in int32
 *   with T*k + T + 1 < 2^31.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,   /* null required pointer, size or enum out of range */
    MOE_ERR_UNSUPPORTED = 2,   /* valid request the library does not support (N > 256, d % 64 on bf16) */
    MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_size() or ws NULL */
    MOE_ERR_HIP = 4            /* a HIP call or kernel launch failed; see moe_last_error() */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;
typedef enum { MOE_GATE_TOPK_SOFTMAX = 0, MOE_GATE_SOFTMAX_TOPK = 1 } moe_gating;
typedef enum { MOE_FFN_RELU2 = 0, MOE_FFN_SWIGLU = 1 } moe_ffn;

/* hipStream_t, passed as an opaque handle (NULL = default stream). */
typedef void *moe_stream_t;

/* Shapes and options of one layer call (all fields by value, host memory). */
typedef struct {
    int32_t T;                 /* tokens (rows of x) */
    int32_t d;                 /* model width */
    int32_t N;                 /* routed experts */
    int32_t k;                 /* experts per token */
    int32_t d_ff;              /* expert hidden width */
    int32_t dtype;             /* moe_dtype */
    int32_t ffn;               /* moe_ffn */
    int32_t gating;            /* moe_gating */
    float capacity_factor;     /* <= 0: no capacity limit */
    int32_t has_shared;        /* 1: one shared expert, weight 1, every token */
} moe_layer_desc;

/* Device pointers to the layer's weights (layouts in the header comment). */
typedef struct {
    const void *w_router;      /* [d, N] */
    const float *logit_bias;   /* [N] fp32, or NULL */
    const void *w_gate;        /* [N, d, d_ff]; NULL for MOE_FFN_RELU2 */
    const void *w_up;          /* [N, d, d_ff] (W1 for RELU2) */
    const void *w_down;        /* [N, d_ff, d] (W2 for RELU2) */
    const void *sh_gate;       /* [d, d_ff] or NULL (required with has_shared and SWIGLU) */
    const void *sh_up;         /* [d, d_ff] or NULL (required with has_shared) */
    const void *sh_down;       /* [d_ff, d] or NULL (required with has_shared) */
} moe_weights;

/* Optional routing outputs of moe_layer_forward (device pointers; any may be NULL). */
typedef struct {
    float *logits;             /* [T, N] fp32 router logits (bias included) */
    int32_t *idx;              /* [T, k] */
    float *w;                  /* [T, k] */
    int32_t *counts;           /* [N] */
    int32_t *offsets;          /* [N + 1] */
    int32_t *perm;             /* [T * k]; entries past offsets[N] are unspecified */
    int32_t *inv;              /* [T * k] */
} moe_routing;

/* Number of pipeline stages whose boundaries moe_layer_forward_timed() marks:
 * route | capacity | permute | ffn_in (gate/up or W1) | ffn_out (down or W2) | combine. */
#define MOE_NUM_STAGES 6

/* Bytes of device workspace a moe_layer_forward() call with this descriptor needs; the
 * per-stage calls need at most as much.  Returns 0 for an invalid descriptor. */
size_t moe_workspace_size(const moe_layer_desc *desc);

/* Steps 1-3 [P1 步驟二, P2 深入原理, P3 MoE核心机制, P5 2.2]: router GEMM, ranking, gating
 * and (if capacity_factor > 0) capacity routing.
 *   x [T, d] (layer dtype); w_router [d, N]; logit_bias [N] fp32 or NULL.
 *   logits [T, N] fp32 output or NULL; idx [T, k] int32 and w [T, k] fp32 outputs (required).
 *   ws/ws_bytes: workspace of at least moe_workspace_size(desc) bytes. */
moe_status moe_route(const moe_layer_desc *desc, const void *x, const void *w_router,
                     const float *logit_bias, float *logits, int32_t *idx, float *w,
                     void *ws, size_t ws_bytes, moe_stream_t stream);

/* Step 4 [P5 3.1]: stable grouping of the T*k slots by expert (idx -1 = dropped slot).
 *   idx [T, k] in; counts [N], offsets [N + 1], perm [T * k], inv [T * k] out (required).
 *   x [T, d] and x_perm [T * k, d]: optional (both or neither); when given, row r of x_perm
 *   receives x[perm[r] / k] for r < offsets[N]. */
moe_status moe_permute(const moe_layer_desc *desc, const int32_t *idx, int32_t *counts,
                       int32_t *offsets, int32_t *perm, int32_t *inv, const void *x,
                       void *x_perm, moe_stream_t stream);

/* Steps 5 [P1 什麼是 MoE 模型, P4 专家粒度]: the expert FFNs, grouped over experts.
 *   Row r < offsets[N] of expert e (offsets[e] <= r < offsets[e+1]) computes
 *   FFN_e(x[perm[r] / k]) and, if row_scale is given, multiplies it by row_scale[perm[r]]
 *   (the slot's gate weight, [T * k] fp32).  With has_shared, rows T*k .. T*k + T - 1 hold
 *   the shared expert's output for tokens 0 .. T-1 (never scaled).
 *   y_perm: [(T * k + (has_shared ? T : 0)), d] fp32; rows not listed above are left
 *   untouched.  ws: workspace (hidden state H, then the grouped GEMMs' schedule: tile-claim counters
 *   and a table of the tiles); moe_workspace_size(desc) bytes always suffice. */
moe_status moe_expert_ffn(const moe_layer_desc *desc, const moe_weights *weights,
                          const void *x, const int32_t *perm, const int32_t *offsets,
                          const float *row_scale, void *y_perm, void *ws, size_t ws_bytes,
                          moe_stream_t stream);

/* Step 6 [P1 步驟六, P2 代码]: y[t] = sum_j s_j * y_perm[inv[t*k + j]] (+ y_perm[T*k + t] with
 * has_shared), summed in slot order in fp32 and rounded once to the layer dtype;
 * s_j = w[t, j] if w is not NULL, else 1 (rows already scaled).  Dropped slots are skipped.
 *   y_perm (fp32) as produced by moe_expert_ffn; inv [T * k]; w [T, k] or NULL; y [T, d] out
 *   in the layer dtype. */
moe_status moe_combine(const moe_layer_desc *desc, const void *y_perm, const int32_t *inv,
                       const float *w, void *y, moe_stream_t stream);

/* The whole layer (steps 1-6) in one call.  y [T, d] out.  routing: optional copies of the
 * routing tensors (NULL = not wanted). */
moe_status moe_layer_forward(const moe_layer_desc *desc, const moe_weights *weights,
                             const void *x, void *y, const moe_routing *routing,
                             void *ws, size_t ws_bytes, moe_stream_t stream);

/* As moe_layer_forward, and additionally records hipEvent_t events[i] (caller-created,
 * i = 0 .. MOE_NUM_STAGES, so MOE_NUM_STAGES + 1 entries) on `stream` before the first stage
 * and after each stage, so that hipEventElapsedTime(events[i], events[i+1]) is stage i's
 * device time.  A stage that does not apply (capacity without a limit) has zero length.
 * A NULL entry records nothing at that boundary (to time one stage, pass only its two
 * events); events may be NULL (then this is moe_layer_forward). */
moe_status moe_layer_forward_timed(const moe_layer_desc *desc, const moe_weights *weights,
                                   const void *x, void *y, const moe_routing *routing,
                                   void *ws, size_t ws_bytes, moe_stream_t stream,
                                   void *const *events);

/* Bytes of the built-in workspace of moe_layer_forward_noalloc (one array per GPU). */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* moe_layer_forward without a caller workspace and without any allocation, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The workspace is a file-scope device array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) in the library, one per GPU, created with the library's
 * code object and held until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress, on the first call made with that device current).  The caller still
 * passes x, y and the optional routing outputs, as for moe_layer_forward; `stream` must belong
 * to the current device.
 * Errors: MOE_ERR_UNSUPPORTED (before anything is enqueued) when moe_workspace_size(desc)
 * exceeds MOE_NOALLOC_SCRATCH_BYTES -- decode-sized batches fit, e.g. T <= 256 tokens on a
 * Mixtral-8x7B-shaped layer -- plus every error of moe_layer_forward.
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (nothing
 * in it needs to start at zero): calls that overlap on one GPU, on different streams or from
 * different threads, race and give undefined results; serialise them. */
moe_status moe_layer_forward_noalloc(const moe_layer_desc *desc, const moe_weights *weights,
                                     const void *x, void *y, const moe_routing *routing,
                                     moe_stream_t stream);

/* Number of values moe_routing_stats() writes to `stats`, in this order:
 *   0 entropy_bits        -sum_i f_i log2 f_i over experts with f_i > 0, f_i = counts[i] / sum(counts)
 *   1 entropy_ideal_bits  log2 N (every expert with the same share)
 *   2 top3_share          share of the kept slots held by the three most used experts
 *   3 max_share           largest f_i
 *   4 cv                  population standard deviation of counts[0..N-1] over their mean
 *   5 balance_loss        alpha * N * sum_i f_i * p_i, p_i = softmax over all N logits, averaged
 *                         over the T tokens
 *   6 reroute_rate        share of the T*k slots whose expert idx[t, j] is not among the token's
 *                         k best-ranked experts (descending logit, ties to the lower id); dropped
 *                         slots count
 *   7 experts_touched     number of experts with counts[i] > 0 */
#define MOE_NUM_STATS 8

/* Routing health statistics of one call [P5 4.2 (entropy against log2 N, top-3 experts, std /
 * mean of the counts), P3 MoE核心机制 (load-balancing loss alpha * N * sum f_i p_i), P5 2.2 and
 * 3.3 (re-routing under capacity, its rate)].
 *   logits [T, N] fp32, idx [T, k] int32 (-1 = dropped), counts [N] int32: the routing of one
 *   call, e.g. moe_layer_forward's moe_routing outputs (counts must be those of idx).
 *   alpha: balance-loss coefficient (the pages use 0.01).
 *   stats [MOE_NUM_STATS] fp64 and top3 [3] int32 (the three most used experts, count
 *   descending, ties to the lower id, -1 past N) out, on the device; prob_mean [N] fp64 out
 *   (p_i above) or NULL.  If no slot is kept (counts all 0) the share-based values 0, 2-5 are NaN.
 *   ws/ws_bytes: workspace of at least moe_workspace_size(desc) bytes (per-block partial sums).
 *   Deterministic: the same inputs give the same bits.  T must be >= 1. */
moe_status moe_routing_stats(const moe_layer_desc *desc, const float *logits, const int32_t *idx,
                             const int32_t *counts, double alpha, double *stats, int32_t *top3,
                             double *prob_mean, void *ws, size_t ws_bytes, moe_stream_t stream);

/* ---- Int4 expert weights for weight-streaming (decode) layers [P3 DeepSeek-V4的MoE架构工程细节:
 * GPTQ/AWQ INT4 expert weights at a quarter of the memory; the pages give no format].  Format:
 * per output r (a column of a [K, rows] weight matrix) and group of 128 consecutive inputs,
 * scale = amax / 7 (fp32), q = clamp(rint(w / scale), -8, 7) (fp32 division, ties to even;
 * all-zero group: scale 0, q 0); the weight stands for scale * q.  Codes q + 8, four bits each,
 * eight per uint32, one row of words per output: within output r and group g, word 4a + s (a, s
 * in 0..3) holds inputs k = 128g + 32s + 8a + i (i = 0..7), input i at bit 4 (i / 2) + 16 (i % 2).
 * A stack of n matrices [K, rows]: codes [n, rows, K / 8] uint32, scales [n, K / 128, rows] fp32
 * (device). */
typedef struct {
    const uint32_t *codes;
    const float *scales;
} moe_q4_matrix;

/* Layer weights with int4 experts; the router stays in the layer dtype (bf16). */
typedef struct {
    const void *w_router;      /* [d, N] bf16 */
    const float *logit_bias;   /* [N] fp32, or NULL */
    moe_q4_matrix w_gate;      /* quantised [N, d, d_ff]: codes [N, d_ff, d/8]; unused for RELU2 */
    moe_q4_matrix w_up;        /* quantised [N, d, d_ff] (W1 for RELU2) */
    moe_q4_matrix w_down;      /* quantised [N, d_ff, d]: codes [N, d, d_ff/8] */
    moe_q4_matrix sh_gate, sh_up, sh_down;   /* shared expert, as the routed ones */
} moe_weights_q4;

/* Quantise n_mats bf16 matrices w [n_mats, K, rows] (device, x W orientation) to the format above.
 * K % 128 == 0 (MOE_ERR_UNSUPPORTED otherwise). */
moe_status moe_quantize_q4(const void *w, int32_t n_mats, int32_t rows, int32_t K, uint32_t *codes,
                           float *scales, moe_stream_t stream);

/* moe_expert_ffn with int4 expert weights: every expert runs as a weight stream (one 16-row
 * tile at a time, the decode regime; larger batches are correct but re-read the weights per
 * tile).  Needs a bf16 layer with d % 128 == 0 and d_ff % 128 == 0.  Other arguments as
 * moe_expert_ffn. */
moe_status moe_expert_ffn_q4(const moe_layer_desc *desc, const moe_weights_q4 *weights,
                             const void *x, const int32_t *perm, const int32_t *offsets,
                             const float *row_scale, void *y_perm, void *ws, size_t ws_bytes,
                             moe_stream_t stream);

/* moe_layer_forward_timed with int4 expert weights (events may be NULL). */
moe_status moe_layer_forward_q4(const moe_layer_desc *desc, const moe_weights_q4 *weights,
                                const void *x, void *y, const moe_routing *routing, void *ws,
                                size_t ws_bytes, moe_stream_t stream, void *const *events);

/* ---- Expert parallelism: the layouts either side of the two all-to-alls [P1 專家平行化詳解 (each
 * GPU owns a subset of the experts; two all-to-alls per layer), P1 動態 token 路由 steps 3-6 (tokens
 * go to the GPUs owning their experts, the outputs come back, the combine runs at the origin)].
 * The exchanges themselves (counts, then rows, then the rows back) belong to the caller's
 * collective library; these calls produce and consume the buffers they carry.
 * owner: HOST array [N], owner[e] = rank holding expert e, each in [0, G); 1 <= G <= MOE_EP_MAX_RANKS.
 * A rank's local experts are the experts it owns, in ascending id (its weight stacks in that order). */
#define MOE_EP_MAX_RANKS 64

/* Send side, on each source rank: the stable grouping of its T*k slots by (owner rank, expert),
 * so that destination r's rows are the contiguous range send_offsets[r] .. send_offsets[r+1]-1
 * and, inside it, each expert's rows are contiguous in ascending slot order.
 *   idx [T, k] in (-1 or an index outside [0, N) = dropped slot).
 *   counts [N], expert_offsets [N + 1] (first send row of expert e; [N] = kept slots),
 *   send_counts [G], send_offsets [G + 1], perm [T * k] (send row -> slot), inv [T * k] (slot ->
 *   send row, -1 if dropped): outputs, required.  counts is what the count exchange sends to
 *   every destination.
 *   x [T, d] and send_buf [T * k, d] (layer dtype): optional (both or neither); send row r
 *   receives x[perm[r] / k]. */
moe_status moe_ep_dispatch(const moe_layer_desc *desc, const int32_t *idx, const int32_t *owner, int32_t G,
                           int32_t *counts, int32_t *expert_offsets, int32_t *send_counts,
                           int32_t *send_offsets, int32_t *perm, int32_t *inv, const void *x,
                           void *send_buf, moe_stream_t stream);

/* Receive side, on rank `rank`: the layout of the rows the sources sent it.
 *   recv_counts [G, N] int32 device: row s = source s's counts (from moe_ep_dispatch).
 *   The receive buffer is source-major: source s's rows are recv_offsets[s] ..
 *   recv_offsets[s+1]-1, ordered as that source sent them.
 *   Outputs: recv_offsets [G + 1]; local_offsets [n_local + 1] (n_local = experts this rank owns):
 *   the grouped order lists local expert 0's rows from every source (source order), then local
 *   expert 1's, ...; recv_perm [max_rows]: grouped row -> receive row; recv_inv [max_rows]:
 *   receive row -> grouped row.  Run the expert FFN on the received rows with
 *   moe_expert_ffn(desc with T = rows, k = 1, N = n_local; x = receive buffer, perm = recv_perm,
 *   offsets = local_offsets; the rank's own weight stacks).
 *   max_rows: capacity of recv_perm / recv_inv; if the sources sent more rows
 *   (recv_offsets[G] > max_rows) the entries past max_rows are not written.
 *   Needs G * n_local <= 4096. */
moe_status moe_ep_receive_layout(int32_t N, int32_t G, const int32_t *owner, int32_t rank,
                                 const int32_t *recv_counts, int32_t max_rows, int32_t *recv_offsets,
                                 int32_t *local_offsets, int32_t *recv_perm, int32_t *recv_inv,
                                 moe_stream_t stream);

/* After the expert FFN on a rank: ret[r] = y_grouped[recv_inv[r]] for every receive row r <
 * min(recv_offsets[G], max_rows), i.e. the expert outputs in receive order, which the return
 * exchange carries back (source s gets rows recv_offsets[s] .. recv_offsets[s+1]-1).  Each
 * source then concatenates what it gets back in rank order, which is its send order, and runs
 * moe_combine with its own inv and gate weights.
 *   y_grouped and ret: max_rows rows each.  row_bytes: bytes per row (d * 4 for fp32 expert
 *   outputs), a multiple of 16. */
moe_status moe_ep_unpack(int32_t G, int32_t max_rows, int32_t row_bytes, const int32_t *recv_offsets,
                         const int32_t *recv_inv, const void *y_grouped, void *ret, moe_stream_t stream);

/* Static text of a status code. */
const char *moe_status_str(moe_status s);
/* Detail of the last error on the calling thread ("" if none). */
const char *moe_last_error(void);
/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
