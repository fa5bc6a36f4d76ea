/*
 * moe.h -- C ABI of the MI355X fused Mixture-of-Experts layer forward (libmoe.so).
 *
 * The layer: per token t, a router picks k experts e_{t,j} with weights w_{t,j}; the output
 * is out[t] = sum_j w_{t,j} * W2_e (SiLU(W1_e x_t) * (W3_e x_t)).  The library computes it
 * on one GPU in five stream-ordered steps, each a hand-written HIP kernel for gfx950:
 *   1. route   -- top-k gate (softmax, sigmoid, or the DeepSeek-V3 biased grouped gate of
 *                 SGLang PR #3191 "Add deepseek_v3 fused gate");
 *   2. align   -- the moe_align_block_size step of vLLM PR #12185 ("[Kernel] add triton
 *                 fused moe kernel for gptq/awq", note 1): pairs sorted by expert, each
 *                 expert padded to whole blocks of block_m rows, no host synchronisation;
 *   3. GEMM1   -- grouped gate/up projection over all experts in one launch (the one-launch
 *                 argument of vLLM PR #12185's opening), SiLU(gate) * up fused;
 *   4. GEMM2   -- grouped down projection, scaled by the pair's top-k weight;
 *   5. reduce  -- unpermute and sum each token's k rows in a fixed order (TensorRT-LLM's
 *                 unpermute_and_reduce, named in the last review comment of SGLang PR #3191),
 *                 with no floating-point atomics (SGLang PR #2333, Background, reports
 *                 atomic_add corrupting the output).
 *
 * Conventions for every function below:
 *  - Pointers marked [device] are GPU addresses (hipMalloc / torch CUDA tensors); [host]
 *    are CPU addresses.  The caller allocates and owns every buffer; the library allocates
 *    nothing, keeps no pointer after returning, and holds no mutable global state apart
 *    from a per-device cache of device properties, so calls from several threads are safe.
 *  - Every GPU-side function only enqueues work on `stream` (a hipStream_t; NULL = the
 *    default stream) and returns without waiting; buffers must stay valid until that work
 *    completes.  Nothing synchronises the host or allocates, so a whole moe_forward may be
 *    captured into a hipGraph (SGLang PR #3191 forbids host synchronisation in the gate for
 *    exactly this reason; vLLM PR #12185 makes align graph-safe).
 *  - All argument checks happen before anything is enqueued: on any error nothing runs.
 *    Launch failures are reported as MOE_ERR_HIP.  Non-finite inputs are outside the
 *    contract (results are then unspecified but every kernel still terminates).
 *  - T = 0 is valid and enqueues nothing.
 *  - Tensors are dense and row-major.  bf16 is the bit pattern of IEEE binary32's upper
 *    half; fp8 is OCP E4M3FN (bias 7, max 448, no infinities); int4 weights are unsigned
 *    nibbles, column c of a row in byte c/2 (low nibble when c is even), dequantised as
 *    (q - z) * s with fp16 scale s and fp16 zero point z per group of 128 columns; z must
 *    hold an integer in [0, 15] (as GPTQ/AWQ packing produces).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,   /* null / misaligned pointer, bad size or mode */
    MOE_ERR_UNSUPPORTED = 2,        /* valid but not built: e.g. a shape outside the tiles */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                 /* a HIP call or kernel launch failed */
} moe_status;

typedef enum {
    MOE_ROUTE_SOFTMAX = 0,              /* p = softmax(logits); top-k of p                      */
    MOE_ROUTE_SIGMOID = 1,              /* s = sigmoid(logits); key = s (+ bias); top-k of key  */
    MOE_ROUTE_GROUPED_SIGMOID_BIAS = 2  /* DeepSeek-V3 grouped gate with correction bias        */
} moe_route_kind;

typedef enum {
    MOE_DT_BF16 = 0,
    MOE_DT_FP32 = 1,
    MOE_DT_FP8_E4M3 = 2,    /* w8a8: per-expert per-tensor weight scales, dynamic
                               per-tensor activation scales */
    MOE_DT_INT4_G128 = 3    /* weights only: the hidden states and the intermediate stay
                               bf16 (the kernels multiply on bf16 MFMA, so no activation is
                               narrowed to a smaller range) */
} moe_dtype;

/*
 * Router configuration.
 *  num_experts E in [1, 256]; top_k k in [1, min(E, 64)].
 *  SOFTMAX: the k experts with the largest logits (ties -> lower expert index), weight p_e
 *    (fp64 softmax over all E), renormalised over the k when `renormalize`.
 *  SIGMOID: key_e = sigmoid(x_e) (+ bias_e when a bias is passed), sigmoid evaluated in fp64
 *    and rounded once to fp32, the key sum in fp32; weight sigmoid(x_e), renormalised when
 *    asked.
 *  GROUPED_SIGMOID_BIAS: key_e = sigmoid(x_e) + bias_e; E experts in n_group groups of
 *    E/n_group consecutive experts (n_group in [1, 64], dividing E); group score = fp32
 *    sum of the group's two largest keys; the topk_group best groups are kept (ties ->
 *    lower group); the k best keys among them are chosen (k <= topk_group * E / n_group);
 *    weight sigmoid(x_e) (the bias never enters a weight), renormalised when asked.
 *  Every mode multiplies the weights by routed_scaling.  Slot order is the selection order
 *  (key descending, expert index ascending), so the result is unique and reproducible.
 *  logits_dtype: MOE_DT_BF16 or MOE_DT_FP32.
 */
typedef struct {
    int32_t num_experts;
    int32_t top_k;
    int32_t kind;            /* moe_route_kind */
    int32_t renormalize;     /* 0 or 1 */
    int32_t n_group;         /* grouped gate only (else ignored) */
    int32_t topk_group;      /* grouped gate only (else ignored) */
    float routed_scaling;    /* 1.0 for none */
    int32_t logits_dtype;    /* moe_dtype: BF16 or FP32 */
} moe_route_cfg;

/*
 * One MoE layer: its router and its E experts' weights [device].  H and I must be
 * multiples of 128; E = route.num_experts.
 *  weight_dtype MOE_DT_BF16:     w13 bf16 [E, 2I, H], w2 bf16 [E, H, I].
 *  weight_dtype MOE_DT_FP8_E4M3: w13/w2 E4M3 codes, same shapes; w13_scale, w2_scale fp32
 *                                [E] (weight = code * scale of its expert and matrix).
 *  weight_dtype MOE_DT_INT4_G128: w13 uint8 [E, 2I, H/2], w2 uint8 [E, H, I/2];
 *                                scales and zero points group-major: w13_s, w13_z fp16
 *                                [E, H/128, 2I]; w2_s, w2_z fp16 [E, I/128, H] (the group
 *                                g of row n of expert e at [e][g][n], so one group's
 *                                values for consecutive rows are contiguous).
 * Rows [0, I) of each w13 matrix are the gate projection (through SiLU), rows [I, 2I) the
 * up projection.  correction_bias: fp32 [E] for the grouped gate (required there), optional
 * for SIGMOID, ignored for SOFTMAX.  Weight pointers must be 16-byte aligned; scale and bias
 * pointers 4-byte aligned.
 */
typedef struct {
    int32_t E, H, I;
    int32_t weight_dtype;            /* moe_dtype */
    moe_route_cfg route;
    const void *w13;
    const void *w2;
    const float *w13_scale, *w2_scale;
    const uint16_t *w13_s, *w13_z, *w2_s, *w2_z;
    const float *correction_bias;
} moe_layer;

/*
 * Execution plan of moe_forward: how the two grouped GEMMs are tiled.  block_m is the
 * align block height and the GEMM tile height; gemm1_tile / gemm2_tile index the tile
 * shapes compiled for the layer's weight type (moe_plan_describe lists them); split_k
 * splits GEMM2's reduction into that many fp32 partial sums, combined in a fixed order by
 * the reduce step; split_k1 (0 or 1: none) splits GEMM1's likewise -- fp32 partial sums of
 * the gate and up projections that a finishing pass adds in a fixed order before SiLU * up
 * (tiles with block_m <= 32 only: the small-T case, where it multiplies the number of
 * workgroups streaming weights).
 * split_tail (0 or 1: off; 2..16 with split_k = 1 and a pipelined bf16 or fp8 GEMM2 tile):
 * GEMM2 runs as a persistent grid, one tile per workgroup per round; when its last round
 * would be at most half full, the row blocks of that round are computed instead as
 * S = min(split_tail, grid / their tiles) K splits -- fp32 partial sums that the reduce
 * step adds in a fixed order -- so that the round's work spreads over the whole grid.  The
 * grid size and the number of row blocks are known on the device only; GEMM2 records the
 * split it took.
 * max_workgroups (0: the whole device) caps the persistent grids of both GEMMs, e.g. to
 * leave compute units to concurrent work.
 * split_tail1 (0 or 1: off; 2..16 with split_k1 <= 1 and a pipelined bf16 or fp8 GEMM1
 * tile): the same for GEMM1 -- the split row blocks' gate and up sums go to fp32 planes and
 * a finishing pass (stage MOE_STAGE_GEMM1_FINISH) adds them in a fixed order and applies
 * SiLU * up to those rows before GEMM2.
 * ragged (0 or 1): 0 pads each expert's rows to whole blocks of block_m (moe_align's
 * layout: filler entries in sorted_token_ids, and the intermediates h and y hold a row for
 * every entry).  1 lays the pairs out with no padding -- the permutation of TensorRT-LLM's
 * expand_and_permute and of the FBGEMM article's MetaShuffling, which the pages name for
 * avoiding padding: sorted_token_ids holds exactly the T*k pairs, expert by expert, and h
 * and y hold T*k rows in that order; the GEMM tiles are cut at expert boundaries (block b
 * covers rows [block_start[b], block_start[b + 1]) of one expert, at most block_m of them),
 * so a tile's rows past its expert's end are computed but never read or stored.
 * moe_default_plan picks a plan per T; any valid plan gives results equal within rounding
 * (and bitwise reproducible for a fixed plan on a fixed device).
 */
typedef struct {
    int32_t block_m;
    int32_t gemm1_tile;
    int32_t gemm2_tile;
    int32_t split_k;
    int32_t split_k1;
    int32_t split_tail;
    int32_t max_workgroups;
    int32_t split_tail1;
    int32_t ragged;
} moe_plan;

/* Steps of moe_forward, for moe_forward_profiled. */
typedef enum {
    MOE_STAGE_ROUTE = 0, MOE_STAGE_ALIGN = 1, MOE_STAGE_ACT_QUANT = 2, MOE_STAGE_GEMM1 = 3,
    MOE_STAGE_H_QUANT = 4, MOE_STAGE_GEMM2 = 5, MOE_STAGE_REDUCE = 6,
    MOE_STAGE_PROLOGUE = 7,   /* T <= 64 (fp8 or more than 64 experts: 16): route, align
                                 and the activation pass in one launch                  */
    MOE_STAGE_GEMM1_FINISH = 8, /* split_k1 > 1 or split_tail1 > 1: sum of GEMM1's
                                   partials, SiLU * up                                  */
    MOE_STAGE_COUNT = 9
} moe_stage;

/* Static text for a status code [host]. */
const char *moe_status_str(moe_status s);

/* Length of sorted_token_ids for (T, k, E, block_m): T*k + min(E, T*k) * (block_m - 1),
 * rounded up to a multiple of block_m; expert_ids then has capacity / block_m entries.
 * Returns -1 for invalid arguments (T < 0, k < 1, E < 1, block_m < 1).  [host, pure] */
int64_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t block_m);

/*
 * Router top-k (one wavefront per token).
 *  logits       [device] [T, E] bf16 or fp32 (cfg->logits_dtype), 2- / 4-byte aligned.
 *  bias         [device] fp32 [E] or NULL (required for GROUPED_SIGMOID_BIAS).
 *  topk_ids     [device] int32 [T, k] out: expert of each slot, in slot order.
 *  topk_weights [device] fp32 [T, k] out.
 *  cfg          [host].
 */
moe_status moe_route(const moe_route_cfg *cfg, int32_t T, const void *logits, const float *bias,
                     int32_t *topk_ids, float *topk_weights, void *stream);

/*
 * Align / permute (one workgroup; LDS histogram, prefix sum, stable scatter; moe_forward
 * also has a chunked multi-workgroup form for large T*k with identical output).  For the
 * T*k pairs (flat index t*k + j) of topk_ids [device] int32 [T, k], each in [0, E):
 *  expert_counts [E]     number of pairs routed to each expert;
 *  sorted_token_ids [capacity]: expert e owns rows [off_e, off_e + P_e), P_e = c_e rounded
 *        up to a multiple of block_m, off_e = sum of P over lower experts; its pairs' flat
 *        indices in ascending order, then the filler value T*k; rows past sum P are also
 *        T*k;
 *  expert_ids [capacity / block_m]: expert of each block, -1 past the last used block;
 *  num_tokens_post_padded [1]: sum of P_e;
 *  inv_pos [T*k]: row of each pair.
 * block_m in [1, 1024]; E in [1, 256].  A pair whose id lies outside [0, E) is outside the
 * contract: it is dropped (counted nowhere, no row), and nothing is written outside the
 * buffers.  All pointers [device], 4-byte aligned.
 */
moe_status moe_align(int32_t T, int32_t k, int32_t E, int32_t block_m, const int32_t *topk_ids,
                     int32_t *sorted_token_ids, int32_t *expert_ids, int32_t *num_tokens_post_padded,
                     int32_t *expert_counts, int32_t *inv_pos, void *stream);

/* The plan moe_forward uses when given none.  [host, pure] */
moe_status moe_default_plan(const moe_layer *layer, int32_t T, moe_plan *plan);

/* Workspace bytes moe_forward needs for T tokens under `plan` (NULL = default). [host, pure] */
moe_status moe_workspace_bytes(const moe_layer *layer, int32_t T, const moe_plan *plan, size_t *bytes);

/*
 * The layer forward.
 *  layer      [host] struct whose pointers are [device].
 *  hidden     [device] bf16 [T, H], 16-byte aligned.
 *  logits     [device] router logits [T, E] in layer->route.logits_dtype.
 *  out        [device] bf16 [T, H] out, 16-byte aligned.
 *  workspace  [device] at least moe_workspace_bytes(layer, T, plan) bytes, 256-byte aligned;
 *             scratch only, its contents on return are unspecified.
 *  plan       [host] or NULL for moe_default_plan.
 * MOE_ERR_UNSUPPORTED when T*k > 2^24, or when T*H*2 or capacity*I*2 bytes exceed 2^32 - 1
 * (the GEMMs address activation rows with 32-bit offsets).
 */
moe_status moe_forward(const moe_layer *layer, int32_t T, const void *hidden, const void *logits,
                       void *out, void *workspace, size_t workspace_bytes, const moe_plan *plan,
                       void *stream);

/*
 * moe_forward for callers that cannot allocate device memory (code under hipGraph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same steps and results as
 * moe_forward with the same plan, but the workspace is a static device array of
 * MOE_STATIC_WORKSPACE_BYTES that the library holds on each GPU it runs on until the
 * process ends (its address is looked up once per device, on the first call with that
 * device current).  Nothing is allocated or freed.
 *  - MOE_ERR_WORKSPACE_TOO_SMALL, before anything is enqueued or any HIP call, when
 *    moe_workspace_bytes(layer, T, plan) exceeds MOE_STATIC_WORKSPACE_BYTES (128 MiB holds
 *    the small and mid batches under the default plans: Mixtral TP2, Qwen2 fp8, DeepSeek
 *    int4 and Llama-4-Scout up to T = 256).
 *  - Every call on one GPU uses that GPU's one array and leaves its contents there: calls
 *    that overlap on one GPU (two streams, or two host threads without ordering between
 *    their streams) race and give undefined results; the caller orders them.
 * Arguments as moe_forward, without workspace and workspace_bytes.
 */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
moe_status moe_forward_static(const moe_layer *layer, int32_t T, const void *hidden, const void *logits,
                              void *out, const moe_plan *plan, void *stream);

/*
 * moe_forward, with a hipEvent_t recorded on `stream` before each step it launches and one
 * after the last.  events [host] holds n_events >= MOE_STAGE_COUNT + 1 hipEvent_t handles;
 * stages [host] int32 [MOE_STAGE_COUNT] receives the moe_stage of each launched step, and
 * *n_stages their number (events[0 .. *n_stages] are recorded).
 */
moe_status moe_forward_profiled(const moe_layer *layer, int32_t T, const void *hidden,
                                const void *logits, void *out, void *workspace,
                                size_t workspace_bytes, const moe_plan *plan, void *stream,
                                void *const *events, int32_t n_events, int32_t *stages,
                                int32_t *n_stages);

/* Text description of a plan's tiles for `layer` (for logs) into buf [host] of `len`
 * bytes, NUL-terminated.  Returns MOE_ERR_INVALID_ARGUMENT when the plan is not valid for
 * this layer at T tokens. [host, pure] */
moe_status moe_plan_describe(const moe_layer *layer, int32_t T, const moe_plan *plan, char *buf,
                             size_t len);

/* Regions of the moe_forward workspace, for inspecting intermediates in tests. */
typedef enum {
    MOE_WS_TOPK_IDS = 0,      /* int32 [T, k]                                        */
    MOE_WS_TOPK_WEIGHTS = 1,  /* fp32 [T, k]                                         */
    MOE_WS_SORTED_IDS = 2,    /* int32 [capacity] (moe_align's sorted_token_ids); ragged:
                                 [T * k], the pairs only                              */
    MOE_WS_EXPERT_IDS = 3,    /* int32 [capacity / block_m]                          */
    MOE_WS_NUM_POST_PAD = 4,  /* int32 [1]                                           */
    MOE_WS_EXPERT_COUNTS = 5, /* int32 [E]                                           */
    MOE_WS_INV_POS = 6,       /* int32 [T * k] row of each pair (in h and y)          */
    MOE_WS_SCALARS = 7,       /* fp8: [0] amax(x) and [1] amax(h) as fp32 bits, [2] the
                                 activation scale s1, [3] the intermediate scale s2     */
    MOE_WS_X_Q = 8,           /* fp8: E4M3 [T, H] quantised hidden states            */
    MOE_WS_H = 9,             /* [rows, I] SiLU(gate) * up per sorted row: bf16, or fp32
                                 for fp8 weights (its E4M3 code is chosen in fp32); rows =
                                 capacity, or T * k when ragged (also below)            */
    MOE_WS_H_Q = 10,          /* fp8: E4M3 [rows, I] quantised h                     */
    MOE_WS_Y = 11,            /* bf16 [rows, H] weighted expert rows, or with split_k > 1
                                 fp32 [split_k, rows, H] partial sums                 */
    MOE_WS_ALIGN_SCRATCH = 12, /* int32 per-chunk expert histograms of the multi-launch
                                  align (T*k > 65536 only)                            */
    MOE_WS_GEMM1_PARTIALS = 13, /* split_k1 > 1: fp32 [split_k1, rows, 2I] gate (columns
                                   [0, I)) and up ([I, 2I)) partial sums              */
    MOE_WS_GEMM2_TAIL = 14,   /* split_tail > 1: int32 [4] = first sorted row of the split
                                 row blocks, S (0: none split), elements per plane, 0;
                                 then at byte 256 fp32 [S, rows, H] partial sums        */
    MOE_WS_GEMM1_TAIL = 15,   /* split_tail1 > 1: the same for GEMM1, planes fp32
                                 [S, rows, 2I] of gate ([0, I)) and up ([I, 2I)) sums  */
    MOE_WS_BLOCK_START = 16,  /* ragged: int32 [capacity / block_m + 1] first row of each
                                 block, T * k past the last block                    */
    MOE_WS_COUNT = 17
} moe_ws_region;

/* Byte offset of each moe_ws_region in the workspace of moe_forward(layer, T, plan) into
 * offsets [host] int64 [MOE_WS_COUNT] (regions unused by the weight type have size 0).
 * The contents are those left by the last moe_forward with the same arguments, once its
 * stream work has completed. [host, pure] */
moe_status moe_workspace_offsets(const moe_layer *layer, int32_t T, const moe_plan *plan, int64_t *offsets);

/*
 * Grouped GEMM over pre-permuted contiguous per-expert segments: the EP-MoE workload of
 * the aijishu article comparing FBGEMM's MoE grouped GEMM with SGLang's (tokens already
 * grouped by expert; bf16 or fp8 per-tensor operands).  Segment e is rows
 * [off_e, off_e + m_sizes[e]) of X, off_e = m_sizes[0] + ... + m_sizes[e-1]; each of its
 * rows r gets
 *     Y[r, n] = x_scale * w_scale[e] * sum_c X[r, c] * W[e, n, c]      (scales 1 for bf16)
 * with fp32 accumulation, rounded to bf16 once.  Rows of Y past the last segment are not
 * written.  The same grouped-GEMM kernels as moe_forward's GEMM2 (pipelined tiles only):
 * blocks of a tile's height cut at segment ends, the partial last block of a segment
 * computed but not stored.
 */
typedef struct {
    int32_t num_groups;          /* E, 1..1024                                          */
    int32_t N, K;                /* output columns; reduction length                    */
    int32_t dtype;               /* MOE_DT_BF16, or MOE_DT_FP8_E4M3 (X and W as E4M3
                                    codes with per-tensor scales)                       */
    const void *w;               /* [device] W [E, N, K], K contiguous, 16-byte aligned */
    const float *w_scale;        /* [device] fp8: [E] per-expert scales (NULL for bf16) */
} moe_grouped_gemm_desc;

/* The tile moe_grouped_gemm uses for M rows when given tile = -1 (a pipelined tile id of
 * the dtype, listed like the layer's).  MOE_ERR_INVALID_ARGUMENT for an invalid
 * descriptor, MOE_ERR_UNSUPPORTED when no compiled tile divides N and K. [host, pure] */
moe_status moe_grouped_gemm_default_tile(const moe_grouped_gemm_desc *desc, int32_t M, int32_t *tile);

/* Workspace bytes of moe_grouped_gemm for M rows and `tile` (-1: default). [host, pure] */
moe_status moe_grouped_gemm_workspace_bytes(const moe_grouped_gemm_desc *desc, int32_t M, int32_t tile,
                                            size_t *bytes);

/* Enqueue the grouped GEMM on `stream` (no host synchronisation: the sizes stay on the
 * device; graph-capturable).
 *  M          rows of X and Y [host]; the sizes must sum to at most M (rows past M are
 *             never read or written; sizes past it are clamped there, negative ones
 *             read as 0)
 *  x          [device] X [M, K] bf16 or E4M3, 16-byte aligned
 *  x_scale    [device] fp8: the per-tensor activation scale (fp32 scalar); NULL for bf16
 *  m_sizes    [device] int32 [E]
 *  y          [device] Y [M, N] bf16, 16-byte aligned
 *  workspace  [device] at least moe_grouped_gemm_workspace_bytes, 256-byte aligned
 *  tile       a pipelined tile id of the dtype whose BN divides N and BK divides K, or -1
 * Errors: MOE_ERR_INVALID_ARGUMENT (checked before anything is enqueued),
 * MOE_ERR_UNSUPPORTED when M*K bytes of X or N*K bytes of one group's W exceed 2^32 - 1
 * (32-bit row offsets; moe_grouped_gemm_default_tile and _workspace_bytes report it too),
 * MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP. */
moe_status moe_grouped_gemm(const moe_grouped_gemm_desc *desc, int32_t M, const void *x, const float *x_scale,
                            const int32_t *m_sizes, void *y, void *workspace, size_t workspace_bytes,
                            int32_t tile, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
