// moe_api.cpp -- the C ABI of libmoe (declared in include/moe.h): argument checks, plans,
// workspace carving and the stream-ordered launch sequence.  No host synchronisation and no
// allocation anywhere, so moe_forward can be captured into a hipGraph.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../include/moe.h"
#include "kernels.h"
#include "plan_table.h"

namespace moe {

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev < 0 || dev >= 64) dev = 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace moe

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int nbits_for(int E) {
    int b = 0;
    while ((1 << b) < E) b++;
    return b;
}

moe_status check_route(const moe_route_cfg *c) {
    if (!c) return MOE_ERR_INVALID_ARGUMENT;
    const int E = c->num_experts, k = c->top_k;
    if (E < 1 || E > 256 || k < 1 || k > E || k > 64) return MOE_ERR_INVALID_ARGUMENT;
    if (c->logits_dtype != MOE_DT_BF16 && c->logits_dtype != MOE_DT_FP32) return MOE_ERR_INVALID_ARGUMENT;
    if (c->renormalize != 0 && c->renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (c->kind == MOE_ROUTE_GROUPED_SIGMOID_BIAS) {
        const int ng = c->n_group, tg = c->topk_group;
        if (ng < 1 || ng > 64 || E % ng != 0 || tg < 1 || tg > ng) return MOE_ERR_INVALID_ARGUMENT;
        if (k > tg * (E / ng)) return MOE_ERR_INVALID_ARGUMENT;
    } else if (c->kind != MOE_ROUTE_SOFTMAX && c->kind != MOE_ROUTE_SIGMOID) {
        return MOE_ERR_INVALID_ARGUMENT;
    }
    return MOE_OK;
}

moe_status check_layer(const moe_layer *L) {
    if (!L) return MOE_ERR_INVALID_ARGUMENT;
    moe_status st = check_route(&L->route);
    if (st != MOE_OK) return st;
    if (L->E != L->route.num_experts) return MOE_ERR_INVALID_ARGUMENT;
    if (L->H < 128 || L->I < 128 || L->H % 128 || L->I % 128) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)L->H * L->I > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
    if (!L->w13 || !L->w2 || !aligned(L->w13, 16) || !aligned(L->w2, 16)) return MOE_ERR_INVALID_ARGUMENT;
    switch (L->weight_dtype) {
    case MOE_DT_BF16:
        break;
    case MOE_DT_FP8_E4M3:
        if (!L->w13_scale || !L->w2_scale || !aligned(L->w13_scale, 4) || !aligned(L->w2_scale, 4))
            return MOE_ERR_INVALID_ARGUMENT;
        break;
    case MOE_DT_INT4_G128:
        if (!L->w13_s || !L->w13_z || !L->w2_s || !L->w2_z) return MOE_ERR_INVALID_ARGUMENT;
        if (!aligned(L->w13_s, 4) || !aligned(L->w13_z, 4) || !aligned(L->w2_s, 4) || !aligned(L->w2_z, 4))
            return MOE_ERR_INVALID_ARGUMENT;
        break;
    default:
        return MOE_ERR_INVALID_ARGUMENT;
    }
    if (L->route.kind == MOE_ROUTE_GROUPED_SIGMOID_BIAS && !L->correction_bias) return MOE_ERR_INVALID_ARGUMENT;
    if (L->correction_bias && !aligned(L->correction_bias, 4)) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// GEMM1's K splits (0 and 1 both mean none)
int split1(const moe_plan *p) { return p->split_k1 > 1 ? p->split_k1 : 1; }

// A plan is valid when both tiles exist for the weight type, share the block height, and
// tile the layer's dimensions exactly.
moe_status check_plan(const moe_layer *L, const moe_plan *p, TileInfo *t1, TileInfo *t2) {
    if (!p) return MOE_ERR_INVALID_ARGUMENT;
    const int wd = L->weight_dtype;
    if (p->gemm1_tile < 0 || p->gemm2_tile < 0 || !gemm_tile_info(wd, p->gemm1_tile, t1) ||
        !gemm_tile_info(wd, p->gemm2_tile, t2))
        return MOE_ERR_INVALID_ARGUMENT;
    if (p->block_m != t1->BM || p->block_m != t2->BM) return MOE_ERR_INVALID_ARGUMENT;
    if (p->split_k < 1 || p->split_k > 16) return MOE_ERR_INVALID_ARGUMENT;
    const int s1 = split1(p);
    if (p->split_k1 < 0 || s1 > 16) return MOE_ERR_INVALID_ARGUMENT;
    // GEMM1 split K: the small-T tiles only, each split a whole number of K steps
    if (s1 > 1 && (t1->BM > 32 || L->H % (t1->BK * s1))) return MOE_ERR_INVALID_ARGUMENT;
    // int4: the pipelined tiles pass h between the GEMMs as bf16 in the nibble order, the
    // register-staged ones in the natural order, so both GEMMs must be of one kind
    if (wd == MOE_DT_INT4_G128 && (t1->stages > 0) != (t2->stages > 0)) return MOE_ERR_INVALID_ARGUMENT;
    // GEMM1: K = H, output columns I (each tile covers BN/2 gate and BN/2 up rows, and each
    // wave an equal number of gate and up fragments)
    if (L->H % t1->BK || L->I % (t1->BN / 2)) return MOE_ERR_INVALID_ARGUMENT;
    if ((t1->BN / t1->WN) % (2 * t1->mfma)) return MOE_ERR_INVALID_ARGUMENT;
    // GEMM2: K = I split split_k ways, output columns H
    if (L->I % (t2->BK * p->split_k) || L->H % t2->BN) return MOE_ERR_INVALID_ARGUMENT;
    // split tail: the unsplit GEMM2 of the pipelined bf16 / fp8 tiles
    if (p->split_tail < 0 || p->split_tail > 16 || p->max_workgroups < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (p->split_tail > 1 && (p->split_k != 1 || t2->stages == 0 || wd == MOE_DT_INT4_G128))
        return MOE_ERR_INVALID_ARGUMENT;
    // GEMM1's split tail: the unsplit GEMM1 of the pipelined bf16 / fp8 tiles
    if (p->split_tail1 < 0 || p->split_tail1 > 16) return MOE_ERR_INVALID_ARGUMENT;
    if (p->split_tail1 > 1 && (s1 > 1 || t1->stages == 0 || wd == MOE_DT_INT4_G128)) return MOE_ERR_INVALID_ARGUMENT;
    if (p->ragged != 0 && p->ragged != 1) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// GEMM2's / GEMM1's split tail on / the tiles x splits their planes hold
bool split_tail(const moe_plan *p) { return p->split_tail > 1; }
bool split_tail1(const moe_plan *p) { return p->split_tail1 > 1; }
constexpr int kTailUnits = 256;
constexpr size_t kTailInfoBytes = 256;

// the one-launch prologue (route, align, activation pass) takes batches up to this size:
// its 16 waves route the tokens in turn, which pays while a token's routing is short (up
// to 64 experts and top-2: Mixtral T=32 265 against 272 us); longer routing keeps one
// wave per token beyond 16 tokens (DeepSeek's grouped top-8 of 256, T=64: 773 against 813
// us; Qwen2's top-8 of 64, T=32: the prologue takes 20 us and the layer 4% longer); the
// fp8 pass holds the batch in one workgroup's registers
int prologue_max_t(const moe_layer *L) {
    const int t = L->E <= 64 && L->route.top_k <= 2 ? kPrologueMaxT : kPrologueMaxTLongRoute;
    if (L->weight_dtype == MOE_DT_FP8_E4M3) return (int)std::min<int64_t>(t, kPrologueFp8Elems / L->H);
    return t;
}

struct Workspace {
    size_t ids, weights, sorted, eids, npp, counts, inv_pos, scal, xq, h, hq, y, align_scratch, g1p, tail, tail1,
        blk_start, total;
    int64_t cap;
    int64_t rows;   // rows of h, y and the K-split planes: cap, or T*k with no padding
};

// scal words: [0] amax(x) bits, [1] amax(h) bits, [2] s1, [3] s2
constexpr int kScalarWords = 4;

// int4 with the pipelined tiles: GEMM1 reads the hidden states as bf16 permuted into the
// order the kernel unpacks nibbles
bool perm_activations(const moe_layer *L, const moe_plan *p) {
    TileInfo t;
    return L->weight_dtype == MOE_DT_INT4_G128 && gemm_tile_info(L->weight_dtype, p->gemm1_tile, &t) && t.stages > 0;
}

// top-1 routing without a K split: each token owns one row of the down projection, which
// GEMM2 writes straight into the output (no unpermute-and-reduce pass)
bool direct_output(const moe_layer *L, const moe_plan *p) { return L->route.top_k == 1 && p->split_k == 1; }

Workspace layout(const moe_layer *L, int T, const moe_plan *p) {
    Workspace w{};
    const int k = L->route.top_k, E = L->E;
    const int64_t pairs = (int64_t)T * k;
    w.cap = moe_align_capacity(T, k, E, p->block_m);
    w.rows = p->ragged ? pairs : w.cap;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + bytes, kAlign);
        return at;
    };
    w.ids = take(pairs * 4);
    w.weights = take(pairs * 4);
    w.sorted = take((p->ragged ? pairs : w.cap) * 4);
    w.eids = take(w.cap / p->block_m * 4);
    w.npp = take(4);
    w.counts = take((size_t)E * 4);
    w.inv_pos = take(pairs * 4);
    w.scal = take(kScalarWords * 4);
    const bool fp8 = L->weight_dtype == MOE_DT_FP8_E4M3;
    w.xq = take(fp8 ? (size_t)T * L->H : perm_activations(L, p) ? (size_t)T * L->H * 2 : 0);
    w.h = take((size_t)w.rows * L->I * (fp8 ? 4 : 2));
    w.hq = take(fp8 ? (size_t)w.rows * L->I : 0);
    w.y = take(direct_output(L, p) ? 0
               : p->split_k > 1 ? (size_t)p->split_k * w.rows * L->H * 4 : (size_t)w.rows * L->H * 2);
    w.align_scratch = take((size_t)align_scratch_bytes(pairs, E));
    w.g1p = take(split1(p) > 1 ? (size_t)split1(p) * w.rows * 2 * L->I * 4 : 0);
    TileInfo t1{}, t2{};
    gemm_tile_info(L->weight_dtype, p->gemm1_tile, &t1);
    gemm_tile_info(L->weight_dtype, p->gemm2_tile, &t2);
    w.tail = take(split_tail(p) ? kTailInfoBytes + (size_t)kTailUnits * t2.BM * t2.BN * 4 : 0);
    // a GEMM1 tile's unit covers BN / 2 gate and BN / 2 up columns: BM x BN fp32 as well
    w.tail1 = take(split_tail1(p) ? kTailInfoBytes + (size_t)kTailUnits * t1.BM * t1.BN * 4 : 0);
    w.blk_start = take(p->ragged ? (size_t)(w.cap / p->block_m + 1) * 4 : 0);
    w.total = o;
    return w;
}

RouteArgs route_args(const moe_route_cfg *c, int T, const void *logits, const float *bias, int32_t *ids,
                     float *weights) {
    RouteArgs a{};
    a.T = T;
    a.E = c->num_experts;
    a.k = c->top_k;
    a.kind = c->kind;
    a.renorm = c->renormalize;
    a.n_group = c->n_group;
    a.topk_group = c->topk_group;
    a.scale = c->routed_scaling;
    a.logits_bf16 = c->logits_dtype == MOE_DT_BF16;
    a.logits = logits;
    a.bias = c->kind == MOE_ROUTE_SOFTMAX ? nullptr : bias;
    a.ids = ids;
    a.weights = weights;
    return a;
}

// The stream-ordered sequence of moe_forward; events (optional) are recorded before each
// step and after the last.
moe_status forward_impl(const moe_layer *L, int32_t T, const void *hidden, const void *logits, void *out,
                        void *workspace, size_t ws_bytes, const moe_plan *plan_in, hipStream_t stream,
                        void *const *events, int32_t n_events, int32_t *stages, int32_t *n_stages) {
    moe_status st = check_layer(L);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
    moe_plan plan;
    if (plan_in) plan = *plan_in;
    else if ((st = moe_default_plan(L, T, &plan)) != MOE_OK) return st;
    TileInfo t1, t2;
    if ((st = check_plan(L, &plan, &t1, &t2)) != MOE_OK) return st;
    if (events && n_events < MOE_STAGE_COUNT + 1) return MOE_ERR_INVALID_ARGUMENT;
    if (events && (!stages || !n_stages)) return MOE_ERR_INVALID_ARGUMENT;
    if (n_stages) *n_stages = 0;
    if (T == 0) return MOE_OK;
    if ((int64_t)T * L->route.top_k > (int64_t)1 << 24) return MOE_ERR_UNSUPPORTED;
    if (!hidden || !logits || !out || !workspace) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(hidden, 16) || !aligned(out, 16) || !aligned(workspace, kAlign)) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(logits, L->route.logits_dtype == MOE_DT_BF16 ? 2 : 4)) return MOE_ERR_INVALID_ARGUMENT;
    const Workspace w = layout(L, T, &plan);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    // the GEMMs address A rows with 32-bit byte offsets from the operand's base
    if ((int64_t)T * L->H * 2 > (int64_t)UINT32_MAX || w.cap * (int64_t)L->I * 2 > (int64_t)UINT32_MAX)
        return MOE_ERR_UNSUPPORTED;

    char *ws = (char *)workspace;
    int32_t *ids = (int32_t *)(ws + w.ids), *sorted = (int32_t *)(ws + w.sorted);
    int32_t *eids = (int32_t *)(ws + w.eids), *npp = (int32_t *)(ws + w.npp);
    int32_t *counts = (int32_t *)(ws + w.counts), *inv_pos = (int32_t *)(ws + w.inv_pos);
    float *topk_w = (float *)(ws + w.weights);
    uint32_t *scal = (uint32_t *)(ws + w.scal);
    const bool fp8 = L->weight_dtype == MOE_DT_FP8_E4M3;
    const int k = L->route.top_k, H = L->H, I = L->I, E = L->E;
    const int pairs = T * k;
    int nst = 0;
    auto mark = [&](moe_stage s) -> hipError_t {
        if (!events) return hipSuccess;
        stages[nst] = s;
        return hipEventRecord((hipEvent_t)events[nst++], stream);
    };
    auto fail = [&](hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; };
    hipError_t err;

    RouteArgs ra = route_args(&L->route, T, logits, L->correction_bias, ids, topk_w);
    int32_t *blk_start = plan.ragged ? (int32_t *)(ws + w.blk_start) : nullptr;
    AlignArgs aa{T, k, E, plan.block_m, nbits_for(E), w.cap, ids, sorted, eids, npp, counts, inv_pos, blk_start};
    const void *a1 = hidden;
    const bool prologue = T <= prologue_max_t(L);
    if (prologue) {
        // 1-3 in one launch for a small batch
        if ((err = mark(MOE_STAGE_PROLOGUE)) != hipSuccess) return MOE_ERR_HIP;
        PrologueArgs pa{};
        pa.route = ra;
        pa.align = aa;
        pa.act = fp8 ? PROLOGUE_ACT_FP8 : perm_activations(L, &plan) ? PROLOGUE_ACT_BF16_PERM : PROLOGUE_ACT_NONE;
        pa.x = (const uint16_t *)hidden;
        pa.n = (int64_t)T * H;
        pa.xq = (uint8_t *)(ws + w.xq);
        pa.xperm = (uint16_t *)(ws + w.xq);
        pa.x_amax = &scal[0];
        pa.x_scale = (float *)&scal[2];
        pa.h_amax = &scal[1];
        if ((err = launch_prologue(pa, stream)) != hipSuccess) return fail(err);
        if (pa.act != PROLOGUE_ACT_NONE) a1 = ws + w.xq;
    } else {
        // 1. route (its first workgroup also clears the scratch words)
        if ((err = mark(MOE_STAGE_ROUTE)) != hipSuccess) return MOE_ERR_HIP;
        ra.zero_ptr = scal;
        ra.zero_n = kScalarWords;
        // fp8: the route's workgroups also take the largest |x| of their tokens, one word each,
        // in h's space (free until GEMM1 writes h); the quantisation reduces them
        uint32_t *x_parts = fp8 ? (uint32_t *)(ws + w.h) : nullptr;
        // int4: the route's waves also write their tokens' rows in the GEMM's nibble order
        const bool perm = !fp8 && perm_activations(L, &plan);
        if (fp8 || perm) {
            ra.x = (const uint16_t *)hidden;
            ra.x_cols = H;
            ra.x_parts = x_parts;
            ra.x_perm = perm ? (uint16_t *)(ws + w.xq) : nullptr;
        }
        if ((err = launch_route(ra, stream)) != hipSuccess) return fail(err);

        // 2. align
        if ((err = mark(MOE_STAGE_ALIGN)) != hipSuccess) return MOE_ERR_HIP;
        int32_t *align_scratch = align_scratch_bytes(pairs, E) ? (int32_t *)(ws + w.align_scratch) : nullptr;
        if ((err = launch_align(aa, align_scratch, stream)) != hipSuccess) return fail(err);

        // 3. fp8: quantise the hidden states with one dynamic scale
        if (fp8) {
            if ((err = mark(MOE_STAGE_ACT_QUANT)) != hipSuccess) return MOE_ERR_HIP;
            QuantArgs q{hidden, 0, (uint8_t *)(ws + w.xq), T, H, &scal[0], (float *)&scal[2], nullptr, nullptr, pairs,
                        x_parts, (T + 3) / 4, &scal[0]};
            if ((err = launch_quant(q, stream)) != hipSuccess) return fail(err);
            a1 = ws + w.xq;
        } else if (perm) {
            // int4: the hidden states in the order the kernel unpacks nibbles (written by the
            // route above)
            if ((err = mark(MOE_STAGE_ACT_QUANT)) != hipSuccess) return MOE_ERR_HIP;
            a1 = ws + w.xq;
        }
    }

    // 4. GEMM1: gate/up with SiLU * up
    if ((err = mark(MOE_STAGE_GEMM1)) != hipSuccess) return MOE_ERR_HIP;
    const int wd = L->weight_dtype;
    const size_t b13_row = wd == MOE_DT_FP8_E4M3 ? H : wd == MOE_DT_INT4_G128 ? H / 2 : (size_t)H * 2;
    const size_t b2_row = wd == MOE_DT_FP8_E4M3 ? I : wd == MOE_DT_INT4_G128 ? I / 2 : (size_t)I * 2;
    GemmArgs g{};
    g.A = a1;
    g.lda = H;
    g.B = L->w13;
    g.ldb = (int64_t)b13_row;
    g.b_expert_stride = (int64_t)b13_row * 2 * I;
    g.bs = L->w13_s;
    g.bz = L->w13_z;
    g.sz_expert_stride = (int64_t)2 * I * (H / 128);
    g.C = ws + w.h;
    g.ldc = I;
    g.sorted = sorted;
    g.eids = eids;
    g.npp = npp;
    g.blk_start = blk_start;
    g.topk_w = topk_w;
    g.K = H;
    g.N = I;
    g.I = I;
    g.top_k = k;
    g.pairs = pairs;
    g.split = 1;
    g.ksplit = H;
    g.a_scale = (const float *)&scal[2];
    g.b_scale = L->w13_scale;
    g.amax_out = fp8 ? &scal[1] : nullptr;
    // weight streaming (about one block of rows per expert): no two tiles share operands,
    // so stagger their K walks across DRAM channels
    g.rotate_k = (int64_t)pairs <= (int64_t)E * plan.block_m;
    const int64_t mblocks_max = w.cap / plan.block_m;
    const int s1 = split1(&plan);
    if (s1 > 1) {   // fp32 partial planes of gate and up, finished below
        g.C = ws + w.g1p;
        g.ldc = 2 * (int64_t)I;
        g.partial_stride = w.rows * 2 * (int64_t)I;
        g.split = s1;
        g.ksplit = H / s1;
        g.amax_out = nullptr;
    }
    // GEMM1's split tail: fp32 planes of the split row blocks, finished below
    int32_t *tail1_info = split_tail1(&plan) ? (int32_t *)(ws + w.tail1) : nullptr;
    g.tail_split = split_tail1(&plan) ? plan.split_tail1 : 0;
    g.tail_cap = kTailUnits;
    g.tail_P = split_tail1(&plan) ? (float *)(ws + w.tail1 + kTailInfoBytes) : nullptr;
    g.tail_info = tail1_info;
    // persistent grids: at most max_workgroups workgroups when the plan caps them
    auto grid_cap = [&](int64_t tiles) {
        return plan.max_workgroups > 0 ? std::min<int64_t>(tiles, plan.max_workgroups) : tiles;
    };
    if ((err = launch_gemm(wd, plan.gemm1_tile, GEMM_GATE_UP, s1 > 1, g,
                           grid_cap(mblocks_max * (I / (t1.BN / 2)) * s1), stream)) != hipSuccess)
        return fail(err);
    // a tiny fp8 batch finishes a split GEMM1 and quantises h in one launch (one workgroup:
    // worth it while the partial sums it reads are a few tens of KB)
    const bool finish_quant = fp8 && s1 > 1 && (int64_t)pairs * I * s1 <= 32768;
    if (s1 > 1) {
        if ((err = mark(MOE_STAGE_GEMM1_FINISH)) != hipSuccess) return MOE_ERR_HIP;
        GateUpFinishArgs f{(const float *)(ws + w.g1p), w.rows * 2 * (int64_t)I, s1, I, sorted, npp, pairs, ws + w.h,
                           fp8 ? GATE_UP_H_F32 : perm_activations(L, &plan) ? GATE_UP_H_BF16_PERM : GATE_UP_H_BF16,
                           fp8 ? &scal[1] : nullptr, nullptr, plan.ragged};
        err = finish_quant ? launch_gate_up_finish_quant(f, inv_pos, (uint8_t *)(ws + w.hq), (float *)&scal[3], stream)
                           : launch_gate_up_finish(f, w.rows, stream);
        if (err != hipSuccess) return fail(err);
    } else if (split_tail1(&plan)) {
        // the split row blocks' h (GEMM1 recorded the rows and planes; none: an empty pass)
        if ((err = mark(MOE_STAGE_GEMM1_FINISH)) != hipSuccess) return MOE_ERR_HIP;
        GateUpFinishArgs f{(const float *)(ws + w.tail1 + kTailInfoBytes), 0, 0, I, sorted, npp, pairs, ws + w.h,
                           fp8 ? GATE_UP_H_F32 : GATE_UP_H_BF16, fp8 ? &scal[1] : nullptr, tail1_info, plan.ragged};
        // at most kTailUnits / (column tiles) row blocks are split
        const int64_t tail_rows = (int64_t)kTailUnits / (I / (t1.BN / 2)) * plan.block_m;
        if ((err = launch_gate_up_finish(f, std::max<int64_t>(tail_rows, plan.block_m), stream)) != hipSuccess)
            return fail(err);
    }

    // 5. fp8: quantise h with its dynamic scale
    const void *a2 = ws + w.h;
    if (fp8 && finish_quant) {
        a2 = ws + w.hq;
    } else if (fp8) {
        if ((err = mark(MOE_STAGE_H_QUANT)) != hipSuccess) return MOE_ERR_HIP;
        // padded: the rows of the layout up to its end, filler rows zeroed; ragged: every row a pair
        QuantArgs q = plan.ragged ? QuantArgs{ws + w.h, 1, (uint8_t *)(ws + w.hq), pairs, I, &scal[1], (float *)&scal[3],
                                              nullptr, nullptr, pairs}
                                  : QuantArgs{ws + w.h, 1, (uint8_t *)(ws + w.hq), w.cap, I, &scal[1], (float *)&scal[3],
                                              sorted, npp, pairs};
        if ((err = launch_quant(q, stream)) != hipSuccess) return fail(err);
        a2 = ws + w.hq;
    }

    // 6. GEMM2: down projection times the top-k weight
    if ((err = mark(MOE_STAGE_GEMM2)) != hipSuccess) return MOE_ERR_HIP;
    GemmArgs d = g;
    d.A = a2;
    d.lda = I;
    d.B = L->w2;
    d.ldb = (int64_t)b2_row;
    d.b_expert_stride = (int64_t)b2_row * H;
    d.bs = L->w2_s;
    d.bz = L->w2_z;
    d.sz_expert_stride = (int64_t)H * (I / 128);
    const bool direct = direct_output(L, &plan);
    d.C = direct ? out : (void *)(ws + w.y);
    d.ldc = H;
    d.out_by_pair = direct;
    d.partial_stride = w.rows * (int64_t)H;
    d.K = I;
    d.N = H;
    d.split = plan.split_k;
    d.ksplit = I / plan.split_k;
    d.a_scale = (const float *)&scal[3];
    d.b_scale = L->w2_scale;
    d.amax_out = nullptr;
    int32_t *tail_info = split_tail(&plan) ? (int32_t *)(ws + w.tail) : nullptr;
    float *tail_P = split_tail(&plan) ? (float *)(ws + w.tail + kTailInfoBytes) : nullptr;
    d.tail_split = split_tail(&plan) ? plan.split_tail : 0;
    d.tail_cap = kTailUnits;
    d.tail_P = tail_P;
    d.tail_info = tail_info;
    const ReduceArgs r{ws + w.y, w.rows * (int64_t)H, plan.split_k > 1 ? plan.split_k : 0, inv_pos, (uint16_t *)out,
                       T, k, H, tail_info, tail_P, direct ? 1 : 0};
    if ((err = launch_gemm(wd, plan.gemm2_tile, GEMM_DOWN, plan.split_k > 1, d,
                           grid_cap(mblocks_max * (H / t2.BN) * plan.split_k), stream)) != hipSuccess)
        return fail(err);

    // 7. unpermute and reduce (top-1 without a split: GEMM2 wrote the output already, but
    //    for the rows of a split tail)
    if (!direct || split_tail(&plan)) {
        if ((err = mark(MOE_STAGE_REDUCE)) != hipSuccess) return MOE_ERR_HIP;
        if ((err = launch_reduce(r, stream)) != hipSuccess) return fail(err);
    }
    if (events) {
        if (hipEventRecord((hipEvent_t)events[nst], stream) != hipSuccess) return MOE_ERR_HIP;
        *n_stages = nst;
    }
    return MOE_OK;
}

// ---- grouped GEMM over contiguous segments ----------------------------------------

constexpr int kMaxGroups = 1024;   // the segment layout runs in one 1024-thread workgroup

moe_status check_grouped(const moe_grouped_gemm_desc *d, int32_t tile, TileInfo *t) {
    if (!d) return MOE_ERR_INVALID_ARGUMENT;
    if (d->num_groups < 1 || d->num_groups > kMaxGroups || d->N < 1 || d->K < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (d->dtype != MOE_DT_BF16 && d->dtype != MOE_DT_FP8_E4M3) return MOE_ERR_INVALID_ARGUMENT;
    if (!d->w || !aligned(d->w, 16)) return MOE_ERR_INVALID_ARGUMENT;
    if (d->dtype == MOE_DT_FP8_E4M3 && (!d->w_scale || !aligned(d->w_scale, 4))) return MOE_ERR_INVALID_ARGUMENT;
    // the pipelined tiles only (they gather A rows through the layout)
    if (tile < 0 || !gemm_tile_info(d->dtype, tile, t) || t->stages == 0) return MOE_ERR_INVALID_ARGUMENT;
    if (d->N % t->BN || d->K % t->BK || (t->BM & (t->BM - 1))) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// Default tile by rows per group r = M / E: narrow blocks while the weights stream, wider
// tiles as the products grow (from timing every tile on the Qwen2-57B TP4 w13 shape,
// M = 8..32768 rows, on MI355X).
int32_t grouped_default_tile(const moe_grouped_gemm_desc *d, int32_t M) {
    const double r = (double)M / d->num_groups;
    static const int bf16[][2] = {{24, 9}, {96, 11}, {384, 22}, {1 << 30, 26}};
    static const int fp8[][2] = {{24, 9}, {96, 10}, {1 << 30, 16}, {1 << 30, 16}};
    const int (*rows)[2] = d->dtype == MOE_DT_FP8_E4M3 ? fp8 : bf16;
    TileInfo t;
    int first = 0;
    while (first < 3 && r > rows[first][0]) first++;
    for (int dd = 0; dd < 8; dd++) {   // the row's tile, else the nearest that tiles N and K
        const int i = dd % 2 == 0 ? first + dd / 2 : first - (dd + 1) / 2;
        if (i < 0 || i > 3) continue;
        if (check_grouped(d, rows[i][1], &t) == MOE_OK) return rows[i][1];
    }
    for (int g = 0; g < 64; g++)
        if (check_grouped(d, g, &t) == MOE_OK) return g;
    return -1;
}

// The GEMM addresses a row of one group's weight matrix with a 32-bit byte offset from the
// group's base: N * K elements must fit that range.
moe_status check_grouped_size(const moe_grouped_gemm_desc *d) {
    if (!d || d->N < 1 || d->K < 1) return MOE_ERR_INVALID_ARGUMENT;
    const int64_t ebytes = d->dtype == MOE_DT_FP8_E4M3 ? 1 : 2;
    return (int64_t)d->N * d->K * ebytes > (int64_t)UINT32_MAX ? MOE_ERR_UNSUPPORTED : MOE_OK;
}

struct GroupedWorkspace {
    size_t sorted, eids, npp, total;
    int64_t cap;
};

GroupedWorkspace grouped_layout(const moe_grouped_gemm_desc *d, int32_t M, int BM) {
    GroupedWorkspace w{};
    w.cap = moe_align_capacity(M, 1, d->num_groups, BM);
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = round_up(o + bytes, kAlign);
        return at;
    };
    w.sorted = take((size_t)w.cap * 4);
    w.eids = take((size_t)w.cap / BM * 4);
    w.npp = take(4);
    w.total = o;
    return w;
}

// ---- the workspace of moe_forward_static --------------------------------------------------

// Device memory the library holds for callers that cannot allocate: one array per GPU (each
// device that loads the library gets its own copy at its own address).  In host code this
// name is only a stand-in for the symbol: kernels are given the device address that
// hipGetSymbolAddress returns for the current device, never the name itself.
static __device__ __align__(256) char scratch[MOE_STATIC_WORKSPACE_BYTES];

// The device address of `scratch` on the current device, looked up on the first call per
// device (with that device current) and kept; null if the lookup fails.
void *static_workspace() {
    static std::atomic<void *> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev].store(p, std::memory_order_release);   // the same value from every thread
    }
    return p;
}

}  // namespace

extern "C" {

const char *moe_status_str(moe_status s) {
    switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

int64_t moe_align_capacity(int32_t T, int32_t k, int32_t E, int32_t block_m) {
    if (T < 0 || k < 1 || E < 1 || block_m < 1) return -1;
    const int64_t pairs = (int64_t)T * k;
    const int64_t used = std::min<int64_t>(pairs, E);
    const int64_t cap = pairs + used * (block_m - 1);
    return (cap + block_m - 1) / block_m * block_m;
}

moe_status moe_route(const moe_route_cfg *cfg, int32_t T, const void *logits, const float *bias,
                     int32_t *topk_ids, float *topk_weights, void *stream) {
    moe_status st = check_route(cfg);
    if (st != MOE_OK) return st;
    if (T < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (cfg->kind == MOE_ROUTE_GROUPED_SIGMOID_BIAS && !bias) return MOE_ERR_INVALID_ARGUMENT;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights) return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned(logits, cfg->logits_dtype == MOE_DT_BF16 ? 2 : 4) || !aligned(topk_ids, 4) ||
        !aligned(topk_weights, 4) || (bias && !aligned(bias, 4)))
        return MOE_ERR_INVALID_ARGUMENT;
    RouteArgs a = route_args(cfg, T, logits, bias, topk_ids, topk_weights);
    return launch_route(a, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_align(int32_t T, int32_t k, int32_t E, int32_t block_m, const int32_t *topk_ids,
                     int32_t *sorted_token_ids, int32_t *expert_ids, int32_t *num_tokens_post_padded,
                     int32_t *expert_counts, int32_t *inv_pos, void *stream) {
    if (T < 0 || k < 1 || E < 1 || E > 256 || block_m < 1 || block_m > 1024) return MOE_ERR_INVALID_ARGUMENT;
    if ((int64_t)T * k > (int64_t)1 << 24) return MOE_ERR_UNSUPPORTED;
    if (T == 0) return MOE_OK;
    const int32_t *ptrs[] = {topk_ids, sorted_token_ids, expert_ids, num_tokens_post_padded, expert_counts, inv_pos};
    for (const int32_t *p : ptrs)
        if (!p || !aligned(p, 4)) return MOE_ERR_INVALID_ARGUMENT;
    AlignArgs a{T, k, E, block_m, nbits_for(E), moe_align_capacity(T, k, E, block_m), topk_ids, sorted_token_ids,
                expert_ids, num_tokens_post_padded, expert_counts, inv_pos};
    return launch_align(a, nullptr, (hipStream_t)stream) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status moe_default_plan(const moe_layer *layer, int32_t T, moe_plan *plan) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (T < 0 || !plan) return MOE_ERR_INVALID_ARGUMENT;
    // The table measured by the tuner (plan_table.h, per layer shape and batch size): a tuned
    // shape takes the plan of its tuned T nearest to T (on a log scale, the smaller on a tie);
    // any other layer the plan of the tuned point of its weight type whose rows per expert
    // are nearest to its own (T k / E, log scale) among those valid for it; else any valid plan.
    const TunedPlan *best = nullptr;
    double bd = 0;
    const double lt = std::log2((double)std::max(T, 1));
    for (const TunedPlan &t : kTunedPlans) {
        if (t.wdtype != layer->weight_dtype || t.E != layer->E || t.k != layer->route.top_k || t.H != layer->H ||
            t.I != layer->I)
            continue;
        const double d = std::fabs(std::log2((double)t.T) - lt);
        if (!best || d < bd || (d == bd && t.T < best->T)) { best = &t; bd = d; }
    }
    auto as_plan = [](const TunedPlan &t) {
        return moe_plan{t.block_m, t.gemm1_tile, t.gemm2_tile, t.split_k, t.split_k1, t.split_tail, t.max_workgroups,
                        t.split_tail1, t.ragged};
    };
    TileInfo t1, t2;
    if (best) {
        moe_plan p = as_plan(*best);
        if (check_plan(layer, &p, &t1, &t2) == MOE_OK) {
            *plan = p;
            return MOE_OK;
        }
    }
    const double lr = std::log2(std::max((double)T * layer->route.top_k / layer->E, 1.0 / 64));
    bool found = false;
    for (const TunedPlan &t : kTunedPlans) {
        if (t.wdtype != layer->weight_dtype) continue;
        moe_plan p = as_plan(t);
        if (check_plan(layer, &p, &t1, &t2) != MOE_OK) continue;
        const double d = std::fabs(std::log2((double)t.T * t.k / t.E) - lr);
        if (!found || d < bd) { *plan = p; bd = d; found = true; }
    }
    if (found) return MOE_OK;
    for (int bm : {16, 32, 64, 128, 256})
        for (int g = 0; g < 64; g++) {
            moe_plan p{bm, g, g, 1, 1};
            if (check_plan(layer, &p, &t1, &t2) == MOE_OK) {
                *plan = p;
                return MOE_OK;
            }
        }
    return MOE_ERR_UNSUPPORTED;
}

moe_status moe_workspace_bytes(const moe_layer *layer, int32_t T, const moe_plan *plan, size_t *bytes) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (T < 0 || !bytes) return MOE_ERR_INVALID_ARGUMENT;
    moe_plan p;
    if (plan) p = *plan;
    else if ((st = moe_default_plan(layer, T, &p)) != MOE_OK) return st;
    TileInfo t1, t2;
    if ((st = check_plan(layer, &p, &t1, &t2)) != MOE_OK) return st;
    *bytes = layout(layer, T, &p).total;
    return MOE_OK;
}

moe_status moe_forward(const moe_layer *layer, int32_t T, const void *hidden, const void *logits, void *out,
                       void *workspace, size_t workspace_bytes, const moe_plan *plan, void *stream) {
    return forward_impl(layer, T, hidden, logits, out, workspace, workspace_bytes, plan, (hipStream_t)stream,
                        nullptr, 0, nullptr, nullptr);
}

moe_status moe_forward_static(const moe_layer *layer, int32_t T, const void *hidden, const void *logits, void *out,
                              const moe_plan *plan, void *stream) {
    // every size check first, without touching the device
    size_t need = 0;
    moe_status st = moe_workspace_bytes(layer, T, plan, &need);
    if (st != MOE_OK) return st;
    if (need > MOE_STATIC_WORKSPACE_BYTES) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (T == 0) return MOE_OK;
    void *ws = static_workspace();
    if (!ws) return MOE_ERR_HIP;
    return forward_impl(layer, T, hidden, logits, out, ws, MOE_STATIC_WORKSPACE_BYTES, plan, (hipStream_t)stream,
                        nullptr, 0, nullptr, nullptr);
}

moe_status moe_forward_profiled(const moe_layer *layer, int32_t T, const void *hidden, const void *logits,
                                void *out, void *workspace, size_t workspace_bytes, const moe_plan *plan,
                                void *stream, void *const *events, int32_t n_events, int32_t *stages,
                                int32_t *n_stages) {
    if (!events) return MOE_ERR_INVALID_ARGUMENT;
    return forward_impl(layer, T, hidden, logits, out, workspace, workspace_bytes, plan, (hipStream_t)stream,
                        events, n_events, stages, n_stages);
}

moe_status moe_plan_describe(const moe_layer *layer, int32_t T, const moe_plan *plan, char *buf, size_t len) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (T < 0 || !plan || !buf || len == 0) return MOE_ERR_INVALID_ARGUMENT;
    TileInfo t1, t2;
    if ((st = check_plan(layer, plan, &t1, &t2)) != MOE_OK) return st;
    std::snprintf(buf, len,
                  "block_m=%d gemm1=%d[BM%d BN%d BK%d waves%dx%d stages%d mfma%d] gemm2=%d[BM%d BN%d BK%d "
                  "waves%dx%d stages%d mfma%d] split_k=%d split_k1=%d split_tail=%d max_workgroups=%d "
                  "split_tail1=%d ragged=%d",
                  plan->block_m, plan->gemm1_tile, t1.BM, t1.BN, t1.BK, t1.WM, t1.WN, t1.stages, t1.mfma,
                  plan->gemm2_tile, t2.BM, t2.BN, t2.BK, t2.WM, t2.WN, t2.stages, t2.mfma, plan->split_k, split1(plan),
                  split_tail(plan) ? plan->split_tail : 0, plan->max_workgroups,
                  split_tail1(plan) ? plan->split_tail1 : 0, plan->ragged);
    return MOE_OK;
}

moe_status moe_workspace_offsets(const moe_layer *layer, int32_t T, const moe_plan *plan, int64_t *offsets) {
    moe_status st = check_layer(layer);
    if (st != MOE_OK) return st;
    if (T < 0 || !offsets) return MOE_ERR_INVALID_ARGUMENT;
    moe_plan p;
    if (plan) p = *plan;
    else if ((st = moe_default_plan(layer, T, &p)) != MOE_OK) return st;
    TileInfo t1, t2;
    if ((st = check_plan(layer, &p, &t1, &t2)) != MOE_OK) return st;
    const Workspace w = layout(layer, T, &p);
    const size_t v[MOE_WS_COUNT] = {w.ids, w.weights, w.sorted, w.eids, w.npp, w.counts, w.inv_pos, w.scal,
                                    w.xq, w.h, w.hq, w.y, w.align_scratch, w.g1p, w.tail, w.tail1, w.blk_start};
    for (int i = 0; i < MOE_WS_COUNT; i++) offsets[i] = (int64_t)v[i];
    return MOE_OK;
}

moe_status moe_grouped_gemm_default_tile(const moe_grouped_gemm_desc *desc, int32_t M, int32_t *tile) {
    if (!desc || !tile || M < 0) return MOE_ERR_INVALID_ARGUMENT;
    TileInfo t;
    if (desc->num_groups < 1 || desc->num_groups > kMaxGroups) return MOE_ERR_INVALID_ARGUMENT;
    moe_status st = check_grouped_size(desc);
    if (st != MOE_OK) return st;
    const int32_t g = grouped_default_tile(desc, M);
    if (g < 0) return check_grouped(desc, 0, &t) == MOE_OK ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARGUMENT;
    *tile = g;
    return MOE_OK;
}

moe_status moe_grouped_gemm_workspace_bytes(const moe_grouped_gemm_desc *desc, int32_t M, int32_t tile,
                                            size_t *bytes) {
    if (!bytes || M < 0) return MOE_ERR_INVALID_ARGUMENT;
    moe_status st;
    if ((st = check_grouped_size(desc)) != MOE_OK) return st;
    if (tile < 0 && (st = moe_grouped_gemm_default_tile(desc, M, &tile)) != MOE_OK) return st;
    TileInfo t;
    if ((st = check_grouped(desc, tile, &t)) != MOE_OK) return st;
    *bytes = grouped_layout(desc, M, t.BM).total;
    return MOE_OK;
}

moe_status moe_grouped_gemm(const moe_grouped_gemm_desc *desc, int32_t M, const void *x, const float *x_scale,
                            const int32_t *m_sizes, void *y, void *workspace, size_t workspace_bytes, int32_t tile,
                            void *stream) {
    if (M < 0) return MOE_ERR_INVALID_ARGUMENT;
    moe_status st;
    if ((st = check_grouped_size(desc)) != MOE_OK) return st;
    if (tile < 0 && (st = moe_grouped_gemm_default_tile(desc, M, &tile)) != MOE_OK) return st;
    TileInfo t;
    if ((st = check_grouped(desc, tile, &t)) != MOE_OK) return st;
    if (M == 0) return MOE_OK;
    if (!x || !m_sizes || !y || !workspace || !aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, kAlign) ||
        !aligned(m_sizes, 4))
        return MOE_ERR_INVALID_ARGUMENT;
    const bool fp8 = desc->dtype == MOE_DT_FP8_E4M3;
    if (fp8 && (!x_scale || !aligned(x_scale, 4))) return MOE_ERR_INVALID_ARGUMENT;
    const GroupedWorkspace w = grouped_layout(desc, M, t.BM);
    if (workspace_bytes < w.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
    const int64_t ebytes = fp8 ? 1 : 2;
    // the GEMM addresses rows of X with 32-bit byte offsets from its base
    if ((int64_t)M * desc->K * ebytes > (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    int32_t *sorted = (int32_t *)(ws + w.sorted), *eids = (int32_t *)(ws + w.eids), *npp = (int32_t *)(ws + w.npp);
    hipError_t err;
    SegmentArgs sa{m_sizes, desc->num_groups, M, t.BM, nbits_for(t.BM), sorted, eids, npp};
    if ((err = launch_segments(sa, w.cap, s)) != hipSuccess) return MOE_ERR_HIP;
    GemmArgs g{};
    g.A = x;
    g.lda = desc->K;
    g.B = desc->w;
    g.ldb = desc->K * ebytes;
    g.b_expert_stride = (int64_t)desc->N * desc->K * ebytes;
    g.C = y;
    g.ldc = desc->N;
    g.sorted = sorted;
    g.eids = eids;
    g.npp = npp;
    g.topk_w = nullptr;
    g.K = desc->K;
    g.N = desc->N;
    g.top_k = 1;
    g.pairs = M;
    g.split = 1;
    g.ksplit = desc->K;
    g.a_scale = x_scale;
    g.b_scale = desc->w_scale;
    g.out_by_pair = 1;
    g.gather_a = 1;
    // weight streaming (about one block per group): stagger the K walks over DRAM channels
    g.rotate_k = (int64_t)M <= (int64_t)desc->num_groups * t.BM;
    if ((err = launch_gemm(desc->dtype, tile, GEMM_DOWN, false, g, w.cap / t.BM * (desc->N / t.BN), s)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

}  // extern "C"
