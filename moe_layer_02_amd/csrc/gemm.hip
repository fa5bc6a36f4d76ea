// gemm.hip -- persistent expert-tiled grouped GEMMs of the MoE layer (gfx950 MFMA).
//
// One launch covers every expert (vLLM PR #12185 "[Kernel] add triton fused moe kernel for
// gptq/awq": a single launch instead of one or more per expert).  The M dimension is the
// align layout: block b of BM rows belongs to expert expert_ids[b]; a tile is (block, N
// tile, K split).  Workgroups are persistent: each walks tiles with a stride of the grid,
// the grid's tiles remapped so that neighbouring tiles (same expert weights, same rows)
// run on the same XCD and share its L2.  Nothing is read back to the host: the number of
// tiles comes from num_tokens_post_padded in device memory.
//
// Per tile: global -> registers (16-byte loads) -> LDS (double buffered, one barrier per K
// step, the next step's loads in flight while the current one multiplies) -> MFMA.
//   bf16: v_mfma_f32_16x16x32_bf16.
//   fp8 (w8a8 per tensor, SGLang PR #2333 / the FBGEMM article): E4M3 operands on
//         v_mfma_scale_f32_16x16x128_f8f6f4 with unit block scales; the per-tensor scales
//         multiply the fp32 accumulator in the epilogue.
//   int4 (GPTQ/AWQ group 128, vLLM PR #12185): packed nibbles stay packed in LDS; each lane
//         turns 8 nibbles into bf16 weights in registers ((q - z) * s in fp32, exact, then
//         rounded once to bf16) and multiplies them with the bf16 activations on
//         v_mfma_f32_16x16x32_bf16.
// Gate/up epilogue: SiLU(gate) * up in fp32, stored as bf16 (fp8: kept in fp32, so that
// its E4M3 code is later decided in fp32, and the tile's largest |h| goes into a device
// word with an integer atomicMax -- max is order-independent).  Down
// epilogue: times the pair's top-k weight; either bf16 rows or fp32 split-K partial planes
// that the reduce step sums in a fixed order (no floating-point atomics: SGLang PR #2333,
// Background, traces its corrupted outputs to atomic_add).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

enum { WT_BF16 = 0, WT_FP8 = 2, WT_INT4 = 3 };

template <int WT, int BM_, int BN_, int BK_, int WM_, int WN_>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
    static constexpr int NT = WM * WN * kWave;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int MFMA_K = WT == WT_FP8 ? 128 : 32;
    static constexpr int A_ROW = WT == WT_FP8 ? BK : BK * 2;                 // bytes in LDS
    static constexpr int B_ROW = WT == WT_FP8 ? BK : WT == WT_INT4 ? BK / 2 : BK * 2;
    static constexpr int A_LDS = A_ROW + 16, B_LDS = B_ROW + 16;            // padded strides
    static constexpr int A_CH = A_ROW / 16, B_CH = B_ROW / 16;              // 16 B chunks per row
    static constexpr int A_IT = (BM * A_CH + NT - 1) / NT, B_IT = (BN * B_CH + NT - 1) / NT;
    static constexpr int STAGE = BM * A_LDS + BN * B_LDS;
    static constexpr int GROUPS = WT == WT_INT4 ? BK / 128 : 1;              // int4 groups per step
    static_assert(BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile / wave grid mismatch");
    static_assert(BK % MFMA_K == 0, "K step must hold whole MFMAs");
    static_assert(WT != WT_INT4 || BK % 128 == 0, "int4 K step must hold whole groups");
};

// 8 nibbles (k = 0..7 of one row, byte b = k/2, low nibble first) -> bf16 (q - z) * s in
// the natural order.  q - z is an integer of at most 4 bits and s an fp16 value, so the
// fp32 product is exact and the bf16 weight is rounded once (to nearest even).
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float z, float s) {
    bf16x8 out;
#pragma unroll
    for (int k = 0; k < 8; k++) out[k] = static_cast<__bf16>(((float)((w >> (4 * k)) & 0xFu) - z) * s);
    return out;
}

template <class C, int WT, int KIND, bool PARTIAL>
__global__ __launch_bounds__(C::NT) void k_gemm(GemmArgs a) {
    __shared__ __attribute__((aligned(16))) char smem[2][C::STAGE];
    const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int npp = *a.npp;
    const int mblocks = npp / C::BM;
    const int n_out = KIND == GEMM_GATE_UP ? C::BN / 2 : C::BN;   // output columns per tile
    const int ntiles = a.N / n_out;
    const int total = mblocks * ntiles * a.split;
    const int G = gridDim.x;
    const int j0 = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int nk = a.ksplit / C::BK;

    const int mn = mblocks * ntiles;
    for (int tile = j0; tile < total; tile += G) {
        // split outermost; then groups of group_m blocks, block index fastest inside a group,
        // so one XCD's window of consecutive tiles covers a compact (block x N tile) patch
        // whose A rows and weight rows its L2 serves to several workgroups
        const int s = tile / mn;
        const int rest = tile - s * mn;
        const int gm0 = rest / (a.group_m * ntiles) * a.group_m;
        const int gsz = min(a.group_m, mblocks - gm0);
        const int local = rest - gm0 * ntiles;
        const int mb = gm0 + local % gsz;
        const int nt = local / gsz;
        const int e = a.eids[mb];
        const BlockRows br = block_rows(a, mb, C::BM);
        const int row0 = br.row0;   // first row of the block in h / y (the layout's)
        const int kbase = s * a.ksplit;

        // ---- per-thread global sources for this tile (fixed over the K loop) ----
        const char *a_src[C::A_IT];
        bool a_ok[C::A_IT];
#pragma unroll
        for (int it = 0; it < C::A_IT; it++) {
            const int c = tid + it * C::NT;
            const int r = c / C::A_CH, ch = c % C::A_CH;
            a_ok[it] = c < C::BM * C::A_CH;
            a_src[it] = nullptr;
            if (a_ok[it]) {
                const int g_ebytes = WT == WT_FP8 ? 1 : 2;     // A element bytes in global
                int64_t arow;
                if (KIND == GEMM_GATE_UP) {
                    const int p = block_pair(a, br, r);
                    a_ok[it] = p < a.pairs;
                    arow = a_ok[it] ? p / a.top_k : 0;
                } else {
                    arow = row0 + (r < br.n ? r : 0);   // past the block's pairs: never stored
                }
                a_src[it] = (const char *)a.A + (arow * a.lda + (int64_t)kbase) * g_ebytes + ch * 16;
            }
        }
        const char *b_src[C::B_IT];
        bool b_ok[C::B_IT];
        const char *bexp = (const char *)a.B + (int64_t)e * a.b_expert_stride;
#pragma unroll
        for (int it = 0; it < C::B_IT; it++) {
            const int c = tid + it * C::NT;
            const int rr = c / C::B_CH, ch = c % C::B_CH;
            b_ok[it] = c < C::BN * C::B_CH;
            int64_t grow = 0;
            if (KIND == GEMM_GATE_UP) {   // LDS rows of wave column w: gate half, then up half
                const int wcol = rr / C::TN, i = rr % C::TN, half = C::TN / 2;
                const int col = nt * (C::BN / 2) + wcol * half + (i % half);
                grow = i < half ? col : a.I + col;
            } else {
                grow = (int64_t)nt * C::BN + rr;
            }
            const int kb = WT == WT_FP8 ? kbase : WT == WT_INT4 ? kbase / 2 : kbase * 2;
            b_src[it] = bexp + grow * a.ldb + kb + ch * 16;
        }
        // int4: this lane's B rows (one per N fragment) for scale / zero lookups; the
        // scales are group-major, sz_rows (the matrix's rows) apart from group to group
        const int64_t sz_rows = KIND == GEMM_GATE_UP ? 2 * (int64_t)a.I : a.N;
        int64_t sz_row[C::FN];
#pragma unroll
        for (int fn = 0; fn < C::FN; fn++) {
            const int rr = wn * C::TN + fn * 16 + (lane & 15);
            int64_t grow;
            if (KIND == GEMM_GATE_UP) {
                const int i = rr % C::TN, half = C::TN / 2;
                const int col = nt * (C::BN / 2) + wn * half + (i % half);
                grow = i < half ? col : a.I + col;
            } else {
                grow = (int64_t)nt * C::BN + rr;
            }
            sz_row[fn] = (int64_t)e * a.sz_expert_stride + grow;   // group-major [K/128][rows]
        }

        uint4 ra[C::A_IT], rb[C::B_IT];
        uint32_t rs[C::GROUPS][C::FN], rz[C::GROUPS][C::FN];
        uint32_t cs[C::GROUPS][C::FN], cz[C::GROUPS][C::FN];
        // with rotate_k each tile walks its K range from its own starting step (see
        // gemm_pipe.hip); the order is fixed per tile
        const int krot = a.rotate_k ? (nt * 3 + mb * 5) % nk : 0;
        auto load_stage = [&](int kstep) {
            const int kr = kstep + krot < nk ? kstep + krot : kstep + krot - nk;
            const int koff = kr * C::BK;
#pragma unroll
            for (int it = 0; it < C::A_IT; it++) {
                const int ab = WT == WT_FP8 ? koff : koff * 2;
                ra[it] = a_ok[it] ? *(const uint4 *)(a_src[it] + ab) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int it = 0; it < C::B_IT; it++) {
                const int bb = WT == WT_FP8 ? koff : WT == WT_INT4 ? koff / 2 : koff * 2;
                rb[it] = b_ok[it] ? *(const uint4 *)(b_src[it] + bb) : make_uint4(0, 0, 0, 0);
            }
            if constexpr (WT == WT_INT4) {
#pragma unroll
                for (int g = 0; g < C::GROUPS; g++)
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const int64_t gi = sz_row[fn] + (int64_t)((kbase + koff) / 128 + g) * sz_rows;
                        rs[g][fn] = a.bs[gi];
                        rz[g][fn] = a.bz[gi];
                    }
            }
        };
        auto store_stage = [&](char *st) {
#pragma unroll
            for (int it = 0; it < C::A_IT; it++) {
                const int c = tid + it * C::NT;
                if (c < C::BM * C::A_CH) {
                    const int r = c / C::A_CH, ch = c % C::A_CH;
                    *(uint4 *)(st + r * C::A_LDS + ch * 16) = ra[it];
                }
            }
            char *sb = st + C::BM * C::A_LDS;
#pragma unroll
            for (int it = 0; it < C::B_IT; it++) {
                const int c = tid + it * C::NT;
                if (c < C::BN * C::B_CH) {
                    const int rr = c / C::B_CH, ch = c % C::B_CH;
                    *(uint4 *)(sb + rr * C::B_LDS + ch * 16) = rb[it];
                }
            }
            if constexpr (WT == WT_INT4) {
#pragma unroll
                for (int g = 0; g < C::GROUPS; g++)
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        cs[g][fn] = rs[g][fn];
                        cz[g][fn] = rz[g][fn];
                    }
            }
        };

        f32x4 acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int j = 0; j < C::FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        load_stage(0);
        store_stage(smem[0]);
        __syncthreads();
        for (int kt = 0; kt < nk; kt++) {
            const char *st = smem[kt & 1];
            // int4: scales of the current step, captured before the next step's loads land
            uint32_t us[C::GROUPS][C::FN], uz[C::GROUPS][C::FN];
            if constexpr (WT == WT_INT4) {
#pragma unroll
                for (int g = 0; g < C::GROUPS; g++)
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        us[g][fn] = cs[g][fn];
                        uz[g][fn] = cz[g][fn];
                    }
            }
            if (kt + 1 < nk) load_stage(kt + 1);
            const char *sa = st, *sb = st + C::BM * C::A_LDS;
#pragma unroll
            for (int kk = 0; kk < C::BK / C::MFMA_K; kk++) {
                if constexpr (WT == WT_BF16) {
                    bf16x8 af[C::FM], bfr[C::FN];
                    const int kb = (kk * 32 + 8 * (lane >> 4)) * 2;
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
                        af[fm] = *(const bf16x8 *)(sa + (wm * C::TM + fm * 16 + (lane & 15)) * C::A_LDS + kb);
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++)
                        bfr[fn] = *(const bf16x8 *)(sb + (wn * C::TN + fn * 16 + (lane & 15)) * C::B_LDS + kb);
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                        for (int fn = 0; fn < C::FN; fn++)
                            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
                } else if constexpr (WT == WT_FP8) {
                    i32x8 af[C::FM], bfr[C::FN];
                    const int kb = kk * 128 + 32 * (lane >> 4);
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
                        af[fm] = *(const i32x8 *)(sa + (wm * C::TM + fm * 16 + (lane & 15)) * C::A_LDS + kb);
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++)
                        bfr[fn] = *(const i32x8 *)(sb + (wn * C::TN + fn * 16 + (lane & 15)) * C::B_LDS + kb);
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                        for (int fn = 0; fn < C::FN; fn++)
                            acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                af[fm], bfr[fn], acc[fm][fn], 0, 0, 0, 127, 0, 127);
                } else {   // int4
                    bf16x8 af[C::FM], bfr[C::FN];
                    const int kel = kk * 32 + 8 * (lane >> 4);
                    const int g = kk * 32 / 128;
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
                        af[fm] = *(const bf16x8 *)(sa + (wm * C::TM + fm * 16 + (lane & 15)) * C::A_LDS + kel * 2);
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const uint32_t w = *(const uint32_t *)(sb + (wn * C::TN + fn * 16 + (lane & 15)) * C::B_LDS + kel / 2);
                        const float sv = (float)__builtin_bit_cast(_Float16, (uint16_t)us[g][fn]);
                        const float zv = (float)__builtin_bit_cast(_Float16, (uint16_t)uz[g][fn]);
                        bfr[fn] = dequant8(w, zv, sv);
                    }
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                        for (int fn = 0; fn < C::FN; fn++)
                            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
                }
            }
            if (kt + 1 < nk) store_stage(smem[(kt + 1) & 1]);
            __syncthreads();
        }

        // ---- epilogue: lane holds rows 4*(lane/16)+i, column lane%16 of each 16x16 fragment ----
        float scale = 1.0f;
        if constexpr (WT == WT_FP8) scale = a.a_scale[0] * a.b_scale[e];
        // the lane's rows, q = fm * 4 + i; their pairs (and GEMM2's weights) are read and
        // pinned before the stores (see pin)
        constexpr int EQ = C::FM * 4;
        auto epi_row = [&](int q) { return wm * C::TM + (q / 4) * 16 + 4 * (lane >> 4) + q % 4; };
        if constexpr (KIND == GEMM_GATE_UP && PARTIAL) {
            // split K: this split's gate and up sums in fp32 (the finishing pass adds the
            // splits in order and applies SiLU * up); filler rows are left out
            int pr[EQ];
#pragma unroll
            for (int q = 0; q < EQ; q++) pr[q] = block_pair_nb(a, br, epi_row(q));
            pin_all(pr);
#pragma unroll
            for (int q = 0; q < EQ; q++) {
                const int fm = q / 4, i = q % 4, row = row0 + epi_row(q);
                if (pr[q] >= a.pairs) continue;
                float *P = (float *)a.C + (int64_t)s * a.partial_stride + (int64_t)row * a.ldc;
#pragma unroll
                for (int f = 0; f < C::FN / 2; f++) {
                    const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * 16 + (lane & 15);
                    P[col] = acc[fm][f][i] * scale;
                    P[a.I + col] = acc[fm][f + C::FN / 2][i] * scale;
                }
            }
        } else if constexpr (KIND == GEMM_GATE_UP) {
            float amax = 0.0f;
            uint32_t seen = 0;   // the h maximum so far, read before the stores (see amax_peek)
            if constexpr (WT == WT_FP8)
                if (lane == 0 && a.amax_out) seen = amax_peek(a.amax_out);
            bool valid[EQ];   // |h| of filler rows stays out of the maximum (fp8 only)
            if constexpr (WT == WT_FP8) {
                int pr[EQ];
#pragma unroll
                for (int q = 0; q < EQ; q++) pr[q] = block_pair_nb(a, br, epi_row(q));
                pin_all(pr);
#pragma unroll
                for (int q = 0; q < EQ; q++) valid[q] = pr[q] < a.pairs;
            }
#pragma unroll
            for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                for (int f = 0; f < C::FN / 2; f++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float g = acc[fm][f][i] * scale, u = acc[fm][f + C::FN / 2][i] * scale;
                        const float hv = silu(g) * u;
                        const int lr = epi_row(fm * 4 + i), row = row0 + lr;
                        if (lr >= br.n) continue;   // without padding: the next block's row
                        const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * 16 + (lane & 15);
                        if constexpr (WT == WT_FP8) {   // fp32: its E4M3 code is decided in fp32
                            ((float *)a.C)[(int64_t)row * a.ldc + col] = hv;
                            if (valid[fm * 4 + i]) amax = fmaxf(amax, fabsf(hv));   // valid rows only
                        } else {
                            ((uint16_t *)a.C)[(int64_t)row * a.ldc + col] = f32_to_bf16_bits(hv);
                        }
                    }
            if constexpr (WT == WT_FP8) {
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
                if (lane == 0 && a.amax_out) amax_raise(a.amax_out, seen, amax);
            }
        } else {
            int pr[EQ];
            float wr[EQ];
#pragma unroll
            for (int q = 0; q < EQ; q++) pr[q] = block_pair_nb(a, br, epi_row(q));
            pin_all(pr);
#pragma unroll
            for (int q = 0; q < EQ; q++) wr[q] = a.topk_w[pr[q] < a.pairs ? pr[q] : 0];   // filler: pair 0's
            pin_all(wr);
#pragma unroll
            for (int q = 0; q < EQ; q++) wr[q] *= scale;
#pragma unroll
            for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int lr = epi_row(fm * 4 + i), row = row0 + lr;
                    const int p = pr[fm * 4 + i];
                    if (p >= a.pairs) continue;   // filler row: never read back
                    const float w = wr[fm * 4 + i];
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const int col = nt * C::BN + wn * C::TN + fn * 16 + (lane & 15);
                        const float v = acc[fm][fn][i] * w;
                        if constexpr (PARTIAL)
                            ((float *)a.C)[(int64_t)s * a.partial_stride + (int64_t)row * a.ldc + col] = v;
                        else
                            ((uint16_t *)a.C)[(a.out_by_pair ? (int64_t)p : row) * a.ldc + col] = f32_to_bf16_bits(v);
                    }
                }
        }
    }
}

// ---- tile tables --------------------------------------------------------------------
#define BF16_TILES(X)              \
    X(0, 16, 64, 256, 1, 2)        \
    X(1, 16, 128, 128, 1, 4)       \
    X(2, 32, 128, 128, 1, 4)       \
    X(3, 64, 128, 64, 2, 2)        \
    X(4, 128, 128, 64, 2, 2)       \
    X(5, 128, 256, 64, 2, 2)
#define FP8_TILES(X)               \
    X(0, 16, 128, 256, 1, 4)       \
    X(1, 16, 128, 128, 1, 4)       \
    X(2, 32, 128, 128, 1, 4)       \
    X(3, 64, 128, 128, 2, 2)       \
    X(4, 128, 128, 128, 2, 2)      \
    X(5, 128, 256, 128, 2, 2)
#define INT4_TILES(X)              \
    X(0, 16, 128, 128, 1, 4)       \
    X(1, 32, 128, 128, 1, 4)       \
    X(2, 64, 128, 128, 2, 2)       \
    X(3, 128, 128, 128, 2, 2)

#define COUNT_TILE(id, bm, bn, bk, wm, wn) +1
constexpr int kBf16Tiles = 0 BF16_TILES(COUNT_TILE);
constexpr int kFp8Tiles = 0 FP8_TILES(COUNT_TILE);
constexpr int kInt4Tiles = 0 INT4_TILES(COUNT_TILE);

template <class C, int WT, int KIND, bool PARTIAL>
hipError_t launch_one(const GemmArgs &a, int64_t max_tiles, hipStream_t s) {
    static int occ_cache[64] = {0};   // per device; benign race (same value computed)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int occ = dev < 64 ? __atomic_load_n(&occ_cache[dev], __ATOMIC_RELAXED) : 0;
    if (occ == 0) {
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemm<C, WT, KIND, PARTIAL>, C::NT, 0);
        if (err != hipSuccess) return err;
        if (occ < 1) occ = 1;
        if (dev < 64) __atomic_store_n(&occ_cache[dev], occ, __ATOMIC_RELAXED);
    }
    int64_t grid = (int64_t)device_cu_count() * occ;
    if (max_tiles < grid) grid = max_tiles;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    // blocks per tile group: about the square root of one XCD's concurrent workgroups
    GemmArgs b = a;
    b.group_m = 1;
    while (b.group_m * b.group_m * 4 <= grid / 8 && b.group_m < 16) b.group_m *= 2;
    hipLaunchKernelGGL((k_gemm<C, WT, KIND, PARTIAL>), dim3((unsigned)grid), dim3(C::NT), 0, s, b);
    return hipGetLastError();
}

template <class C, int WT>
hipError_t launch_kind(GemmKind kind, bool partial, const GemmArgs &a, int64_t max_tiles, hipStream_t s) {
    if (kind == GEMM_GATE_UP) {
        if (!partial) return launch_one<C, WT, GEMM_GATE_UP, false>(a, max_tiles, s);
        if constexpr (C::BM <= 32) return launch_one<C, WT, GEMM_GATE_UP, true>(a, max_tiles, s);
        return hipErrorInvalidValue;   // GEMM1 split-K is built for the small-T tiles only
    }
    if (partial) return launch_one<C, WT, GEMM_DOWN, true>(a, max_tiles, s);
    return launch_one<C, WT, GEMM_DOWN, false>(a, max_tiles, s);
}

}  // namespace

int gemm_tile_count(int wdtype) {
    return wdtype == WT_BF16 ? kBf16Tiles : wdtype == WT_FP8 ? kFp8Tiles : wdtype == WT_INT4 ? kInt4Tiles : 0;
}

bool gemm_tile_info(int wdtype, int tile, TileInfo *info) {
#define INFO_TILE(id, bm, bn, bk, wm, wn) \
    if (tile == id) {                     \
        *info = TileInfo{bm, bn, bk, wm, wn, 0, 16}; \
        return true;                      \
    }
    if (wdtype == WT_BF16) { BF16_TILES(INFO_TILE) }
    if (wdtype == WT_FP8) { FP8_TILES(INFO_TILE) }
    if (wdtype == WT_INT4) { INT4_TILES(INFO_TILE) }
#undef INFO_TILE
    return pipe_tile_info(wdtype, tile, info);
}

hipError_t launch_gemm(int wdtype, int tile, GemmKind kind, bool partial, const GemmArgs &a,
                       int64_t max_tiles, hipStream_t s) {
#define LAUNCH_TILE(WT, id, bm, bn, bk, wm, wn) \
    if (tile == id) return launch_kind<Cfg<WT, bm, bn, bk, wm, wn>, WT>(kind, partial, a, max_tiles, s);
#define L_BF16(id, bm, bn, bk, wm, wn) LAUNCH_TILE(WT_BF16, id, bm, bn, bk, wm, wn)
#define L_FP8(id, bm, bn, bk, wm, wn) LAUNCH_TILE(WT_FP8, id, bm, bn, bk, wm, wn)
#define L_INT4(id, bm, bn, bk, wm, wn) LAUNCH_TILE(WT_INT4, id, bm, bn, bk, wm, wn)
    if (wdtype == WT_BF16) { BF16_TILES(L_BF16) }
    if (wdtype == WT_FP8) { FP8_TILES(L_FP8) }
    if (wdtype == WT_INT4) { INT4_TILES(L_INT4) }
    return launch_gemm_pipe(wdtype, tile, kind, partial, a, max_tiles, s);
}

}  // namespace moe
