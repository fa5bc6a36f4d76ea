// gemm_i4.hip -- the grouped GEMMs for int4 group-128 weights, direct-to-LDS pipelined.
//
// The w4a16 kernel of vLLM PR #12185 ("[Kernel] add triton fused moe kernel for gptq/awq":
// one launch for every expert, GPTQ/AWQ packing, dequantisation inside the GEMM), laid out
// for gfx950.  Weights stay packed all the way into LDS: a stage holds one 128-byte slab of
// every B row (256 K values, two quantisation groups), the rows' two fp16 scales and two
// fp16 zero points, and the matching 256 K values of every A row in bf16 -- all moved by
// global_load_lds (16 bytes per lane for the slabs, 4 for the scales and zeros), ST stages
// in flight, as in gemm_pipe.hip.
//
// Dequantisation is split between the VALU and the MFMA's fp32 accumulation.  OR-ing a
// nibble into the low bits of bf16 128.0 (0x4300) gives exactly 128 + q (bf16 holds every
// integer of [128, 256)); two nibbles are taken per 32-bit operation (nibbles i and i + 4
// of a word land in the two halves of a packed bf16 pair), so a word of 8 consecutive K
// values costs 7 VALU operations and comes out in the order (0,4,1,5,2,6,3,7).  The MFMAs
// of one quantisation group accumulate D = sum a (128 + q) and, against a fragment of
// ones, R = sum a; the group then adds s D - s (128 + z) R = s sum a (q - z) to the output
// in fp32 -- the exact dequantised product up to fp32 rounding of terms about 128 times
// larger than the weights.  The activations stay bf16, so every bf16 hidden value is
// taken as it is (no narrowing to a smaller exponent range); they are stored in the
// nibble order inside every group of 8 (a permutation pass reorders the hidden states;
// GEMM1 writes h permuted), so A and B agree element for element and the dot products are
// unchanged.
//
// K assignment per MFMA (v_mfma_f32_16x16x32_bf16, lane group g = lane / 16): in step
// (half, d), half = 0..1 the group of the slab and d = 0..3, lane group g takes the K
// values 128 half + 32 g + 8 d .. +7 -- dword d of 16-byte chunk g + 4 half of its B row,
// and 16-byte chunk 4 (g & 1) + d of bf16 A slab 2 half + g / 2.  Each B row is therefore
// read with two 16-byte LDS reads per stage, and each A row with one per MFMA.
#include "common.h"
#include "kernels.h"
#include "pipe.h"

namespace moe {
namespace {

template <int BM_, int BN_, int ST_, int WM_, int WN_>
struct ICfg {
    static constexpr int BM = BM_, BN = BN_, ST = ST_, WM = WM_, WN = WN_;
    static constexpr int NW = WM * WN, NT = NW * kWave;
    static constexpr int BK = 256;                             // K per stage: one packed slab
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / 16, FN = TN / 16;
    static constexpr int A_SLABS = 4;                          // 4 x 64 bf16 per A row
    static constexpr int A_STAGE = A_SLABS * BM * 128, B_STAGE = BN * 128, SZ = BN * 4;
    static constexpr int STAGE = A_STAGE + B_STAGE + 2 * SZ;
    static constexpr int A_LOADS = A_SLABS * BM / 8, B_LOADS = BN / 8;
    // a stage's scales (and zero points) are 2 groups x BN rows of fp16, two contiguous
    // runs of the group-major arrays: BN / 4 chunks of 16 bytes, spread over SZ_PARTS
    // instructions each, with SZ_PARTS the fewest that keep every wave's load count equal
    static constexpr int sz_parts() {
        int p = 1;
        while ((A_LOADS + B_LOADS + 2 * p) % NW) p++;
        return p;
    }
    static constexpr int SZ_PARTS = sz_parts(), SZ_LOADS = 2 * SZ_PARTS;
    static constexpr int SZ_LANES = (BN / 4 + SZ_PARTS - 1) / SZ_PARTS;   // chunks per instruction
    static_assert(SZ_LANES <= 64 && (SZ_PARTS - 1) * SZ_LANES < BN / 4, "every part instruction loads");
    static constexpr int LOADS = A_LOADS + B_LOADS + SZ_LOADS;
    static constexpr int LPW = LOADS / NW;
    static_assert(LOADS % NW == 0, "stage loads must split evenly over the waves");
    static_assert(BN % 64 == 0 && BM % (16 * WM) == 0 && BN % (16 * WN) == 0, "tile / wave grid mismatch");
    static_assert((ST - 2) * LPW <= 63, "vmcnt range");
    static constexpr bool SKIP_FILLER = BM <= 32;   // as in gemm_pipe.hip
};

// 8 nibbles (K values 0..7 of one row, low nibble first in each byte) -> bf16 128 + q in
// the order (0,4,1,5,2,6,3,7)
__device__ __forceinline__ bf16x8 raw8(uint32_t w) {
    uint4 r;
    r.x = (w & 0x000F000Fu) | 0x43004300u;
    r.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
    r.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
    r.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
    return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ _Float16 half_of(uint32_t w, int hi) {
    return __builtin_bit_cast(_Float16, (uint16_t)(hi ? w >> 16 : w & 0xFFFFu));
}

// column c of h is stored at this position (the (0,4,1,5,2,6,3,7) order inside each 8)
__device__ __forceinline__ int perm_col(int c) { return (c & ~7) | ((c & 3) << 1) | ((c >> 2) & 1); }

enum { LD_A = 0, LD_B = 1, LD_S = 2, LD_Z = 3 };

template <class C, int KIND, bool PARTIAL>
__global__ __launch_bounds__(C::NT, 1) void k_gemm_i4(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[C::ST * C::STAGE];
    const int lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int npp = *a.npp;
    const int mblocks = npp / C::BM;
    const int n_out = KIND == GEMM_GATE_UP ? C::BN / 2 : C::BN;
    const int ntiles = a.N / n_out;
    const int mn = mblocks * ntiles;
    const int total = mn * a.split;
    const int G = gridDim.x;
    const int nk = a.ksplit / C::BK;
    const int64_t sz_rows = KIND == GEMM_GATE_UP ? 2 * (int64_t)a.I : a.N;   // rows of the B matrix

    for (int tile = xcd_first_tile(blockIdx.x, G); tile < total; tile += G) {
        const TileCoord tc = tile_coord(tile, mn, mblocks, ntiles, a.group_m);
        const int s = tc.s, mb = tc.mb, nt = tc.nt;
        const int e = __builtin_amdgcn_readfirstlane(a.eids[mb]);
        const BlockRows br = block_rows(a, mb, C::BM);
        const int row0 = br.row0;   // first row of the block in h / y (the layout's)

        // B row (of the expert's matrix) that tile row rr of the B slab holds
        auto b_row = [&](int rr) -> int64_t {
            if (KIND == GEMM_GATE_UP) {   // rows of wave column w: its gate half, then its up half
                const int wcol = rr / C::TN, i = rr % C::TN, half = C::TN / 2;
                const int col = nt * (C::BN / 2) + wcol * half + (i % half);
                return i < half ? col : a.I + col;
            }
            return (int64_t)nt * C::BN + rr;
        };

        // per load instruction q of this wave: kind, the lane's global source at the split's
        // first K, the bytes it advances per K step, and the wave's LDS offset in a stage
        uint32_t voff[C::LPW];
        int dst[C::LPW], kind[C::LPW];
        bool on[C::LPW];   // lane loads (filler rows of A are skipped, as in gemm_pipe.hip)
#pragma unroll
        for (int q = 0; q < C::LPW; q++) {
            on[q] = true;
            const int ins = wave + q * C::NW;
            if (ins < C::A_LOADS) {
                const int slab = ins / (C::BM / 8), rb = ins % (C::BM / 8) * 8;
                const int r = rb + (lane >> 3);
                const int chunk = (lane & 7) ^ swz_key<2>(r);   // A's layout key (pipe.h)
                const int p = block_pair(a, br, r);
                // a row past the block's pairs reads its block's first row (never stored)
                const int64_t arow = KIND == GEMM_GATE_UP ? (p < a.pairs ? p / a.top_k : 0) : row0 + (r < br.n ? r : 0);
                on[q] = !C::SKIP_FILLER || p < a.pairs || (lane >> 3) == 0;
                voff[q] = (uint32_t)(arow * a.lda * 2 + slab * 128 + chunk * 16);
                dst[q] = (slab * C::BM + rb) * 128;
                kind[q] = LD_A;
            } else if (ins < C::A_LOADS + C::B_LOADS) {
                const int rb = (ins - C::A_LOADS) * 8;
                const int rr = rb + (lane >> 3);
                const int chunk = (lane & 7) ^ swz(rr);
                voff[q] = (uint32_t)(b_row(rr) * a.ldb + chunk * 16);
                dst[q] = C::A_STAGE + rb * 128;
                kind[q] = LD_B;
            } else {   // scales (or zero points): chunk c = 8 rows of group c / (BN / 8)
                const int j = ins - C::A_LOADS - C::B_LOADS;
                const int which = j / C::SZ_PARTS, c = j % C::SZ_PARTS * C::SZ_LANES + lane;
                const int grp = c / (C::BN / 8), t0 = c % (C::BN / 8) * 8;   // t0: tile row in global order
                int64_t grow;
                if (KIND == GEMM_GATE_UP)   // the tile's gate rows, then its up rows
                    grow = t0 < C::BN / 2 ? nt * (C::BN / 2) + t0 : a.I + nt * (C::BN / 2) + (t0 - C::BN / 2);
                else
                    grow = (int64_t)nt * C::BN + t0;
                on[q] = lane < C::SZ_LANES && c < C::BN / 4;
                voff[q] = (uint32_t)((grp * sz_rows + grow) * 2);
                dst[q] = C::A_STAGE + C::B_STAGE + which * C::SZ + j % C::SZ_PARTS * C::SZ_LANES * 16;
                kind[q] = which ? LD_Z : LD_S;
            }
        }
        // weight streaming: each tile starts its K walk at a step of its expert and column
        // tile, so an expert's row blocks stay in step (see gemm_pipe.hip)
        const int krot = a.rotate_k ? (nt * 3 + e * 5) % nk : 0;
        // operand bases at the split's first K (wave-uniform); a K step advances A by 512
        // bytes (256 bf16), B by 128 (256 nibbles), scales and zeros by 4 (two groups)
        const char *base_a = uniform_ptr((const char *)a.A + (int64_t)s * a.ksplit * 2);
        const char *base_b = uniform_ptr((const char *)a.B + (int64_t)e * a.b_expert_stride + (int64_t)s * a.ksplit / 2);
        const int64_t sz0 = (int64_t)e * a.sz_expert_stride + (int64_t)s * a.ksplit / 128 * sz_rows;
        const char *base_s = uniform_ptr((const char *)(a.bs + sz0));
        const char *base_z = uniform_ptr((const char *)(a.bz + sz0));
        const char *qbase[C::LPW];
        int qstep[C::LPW];
#pragma unroll
        for (int q = 0; q < C::LPW; q++) {
            qbase[q] = kind[q] == LD_A ? base_a : kind[q] == LD_B ? base_b : kind[q] == LD_S ? base_s : base_z;
            qstep[q] = kind[q] == LD_A ? C::A_SLABS * 128 : kind[q] == LD_B ? 128 : 4 * sz_rows;
        }
        auto issue = [&](int kstep) {
            const uint32_t st = lds_addr(smem) + (kstep % C::ST) * C::STAGE;
            const int kr = __builtin_amdgcn_readfirstlane(kstep + krot < nk ? kstep + krot : kstep + krot - nk);
#pragma unroll
            for (int q = 0; q < C::LPW; q++) {
                const char *g = qbase[q] + (int64_t)kr * qstep[q];
                if (on[q]) lds_dma_off<16>(g, voff[q], st + dst[q]);
            }
        };

        f32x4 acc[C::FM][C::FN];
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int j = 0; j < C::FN; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        block_barrier();   // every wave is done with the previous tile's buffers
#pragma unroll
        for (int p = 0; p < C::ST - 1; p++)
            if (p < nk) issue(p);

        const int g = lane >> 4;
        for (int kt = 0; kt < nk; kt++) {
            wait_stages<C::LPW, C::ST - 2>(min(C::ST - 2, nk - 1 - kt));
            block_barrier();
            if (kt + C::ST - 1 < nk) issue(kt + C::ST - 1);
            const char *sa = smem + (kt % C::ST) * C::STAGE;
            const char *sb = sa + C::A_STAGE, *ss = sb + C::B_STAGE, *sz = ss + C::SZ;

            uint4 braw[2][C::FN];
            uint32_t sw[C::FN], zw[C::FN];
#pragma unroll
            for (int fn = 0; fn < C::FN; fn++) {
                const int r = wn * C::TN + fn * 16 + (lane & 15);
                braw[0][fn] = *(const uint4 *)(sb + r * 128 + ((g ^ swz(r)) << 4));
                braw[1][fn] = *(const uint4 *)(sb + r * 128 + (((g + 4) ^ swz(r)) << 4));
                // scale and zero point of B row r for the stage's 2 groups ([group][row] in
                // the global row order: the tile's gate rows, then its up rows)
                int t;
                if (KIND == GEMM_GATE_UP) {
                    const int wcol = r / C::TN, i = r % C::TN, half = C::TN / 2;
                    t = i < half ? wcol * half + i : C::BN / 2 + wcol * half + (i - half);
                } else {
                    t = r;
                }
                const uint16_t *s16 = (const uint16_t *)ss, *z16 = (const uint16_t *)sz;
                sw[fn] = (uint32_t)s16[t] | ((uint32_t)s16[C::BN + t] << 16);
                zw[fn] = (uint32_t)z16[t] | ((uint32_t)z16[C::BN + t] << 16);
            }
            const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
#pragma unroll
            for (int half = 0; half < 2; half++) {
                f32x4 dg[C::FM][C::FN], rs[C::FM];
#pragma unroll
                for (int d = 0; d < 4; d++) {
                    bf16x8 bq[C::FN];
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const uint4 v = braw[half][fn];
                        bq[fn] = raw8(d == 0 ? v.x : d == 1 ? v.y : d == 2 ? v.z : v.w);
                    }
                    const int slab = 2 * half + (g >> 1), chunk = 4 * (g & 1) + d;
                    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++) {
                        const int r = wm * C::TM + fm * 16 + (lane & 15);
                        const bf16x8 af = *(const bf16x8 *)(sa + (slab * C::BM + r) * 128 + ((chunk ^ swz_key<2>(r)) << 4));
                        rs[fm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, ones, d ? rs[fm] : zero, 0, 0, 0);
#pragma unroll
                        for (int fn = 0; fn < C::FN; fn++)
                            dg[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bq[fn], d ? dg[fm][fn] : zero, 0, 0, 0);
                    }
                }
                // the group's scale and zero point: acc += s D - s (128 + z) R
#pragma unroll
                for (int fn = 0; fn < C::FN; fn++) {
                    const float sv = (float)half_of(sw[fn], half);
                    const float zv = sv * (128.0f + (float)half_of(zw[fn], half));
#pragma unroll
                    for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            acc[fm][fn][i] = __builtin_fmaf(-zv, rs[fm][i], __builtin_fmaf(sv, dg[fm][fn][i], acc[fm][fn][i]));
                }
            }
        }

        // ---- epilogue: accumulator value i of fragment (fm, fn) is row frag_row(lane, i),
        //      column lane % 16 of that fragment ----
        const int lcol = lane & 15;
        // the lane's rows, q = fm * 4 + i; their pairs (and GEMM2's weights) are read and
        // pinned before the stores (see pin)
        constexpr int EQ = C::FM * 4;
        auto epi_row = [&](int q) { return wm * C::TM + (q / 4) * 16 + frag_row<16>(lane, q % 4); };
        if constexpr (KIND == GEMM_GATE_UP && PARTIAL) {
            // split K: this split's gate and up sums in fp32, natural column order (the
            // finishing pass adds the splits, applies SiLU * up and permutes); filler rows
            // are left out
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
                    const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * 16 + lcol;
                    P[col] = acc[fm][f][i];
                    P[a.I + col] = acc[fm][f + C::FN / 2][i];
                }
            }
        } else if constexpr (KIND == GEMM_GATE_UP) {
            // h = SiLU(gate) * up in bf16, columns in the permuted order GEMM2's A expects
#pragma unroll
            for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int lr = wm * C::TM + fm * 16 + frag_row<16>(lane, i), row = row0 + lr;
                    if (lr >= br.n) continue;   // without padding: the next block's row
#pragma unroll
                    for (int f = 0; f < C::FN / 2; f++) {
                        const float hv = silu(acc[fm][f][i]) * acc[fm][f + C::FN / 2][i];
                        const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * 16 + lcol;
                        ((uint16_t *)a.C)[(int64_t)row * a.ldc + perm_col(col)] = f32_to_bf16_bits(hv);
                    }
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
            for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int lr = epi_row(fm * 4 + i), row = row0 + lr;
                    const int p = pr[fm * 4 + i];
                    if (p >= a.pairs) continue;   // filler row: never read back
                    const float w = wr[fm * 4 + i];
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const int col = nt * C::BN + wn * C::TN + fn * 16 + lcol;
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

// ---- tile table (ids continue gemm.hip's register-staged int4 tiles) ----------------------
//        id  BM   BN  ST WM WN
#define I4_TILES(X)             \
    X(4, 16, 128, 4, 1, 4)      \
    X(5, 16, 256, 3, 1, 4)      \
    X(6, 32, 128, 4, 1, 4)      \
    X(7, 64, 128, 3, 2, 2)      \
    X(8, 16, 64, 4, 1, 2)       \
    X(9, 32, 256, 3, 1, 4)      \
    X(10, 16, 128, 3, 1, 4)     \
    X(11, 16, 256, 3, 1, 8)     \
    X(12, 32, 256, 3, 1, 8)     \
    X(13, 32, 128, 2, 1, 4)     \
    X(14, 64, 256, 2, 1, 8)

template <class C, int KIND, bool PARTIAL>
hipError_t launch_one(const GemmArgs &a, int64_t max_tiles, hipStream_t s) {
    static int occ_cache[64] = {0};   // per device; benign race (same value computed)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int occ = dev < 64 ? __atomic_load_n(&occ_cache[dev], __ATOMIC_RELAXED) : 0;
    if (occ == 0) {
        hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemm_i4<C, KIND, PARTIAL>, C::NT, 0);
        if (err != hipSuccess) return err;
        if (occ < 1) occ = 1;
        if (dev < 64) __atomic_store_n(&occ_cache[dev], occ, __ATOMIC_RELAXED);
    }
    int64_t grid = (int64_t)device_cu_count() * occ;
    if (max_tiles < grid) grid = max_tiles;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    GemmArgs b = a;
    b.group_m = 1;
    while (b.group_m * b.group_m * 4 <= grid / 8 && b.group_m < 16) b.group_m *= 2;
    hipLaunchKernelGGL((k_gemm_i4<C, KIND, PARTIAL>), dim3((unsigned)grid), dim3(C::NT), 0, s, b);
    return hipGetLastError();
}

template <class C>
hipError_t launch_kind(GemmKind kind, bool partial, const GemmArgs &a, int64_t max_tiles, hipStream_t s) {
    if (kind == GEMM_GATE_UP) {
        if (!partial) return launch_one<C, GEMM_GATE_UP, false>(a, max_tiles, s);
        if constexpr (C::BM <= 32) return launch_one<C, GEMM_GATE_UP, true>(a, max_tiles, s);
        return hipErrorInvalidValue;   // GEMM1 split-K is built for the small-T tiles only
    }
    if (partial) return launch_one<C, GEMM_DOWN, true>(a, max_tiles, s);
    return launch_one<C, GEMM_DOWN, false>(a, max_tiles, s);
}

}  // namespace

bool i4_tile_info(int tile, TileInfo *info) {
#define I4INFO(id, bm, bn, st, wm, wn)                     \
    if (tile == id) {                                      \
        *info = TileInfo{bm, bn, 256, wm, wn, st, 16};     \
        return true;                                       \
    }
    I4_TILES(I4INFO)
#undef I4INFO
    return false;
}

hipError_t launch_gemm_i4(int tile, GemmKind kind, bool partial, const GemmArgs &a, int64_t max_tiles,
                          hipStream_t s) {
#define I4LAUNCH(id, bm, bn, st, wm, wn) \
    if (tile == id) return launch_kind<ICfg<bm, bn, st, wm, wn>>(kind, partial, a, max_tiles, s);
    I4_TILES(I4LAUNCH)
#undef I4LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace moe
