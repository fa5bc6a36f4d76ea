// gemm_pipe.hip -- the grouped GEMMs with a multi-stage direct-to-LDS pipeline (bf16, fp8;
// int4 in gemm_i4.hip).
//
// Same tiles, tile order and epilogues as gemm.hip, but the operands never pass through
// VGPRs: gfx950's global_load_lds_dwordx4 moves 16 bytes per lane from HBM/L2 straight into
// LDS, so ST stages of the K loop can be in flight at once (the register-staged kernels keep
// one).  A stage holds KS "slabs"; a slab is 128 bytes of K (64 bf16 / 128 E4M3) for every
// A row and B row of the tile.  One wave instruction fills 8 rows x 128 bytes of one slab;
// to keep the MFMA fragment reads free of bank conflicts without padding (the DMA writes
// LDS contiguously), chunk c (16 bytes) of row r is stored at position c ^ swz(r) with
// swz(r) = (r >> 1) & 7: a pair of rows shares a position but sits in the other half of
// the 64 banks, and 8 pairs cover all positions -- measured on gfx950 at the full
// ds_read_b128 rate for both the 16x16 and the 32x32 fragment patterns, where c ^ (r & 7)
// loses 20-35% to conflicts.  Lane l of an instruction (8 rows from a multiple of 8)
// therefore fetches the chunk (l & 7) ^ swz(row of l).  The fp8 tiles, whose fragment reads
// take chunks 2g and 2g + 1, use the key that is conflict-free for that pattern (pipe.h).
//
// K loop, per step kt: wait until this wave's loads of stage kt have landed (s_waitcnt
// vmcnt with the later stages still counted), s_barrier (so every wave's part has
// landed, and every wave is done reading the buffer about to be refilled), issue the loads
// of stage kt + ST - 1 into that buffer, then run the MFMAs of stage kt.  The barrier is a
// plain s_barrier: a __syncthreads() fence would make the compiler drain every in-flight
// load at each step.
#include "common.h"
#include "kernels.h"
#include "pipe.h"

namespace moe {
namespace {

enum { WT_BF16 = 0, WT_FP8 = 2, WT_INT4 = 3 };

template <int WT, int BM_, int BN_, int KS_, int ST_, int WM_, int WN_, int MS_, int SB_, int BX_ = 0, int IL_ = 0,
          int XT_ = 0>
struct PCfg {
    static constexpr int BM = BM_, BN = BN_, KS = KS_, ST = ST_, WM = WM_, WN = WN_;
    // BX = 1 (-1): B (A) gets one stage more than the other operand, each operand in a ring
    // of its own, so its loads run two K steps ahead while the other's run one (two
    // stages; 160 KB of LDS for a 256x256 tile)
    static constexpr int BX = BX_;
    // IL = 1 (bf16, 16x16 MFMAs, every buffer filled ahead): each wave holds the fragments of
    // two 32-K substeps in registers and reads the next substep's while the MFMAs of the
    // current one run (interleaved by the scheduler); the stage barrier sits between a
    // stage's last two substeps, so the next stage's first fragments are read while that
    // stage's last MFMAs run.  Built for 8 waves of 64x64 each (a 128x256 or 256x128 tile):
    // at two waves per SIMD a lane has 256 registers, room for two fragment sets beside the
    // accumulators.
    static constexpr int IL = IL_;
    // XT = 1: a unit's epilogue is deferred into the next unit's start, after that unit's
    // first stages are issued, so their loads land while the stores go out (the units of a
    // round otherwise read, compute and store in lockstep across the device: the first-stage
    // wait and the store burst add up per unit, which dominates at short K)
    static constexpr int XT = XT_;
    static_assert(!IL || (WT == WT_BF16 && MS_ == 16 && BX == 0 && SB_ == 128 && KS == 1),
                  "interleaved fragments: bf16 16x16 tiles of one 128-byte slab per stage");
    static constexpr int DA = ST + (BX < 0), DB = ST + (BX > 0);   // ring depths
    static constexpr int MS = MS_;                            // MFMA output tile: 16x16 or 32x32
    static constexpr int SB = SB_;                            // bytes of K per row and slab: 128 or 64
    static constexpr int SWZ = WT == WT_FP8 ? 1 : 0;          // LDS layout key (pipe.h: swz_key)
    static constexpr int NW = WM * WN, NT = NW * kWave;
    static constexpr int SLAB_K = WT == WT_FP8 ? SB : SB / 2; // K elements in a slab row
    static constexpr int BK = KS * SLAB_K;
    static constexpr int TM = BM / WM, TN = BN / WN, FM = TM / MS, FN = TN / MS;
    static constexpr int RPI = 1024 / SB;                     // rows one DMA instruction fills
    static constexpr int A_STAGE = KS * BM * SB, STAGE = KS * (BM + BN) * SB;
    static constexpr int A_LOADS = KS * BM / RPI, LOADS = KS * (BM + BN) / RPI;   // wave instructions per stage
    static constexpr int LPW = LOADS / NW;
    static_assert(LOADS % NW == 0, "stage loads must split evenly over the waves");
    static_assert(BM % (MS * WM) == 0 && BN % (MS * WN) == 0 && BM % RPI == 0, "tile / wave grid mismatch");
    static_assert(MS == 16 || (MS == 32 && WT == WT_BF16), "32x32 MFMA tiles are bf16 only");
    static_assert(SB == 128 || (SB == 64 && WT == WT_BF16), "64-byte slabs hold whole MFMA K steps for bf16 only");
    static_assert((ST - 2) * LPW <= 63, "vmcnt range");
    static constexpr int B_STAGE = STAGE - A_STAGE;
    static constexpr int LA = A_LOADS / NW, LB = (LOADS - A_LOADS) / NW;   // per wave and stage
    static constexpr int L_AHEAD = BX > 0 ? LB : LA;
    static_assert(BX == 0 || ((BX == 1 || BX == -1) && ST == 2 && A_LOADS % NW == 0),
                  "the one-operand-ahead rings are built for two stages with loads split evenly per wave");
    static constexpr int LDS_BYTES = BX ? DA * A_STAGE + DB * B_STAGE : ST * STAGE;
    // 4-wave tiles of at most 80 KB of LDS are built for two workgroups per CU: at most 256
    // registers a lane (two waves per SIMD)
    static constexpr int MINW = NW == 4 && LDS_BYTES <= 80 * 1024 ? 2 : 1;
    // LDS offsets of step k's A and B
    static __device__ __forceinline__ int a_off(int k) { return BX ? (k % DA) * A_STAGE : (k % ST) * STAGE; }
    static __device__ __forceinline__ int b_off(int k) {
        return BX ? DA * A_STAGE + (k % DB) * B_STAGE : (k % ST) * STAGE + A_STAGE;
    }
    // skip loading A's filler rows: worth it where a block is mostly padding (small blocks,
    // small T); large tiles keep the registers the per-load flags would take
    static constexpr bool SKIP_FILLER = BM <= 32;
};

template <class C, int WT, int KIND, bool PARTIAL>
__global__ __launch_bounds__(C::NT, C::MINW) void k_gemm_pipe(GemmArgs a) {
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];
    const int tid = threadIdx.x, lane = lane_id();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int npp = *a.npp;
    const int mblocks = npp / C::BM;
    const int n_out = KIND == GEMM_GATE_UP ? C::BN / 2 : C::BN;
    const int ntiles = a.N / n_out;
    const int mn = mblocks * ntiles;
    const int G = gridDim.x;
    const int nk = a.ksplit / C::BK;
    const int ebytes = WT == WT_FP8 ? 1 : 2;                  // A and B element bytes

    // Split tail (a GEMM without a K split): with one tile per workgroup and round, a last
    // round of rem = mn % G tiles leaves G - rem workgroups idle.  When the row blocks
    // holding those tiles make at most half a round, they are computed as S K splits
    // instead (fp32 planes, added in order by the reduce step after GEMM2, or by the
    // finishing pass that applies SiLU * up after GEMM1): after the whole rounds of the
    // other blocks, S x their tiles units of 1/S of the work fill the grid.  A plane row
    // holds GEMM2's H outputs, or GEMM1's I gate then I up sums.
    constexpr bool TAIL = !PARTIAL;
    const int tail_ld = KIND == GEMM_GATE_UP ? 2 * a.I : (int)a.ldc;
    int mb_dp = mblocks, tail_s = 0, tail_tiles = 0;
    if constexpr (TAIL) {
        if (a.tail_split >= 2) {
            const int rem = mn % G;
            if (rem > 0) {
                const int tmb = (rem + ntiles - 1) / ntiles, tt = tmb * ntiles;
                const int sk = min(min(a.tail_split, G / tt), min(a.tail_cap / tt, nk));
                if (sk >= 2) {
                    mb_dp = mblocks - tmb;
                    tail_s = sk;
                    tail_tiles = tt;
                }
            }
            if (blockIdx.x == 0 && tid == 0) {
                a.tail_info[0] = block_rows(a, mb_dp, C::BM).row0;   // the tail's first row
                a.tail_info[1] = tail_s;
                a.tail_info[2] = (mblocks - mb_dp) * C::BM * tail_ld;
                a.tail_info[3] = 0;
            }
        }
    }
    const int mn_dp = mb_dp * ntiles;
    const int total = TAIL ? mn_dp + tail_tiles * tail_s : mn * a.split;
    const int64_t tail_plane = (int64_t)(mblocks - mb_dp) * C::BM * tail_ld;   // at least the tail's rows
    const int tail_row0 = tail_tiles ? block_rows(a, mb_dp, C::BM).row0 : 0;

    using Acc = typename AccOf<C::MS>::type;
    constexpr int NR = C::MS == 32 ? 16 : 4;              // accumulator values per lane per fragment
    Acc acc[C::FM][C::FN];
    // the epilogue of a unit (its accumulators in acc); before_stores() runs once, after the
    // epilogue's loads have landed and before its first store
    auto epilogue = [&](const bool tail, const int s, const int nt, const int e, const BlockRows br,
                        auto &&before_stores) {
        const int row0 = br.row0;
        // ---- epilogue: accumulator value i of fragment (fm, fn) is row frag_row(lane, i),
        //      column lane % MS of that fragment ----
        float scale = 1.0f;
        if constexpr (WT == WT_FP8) scale = a.a_scale[0] * a.b_scale[e];
        // before the first store: every load of the epilogue has landed (a wait placed later
        // would also wait for whatever before_stores issues)
        auto ready = [&]() {
            pin(scale);
            before_stores();
        };
        const int lcol = lane & (C::MS - 1);
        // The rows of this lane's accumulators, q = fm * NR + i, in chunks of at most 16: a
        // chunk's pairs (and GEMM2's weights) are read and pinned before its stores (see pin)
        constexpr int EQ = C::FM * NR, EQC = EQ < 16 ? EQ : 16;
        // a chunk's loads pinned together where the tile has room for them (up to 128 x 256
        // outputs, not the 16-wave tiles of 32 x 32 fragments); the others pin value by value
        // and take the weight times the scale per value, which spills less there
        constexpr int PG = C::BM * C::BN <= 128 * 256 && !(C::NW >= 16 && C::MS == 32) ? EQC : 1;
        auto epi_row = [&](int q) { return wm * C::TM + (q / NR) * C::MS + frag_row<C::MS>(lane, q % NR); };
        auto epi_pair = [&](int q) { return block_pair_nb(a, br, epi_row(q)); };
        if constexpr (KIND == GEMM_GATE_UP && PARTIAL) {
            // split K: this split's gate and up sums in fp32 (the finishing pass adds the
            // splits in order and applies SiLU * up); filler rows are left out
#pragma unroll
            for (int q0 = 0; q0 < EQ; q0 += EQC) {
                int pr[EQC];
#pragma unroll
                for (int j = 0; j < EQC; j++) pr[j] = epi_pair(q0 + j);
                pin_groups<1>(pr);
                if (q0 == 0) ready();
#pragma unroll
                for (int j = 0; j < EQC; j++) {
                    const int fm = (q0 + j) / NR, i = (q0 + j) % NR, row = row0 + epi_row(q0 + j);
                    if (pr[j] >= a.pairs) continue;
                    float *P = (float *)a.C + (int64_t)s * a.partial_stride + (int64_t)row * a.ldc;
#pragma unroll
                    for (int f = 0; f < C::FN / 2; f++) {
                        const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * C::MS + lcol;
                        P[col] = acc[fm][f][i] * scale;
                        P[a.I + col] = acc[fm][f + C::FN / 2][i] * scale;
                    }
                }
            }
        } else if (KIND == GEMM_GATE_UP && tail) {
            // split tail: this split's gate and up sums in fp32 (the finishing pass adds the
            // splits in order and applies SiLU * up; for fp8 it also folds |h|)
#pragma unroll
            for (int q0 = 0; q0 < EQ; q0 += EQC) {
                int pr[EQC];
#pragma unroll
                for (int j = 0; j < EQC; j++) pr[j] = epi_pair(q0 + j);
                pin_groups<1>(pr);
                if (q0 == 0) ready();
#pragma unroll
                for (int j = 0; j < EQC; j++) {
                    const int fm = (q0 + j) / NR, i = (q0 + j) % NR, row = row0 + epi_row(q0 + j);
                    if (pr[j] >= a.pairs) continue;
                    float *P = a.tail_P + s * tail_plane + (int64_t)(row - tail_row0) * tail_ld;
#pragma unroll
                    for (int f = 0; f < C::FN / 2; f++) {
                        const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * C::MS + lcol;
                        P[col] = acc[fm][f][i] * scale;
                        P[a.I + col] = acc[fm][f + C::FN / 2][i] * scale;
                    }
                }
            }
        } else if constexpr (KIND == GEMM_GATE_UP) {
            float amax = 0.0f;
            uint32_t seen = 0;   // the h maximum so far, read before the stores (see amax_peek)
            if constexpr (WT == WT_FP8)
                if (lane == 0 && a.amax_out) seen = amax_peek(a.amax_out);
#pragma unroll
            for (int q0 = 0; q0 < EQ; q0 += EQC) {
                bool valid[EQC];   // |h| of filler rows stays out of the maximum (fp8 only)
                if constexpr (WT == WT_FP8) {
                    int pr[EQC];
#pragma unroll
                    for (int j = 0; j < EQC; j++) pr[j] = epi_pair(q0 + j);
                    pin_groups<1>(pr);
#pragma unroll
                    for (int j = 0; j < EQC; j++) valid[j] = pr[j] < a.pairs;
                } else {
#pragma unroll
                    for (int j = 0; j < EQC; j++) valid[j] = true;
                }
                if (q0 == 0) {   // the maximum so far has landed too
                    pin(seen);
                    ready();
                }
#pragma unroll
                for (int j = 0; j < EQC; j++) {
                    const int fm = (q0 + j) / NR, i = (q0 + j) % NR, lr = epi_row(q0 + j), row = row0 + lr;
                    // without padding the rows past the block are the next block's: not written
                    if (lr >= br.n) continue;
#pragma unroll
                    for (int f = 0; f < C::FN / 2; f++) {
                        const float g = acc[fm][f][i] * scale, u = acc[fm][f + C::FN / 2][i] * scale;
                        const float hv = silu(g) * u;
                        const int col = nt * (C::BN / 2) + wn * (C::TN / 2) + f * C::MS + lcol;
                        if constexpr (WT == WT_FP8) {
                            ((float *)a.C)[(int64_t)row * a.ldc + col] = hv;
                            if (valid[j]) amax = fmaxf(amax, fabsf(hv));
                        } else {
                            ((uint16_t *)a.C)[(int64_t)row * a.ldc + col] = f32_to_bf16_bits(hv);
                        }
                    }
                }
            }
            if constexpr (WT == WT_FP8) {
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
                if (lane == 0 && a.amax_out) amax_raise(a.amax_out, seen, amax);
            }
        } else {
            // per chunk of rows: every row's pair, then every row's weight, then the stores
#pragma unroll
            for (int q0 = 0; q0 < EQ; q0 += EQC) {
                int pr[EQC];
                float wr[EQC];
#pragma unroll
                for (int j = 0; j < EQC; j++) pr[j] = epi_pair(q0 + j);
                pin_groups<PG>(pr);
                if (a.topk_w && PG > 1) {   // filler rows read pair 0's weight
#pragma unroll
                    for (int j = 0; j < EQC; j++) wr[j] = a.topk_w[pr[j] < a.pairs ? pr[j] : 0];
                    pin_groups<PG>(wr);
#pragma unroll
                    for (int j = 0; j < EQC; j++) wr[j] *= scale;
                } else {
                    if (a.topk_w) {
#pragma unroll
                        for (int j = 0; j < EQC; j++) wr[j] = a.topk_w[pr[j] < a.pairs ? pr[j] : 0] * scale;
                    } else {      // the grouped GEMM has no weight
#pragma unroll
                        for (int j = 0; j < EQC; j++) wr[j] = scale;
                    }
                    pin_groups<1>(wr);
                }
                if (q0 == 0) ready();
#pragma unroll
                for (int j = 0; j < EQC; j++) {
                    const int fm = (q0 + j) / NR, i = (q0 + j) % NR;
                    const int lr = epi_row(q0 + j), row = row0 + lr, p = pr[j];
                    if (p >= a.pairs) continue;   // filler row: never read back
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++) {
                        const int col = nt * C::BN + wn * C::TN + fn * C::MS + lcol;
                        const float v = acc[fm][fn][i] * wr[j];
                        if constexpr (PARTIAL)
                            ((float *)a.C)[(int64_t)s * a.partial_stride + (int64_t)row * a.ldc + col] = v;
                        else if (tail)
                            a.tail_P[s * tail_plane + (int64_t)(row - tail_row0) * a.ldc + col] = v;
                        else
                            ((uint16_t *)a.C)[(a.out_by_pair ? (int64_t)p : row) * a.ldc + col] = f32_to_bf16_bits(v);
                    }
                }
            }
        }
    };
    // XT: the unit whose epilogue is pending
    bool pv_valid = false, pv_tail = false;
    int pv_s = 0, pv_nt = 0, pv_e = 0;
    BlockRows pv_br{0, 0};

    for (int tile = xcd_first_tile(blockIdx.x, G); tile < total; tile += G) {
        // unit: whole-K tile (or one of split_k splits), or one split of a tail tile
        const bool tail = TAIL && tile >= mn_dp;
        const TileCoord tc = tail ? tile_coord(tile - mn_dp, tail_tiles, mblocks - mb_dp, ntiles, a.group_m)
                             : a.expert_groups ? tile_coord_expert(tile, mn_dp, mb_dp, ntiles, a.eids, a.expert_groups)
                                               : tile_coord(tile, mn_dp, mb_dp, ntiles, a.group_m);
        const int s = tc.s, mb = tail ? mb_dp + tc.mb : tc.mb, nt = tc.nt;
        const int kbeg = tail ? s * nk / tail_s : s * nk;     // first K step and number of steps
        const int nku = tail ? (s + 1) * nk / tail_s - kbeg : nk;
        // the block's expert and rows through the scalar cache (see sload)
        const int e = sload(a.eids + mb);
        BlockRows br{mb * C::BM, C::BM};
        if (a.blk_start) {
            const int2 be = sload_pair(a.blk_start + mb);
            br = BlockRows{be.x, be.y - be.x};
        }
        const int row0 = br.row0;   // first row of the block in h / y (the layout's)
        const int64_t kb = (int64_t)kbeg * C::BK * ebytes;    // byte offset of this unit's K

        // per load instruction q of this wave: operand (A or B), the lane's byte offset from
        // the operand's base at the split's first K, and the wave's LDS offset in a stage
        uint32_t voff[C::LPW];
        int dst[C::LPW];
        bool is_a[C::LPW];
        bool on[C::LPW];   // lane loads (filler rows of A are skipped, see below)
#pragma unroll
        for (int q = 0; q < C::LPW; q++) {
            on[q] = true;
            const int ins = wave + q * C::NW;
            is_a[q] = ins < C::A_LOADS;
            if (ins < C::A_LOADS) {
                const int slab = ins / (C::BM / C::RPI), rb = ins % (C::BM / C::RPI) * C::RPI;
                int r, chunk;
                dma_lane<C::SB, C::SWZ>(lane, rb, r, chunk);
                const int p = block_pair(a, br, r);
                // a row past the block's pairs reads its block's first row (in bounds; its
                // products are never stored)
                const int64_t arow = KIND == GEMM_GATE_UP ? (p < a.pairs ? p / a.top_k : 0)
                                     : a.gather_a       ? (p < a.pairs ? p : 0)
                                                        : row0 + (r < br.n ? r : 0);
                // a filler row's products are never read back, so its LDS row may keep stale
                // data; the lanes of the instruction's first row always load, so every load
                // instruction runs with a non-empty mask and counts in vmcnt
                on[q] = !C::SKIP_FILLER || p < a.pairs || (lane >> 3) == 0;
                voff[q] = (uint32_t)(arow * a.lda * ebytes + slab * C::SB + chunk * 16);
                dst[q] = (slab * C::BM + rb) * C::SB;
            } else {
                const int j = ins - C::A_LOADS;
                const int slab = j / (C::BN / C::RPI), rb = j % (C::BN / C::RPI) * C::RPI;
                int rr, chunk;
                dma_lane<C::SB, C::SWZ>(lane, rb, rr, chunk);
                int64_t grow;
                if (KIND == GEMM_GATE_UP) {   // LDS rows of wave column w: its gate half, then its up half
                    const int wcol = rr / C::TN, i = rr % C::TN, half = C::TN / 2;
                    const int col = nt * (C::BN / 2) + wcol * half + (i % half);
                    grow = i < half ? col : a.I + col;
                } else {
                    grow = (int64_t)nt * C::BN + rr;
                }
                voff[q] = (uint32_t)(grow * a.ldb + slab * C::SB + chunk * 16);
                dst[q] = C::A_STAGE + (slab * C::BN + rb) * C::SB;
            }
        }
        // with rotate_k (weight streaming: about one block of rows per expert) each tile walks
        // its K range from its own starting step, cyclically, so that concurrent tiles spread
        // over DRAM channels instead of all reading the same column slice of rows that share
        // address bits.  The start depends on the expert and the column tile, not on the row
        // block, so that the blocks of an expert with more rows than one block stream their
        // common weight tile in step (L2 reuse); without rotate_k every tile keeps K in step.
        // The order is fixed per tile, so results stay reproducible.
        const int krot = a.rotate_k ? (nt * 3 + e * 5) % nku : 0;
        const char *base_a = uniform_ptr((const char *)a.A + kb);
        const char *base_b = uniform_ptr((const char *)a.B + (int64_t)e * a.b_expert_stride + kb);
        // the loads of step kstep: A's, B's or both (dst holds B's offsets past A_STAGE)
        auto issue = [&](int kstep, bool do_a, bool do_b) {
            const uint32_t sta = lds_addr(smem) + C::a_off(kstep);
            const uint32_t stb = lds_addr(smem) + C::b_off(kstep) - C::A_STAGE;
            const int kr = __builtin_amdgcn_readfirstlane(kstep + krot < nku ? kstep + krot : kstep + krot - nku);
            const int64_t koff = (int64_t)kr * C::KS * C::SB;
#pragma unroll
            for (int q = 0; q < C::LPW; q++)
                if (on[q] && (is_a[q] ? do_a : do_b))
                    lds_dma_off<16>((is_a[q] ? base_a : base_b) + koff, voff[q], (is_a[q] ? sta : stb) + dst[q]);
        };

        // A block holds its expert's rows first and padding after them, so a wave row range
        // with no real row starts with padding: such waves (the tail block of an expert at
        // large block heights) skip their LDS reads and MFMAs but still load and synchronise
        const bool wave_rows = __builtin_amdgcn_readfirstlane(block_pair(a, br, wm * C::TM) < a.pairs);
        // this unit's first stages (after every wave is done with the previous unit's buffers)
        auto start_stages = [&]() {
            block_barrier();
            if constexpr (C::IL) {
#pragma unroll
                for (int p = 0; p < C::ST; p++)
                    if (p < nku) issue(p, true, true);
            } else {
#pragma unroll
                for (int p = 0; p < C::ST - 1; p++)
                    if (p < nku) issue(p, true, true);
                if constexpr (C::BX != 0)   // the operand that runs ahead: its step 1 too
                    if (1 < nku) issue(1, C::BX < 0, C::BX > 0);
            }
        };
        if constexpr (C::XT) {
            if (pv_valid) epilogue(pv_tail, pv_s, pv_nt, pv_e, pv_br, start_stages);
            else start_stages();
        } else {
            start_stages();
        }
#pragma unroll
        for (int i = 0; i < C::FM; i++)
#pragma unroll
            for (int j = 0; j < C::FN; j++)
#pragma unroll
                for (int r = 0; r < NR; r++) acc[i][j][r] = 0.f;

        if constexpr (C::IL) {
            // every buffer filled ahead; a stage's buffer is refilled after the barrier that
            // follows every wave's last read of it
            constexpr int NK = C::SB / 64;                  // 32-K substeps per stage (2)
            bf16x8 af[2][C::FM], bfr[2][C::FN];
            // fragments of substep q of stage k into set buf: lane l holds row l % 16 and K
            // elements 8 (l / 16) .. +7 of the substep
            auto frag_load = [&](int k, int q, int buf) {
                const char *sa = smem + C::a_off(k), *sb = smem + C::b_off(k);
                const int ci = q * 4 + (lane >> 4);
#pragma unroll
                for (int fm = 0; fm < C::FM; fm++)
                    af[buf][fm] = *(const bf16x8 *)(sa + slab_off<C::SB, C::SWZ>(wm * C::TM + fm * 16 + (lane & 15), ci));
#pragma unroll
                for (int fn = 0; fn < C::FN; fn++)
                    bfr[buf][fn] = *(const bf16x8 *)(sb + slab_off<C::SB, C::SWZ>(wn * C::TN + fn * 16 + (lane & 15), ci));
            };
            auto mma = [&](int buf) {
#pragma unroll
                for (int fm = 0; fm < C::FM; fm++)
#pragma unroll
                    for (int fn = 0; fn < C::FN; fn++)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[buf][fm], bfr[buf][fn], acc[fm][fn], 0, 0, 0);
            };
            // the reads issued above go between the MFMAs: one read after every few MFMAs
            auto interleave = [&]() {
                constexpr int NR = C::FM + C::FN, NM = C::FM * C::FN, PER = NM / NR;
#pragma unroll
                for (int i = 0; i < NR; i++) {
                    __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);   // MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // LDS read
                }
                __builtin_amdgcn_sched_group_barrier(0x008, NM - PER * NR, 0);
            };
            // stage 0 landed (later stages may still be in flight)
            wait_stages<C::LPW, C::ST - 1>(min(C::ST - 1, nku - 1));
            block_barrier();
            if (wave_rows) frag_load(0, 0, 0);
            for (int kt = 0; kt < nku; kt++) {
#pragma unroll
                for (int q = 0; q < NK; q++) {
                    const int cur = q & 1;
                    if (q + 1 < NK) {
                        if (wave_rows) {
                            frag_load(kt, q + 1, cur ^ 1);
                            mma(cur);
                            interleave();
                        }
                    } else {
                        if (kt + 1 < nku) {
                            // this wave's reads of stage kt done, stage kt + 1 landed; after the
                            // barrier no wave reads stage kt's buffer any more: refill it
                            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                            wait_stages<C::LPW, C::ST - 1>(min(C::ST - 2, nku - 2 - kt));
                            block_barrier();
                            if (kt + C::ST < nku) issue(kt + C::ST, true, true);
                            if (wave_rows) {
                                frag_load(kt + 1, 0, cur ^ 1);
                                mma(cur);
                                interleave();
                            }
                        } else if (wave_rows) {
                            mma(cur);
                        }
                    }
                }
            }
        } else {
            for (int kt = 0; kt < nku; kt++) {
                if constexpr (C::BX != 0) {
                    // issued after this step's last operand: the ahead operand's step kt + 1, if
                    // it exists (two stages)
                    if (kt + 1 < nku) wait_vmcnt<C::L_AHEAD>(); else wait_vmcnt<0>();
                } else {
                    wait_stages<C::LPW, C::ST - 2>(min(C::ST - 2, nku - 1 - kt));
                }
                block_barrier();
                // the operand one step ahead, then (ahead rings) the other two steps ahead
                if (kt + C::ST - 1 < nku) issue(kt + C::ST - 1, C::BX >= 0, C::BX <= 0);
                if constexpr (C::BX != 0)
                    if (kt + 2 < nku) issue(kt + 2, C::BX < 0, C::BX > 0);
                const char *sa = smem + C::a_off(kt), *sb = smem + C::b_off(kt);
                if (wave_rows) {   // a wave whose rows are all padding only loads and keeps step
                // Fragments of step k + 1 can be read while the MFMAs of step k run (see DB below).
                if constexpr (WT == WT_BF16 && C::MS == 32) {
                    // 32x32x16: lane l holds row l%32, K elements 8*(l/32) .. +7 of the step.
                    // Double-buffered: the reads of step k + 1 are issued before the MFMAs of
                    // step k (scheduling barriers keep that order).
                    constexpr int KPS = C::SB / 32;                 // 16-K steps per slab
                    constexpr int NK = C::KS * KPS;
                    bf16x8 af[2][C::FM], bfr[2][C::FN];
                    auto load = [&](int k, int buf) {
                        const int sl = k / KPS, ci = (k % KPS) * 2 + (lane >> 5);
    #pragma unroll
                        for (int fm = 0; fm < C::FM; fm++) {
                            const int r = wm * C::TM + fm * 32 + (lane & 31);
                            af[buf][fm] = *(const bf16x8 *)(sa + sl * C::BM * C::SB + slab_off<C::SB, C::SWZ>(r, ci));
                        }
    #pragma unroll
                        for (int fn = 0; fn < C::FN; fn++) {
                            const int r = wn * C::TN + fn * 32 + (lane & 31);
                            bfr[buf][fn] = *(const bf16x8 *)(sb + sl * C::BN * C::SB + slab_off<C::SB, C::SWZ>(r, ci));
                        }
                    };
                    load(0, 0);
    #pragma unroll
                    for (int k = 0; k < NK; k++) {
                        if (k + 1 < NK) load(k + 1, (k + 1) & 1);
                        __builtin_amdgcn_sched_barrier(0);
    #pragma unroll
                        for (int fm = 0; fm < C::FM; fm++)
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++)
                                acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[k & 1][fm], bfr[k & 1][fn],
                                                                                     acc[fm][fn], 0, 0, 0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else if constexpr (WT == WT_BF16 && C::NW >= 16) {
                    // 16 waves (128 registers a lane): all FM A fragments do not fit beside the
                    // accumulators, so A is read two fragments deep: A(fm + 1) is read from LDS
                    // before the MFMAs of A(fm) are issued, and its latency is spent under them
                    // (scheduling groups keep that order; the MFMA sequence is unchanged)
    #pragma unroll
                    for (int sl = 0; sl < C::KS; sl++)
    #pragma unroll
                        for (int kk = 0; kk < C::SB / 64; kk++) {
                            const int ci = kk * 4 + (lane >> 4);
                            const char *pa = sa + sl * C::BM * C::SB, *pb = sb + sl * C::BN * C::SB;
                            bf16x8 af[2], bfr[C::FN];
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++)
                                bfr[fn] = *(const bf16x8 *)(pb + slab_off<C::SB, C::SWZ>(wn * C::TN + fn * 16 + (lane & 15), ci));
                            af[0] = *(const bf16x8 *)(pa + slab_off<C::SB, C::SWZ>(wm * C::TM + (lane & 15), ci));
    #pragma unroll
                            for (int fm = 0; fm < C::FM; fm++) {
                                if (fm + 1 < C::FM)
                                    af[(fm + 1) & 1] = *(const bf16x8 *)(pa + slab_off<C::SB, C::SWZ>(
                                                                            wm * C::TM + (fm + 1) * 16 + (lane & 15), ci));
    #pragma unroll
                                for (int fn = 0; fn < C::FN; fn++)
                                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm & 1], bfr[fn], acc[fm][fn], 0, 0, 0);
                            }
                            __builtin_amdgcn_sched_group_barrier(0x100, C::FN + 1, 0);   // B, A(0)
    #pragma unroll
                            for (int fm = 0; fm < C::FM; fm++) {
                                if (fm + 1 < C::FM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // A(fm + 1)
                                __builtin_amdgcn_sched_group_barrier(0x008, C::FN, 0);                   // MFMAs of A(fm)
                            }
                        }
                } else if constexpr (WT == WT_BF16) {
    #pragma unroll
                    for (int sl = 0; sl < C::KS; sl++)
    #pragma unroll
                        for (int kk = 0; kk < C::SB / 64; kk++) {
                            // 16x16x32: lane l holds row l%16, K elements 8*(l/16) .. +7 of the step
                            const int ci = kk * 4 + (lane >> 4);
                            bf16x8 af[C::FM], bfr[C::FN];
    #pragma unroll
                            for (int fm = 0; fm < C::FM; fm++) {
                                const int r = wm * C::TM + fm * 16 + (lane & 15);
                                af[fm] = *(const bf16x8 *)(sa + sl * C::BM * C::SB + slab_off<C::SB, C::SWZ>(r, ci));
                            }
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++) {
                                const int r = wn * C::TN + fn * 16 + (lane & 15);
                                bfr[fn] = *(const bf16x8 *)(sb + sl * C::BN * C::SB + slab_off<C::SB, C::SWZ>(r, ci));
                            }
    #pragma unroll
                            for (int fm = 0; fm < C::FM; fm++)
    #pragma unroll
                                for (int fn = 0; fn < C::FN; fn++)
                                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
                        }
                } else if constexpr (C::NW >= 16) {
                    // fp8 with 16 waves (128 registers a lane): all A fragments of the slab, then
                    // the B fragments one or two at a time
                    const int c0 = 2 * (lane >> 4);
                    // where two B fragments fit beside the A fragments and the accumulators
                    // (wave tiles of 32x64 and 64x32), B(fn + 1) is read before the MFMAs of
                    // B(fn) are issued, so that its latency is spent under them
                    constexpr bool B2 = 8 * (C::FM + 2) + 4 * C::FM * C::FN <= 96;
                    auto frag = [&](const char *slab, int r) {
                        const uint4 lo = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0));
                        const uint4 hi = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0 + 1));
                        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    };
    #pragma unroll
                    for (int sl = 0; sl < C::KS; sl++) {
                        i32x8 af[C::FM];
    #pragma unroll
                        for (int fm = 0; fm < C::FM; fm++)
                            af[fm] = frag(sa + sl * C::BM * 128, wm * C::TM + fm * 16 + (lane & 15));
                        if constexpr (B2) {
                            const char *slab = sb + sl * C::BN * 128;
                            i32x8 bfr[2];
                            bfr[0] = frag(slab, wn * C::TN + (lane & 15));
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++) {
                                if (fn + 1 < C::FN) bfr[(fn + 1) & 1] = frag(slab, wn * C::TN + (fn + 1) * 16 + (lane & 15));
    #pragma unroll
                                for (int fm = 0; fm < C::FM; fm++)
                                    acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                        af[fm], bfr[fn & 1], acc[fm][fn], 0, 0, 0, 127, 0, 127);
                            }
                            __builtin_amdgcn_sched_group_barrier(0x100, 2 * C::FM + 2, 0);   // A, B(0)
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++) {
                                if (fn + 1 < C::FN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // B(fn + 1)
                                __builtin_amdgcn_sched_group_barrier(0x008, C::FM, 0);                   // MFMAs of B(fn)
                            }
                        } else {   // one B fragment at a time: fragments take 8 (FM + 1) registers
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++) {
                                const i32x8 b = frag(sb + sl * C::BN * 128, wn * C::TN + fn * 16 + (lane & 15));
    #pragma unroll
                                for (int fm = 0; fm < C::FM; fm++)
                                    acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[fm], b, acc[fm][fn], 0, 0,
                                                                                                0, 127, 0, 127);
                                __builtin_amdgcn_sched_barrier(0);   // keep the B loads from being hoisted together
                            }
                        }
                    }
                } else {   // fp8: one 16x16x128 MFMA per slab; a lane's 32 bytes are two swizzled chunks
                    const int c0 = 2 * (lane >> 4);
                    i32x8 af[2][C::FM], bfr[2][C::FN];
                    auto load = [&](int sl, int buf) {
    #pragma unroll
                        for (int fm = 0; fm < C::FM; fm++) {
                            const int r = wm * C::TM + fm * 16 + (lane & 15);
                            const char *slab = sa + sl * C::BM * 128;
                            const uint4 lo = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0));
                            const uint4 hi = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0 + 1));
                            af[buf][fm] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                                (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        }
    #pragma unroll
                        for (int fn = 0; fn < C::FN; fn++) {
                            const int r = wn * C::TN + fn * 16 + (lane & 15);
                            const char *slab = sb + sl * C::BN * 128;
                            const uint4 lo = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0));
                            const uint4 hi = *(const uint4 *)(slab + slab_off<128, C::SWZ>(r, c0 + 1));
                            bfr[buf][fn] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                                 (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        }
                    };
                    load(0, 0);
    #pragma unroll
                    for (int sl = 0; sl < C::KS; sl++) {
                        if (sl + 1 < C::KS) load(sl + 1, (sl + 1) & 1);
    #pragma unroll
                        for (int fm = 0; fm < C::FM; fm++)
    #pragma unroll
                            for (int fn = 0; fn < C::FN; fn++)
                                acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                    af[sl & 1][fm], bfr[sl & 1][fn], acc[fm][fn], 0, 0, 0, 127, 0, 127);
                    }
                }
                }
            }
        }

        if constexpr (C::XT) {
            pv_valid = true;
            pv_tail = tail;
            pv_s = s;
            pv_nt = nt;
            pv_e = e;
            pv_br = br;
        } else {
            epilogue(tail, s, nt, e, br, []() {});
        }
    }
    if constexpr (C::XT)
        if (pv_valid) epilogue(pv_tail, pv_s, pv_nt, pv_e, pv_br, []() {});
}

// ---- tile tables (ids continue gemm.hip's per weight type) --------------------------------
// Tiles of at most 80 KB of LDS and 4 waves (bf16 44/45, fp8 19/20: two stages of a 128x128
// or 64x256 tile) run two workgroups per CU, so one can load or store while the other
// computes: for short K (the fp8 GEMM2 of a small I) a tile's fill and epilogue are a large
// part of its time.
//        id  BM   BN  KS ST WM WN MS  SB
#define PIPE_BF16_TILES(X)              \
    X(7, 128, 256, 1, 3, 2, 2, 16, 128)      \
    X(8, 128, 128, 1, 4, 2, 2, 16, 128)      \
    X(9, 16, 128, 2, 4, 1, 4, 16, 128)       \
    X(10, 16, 64, 4, 3, 1, 2, 16, 128)       \
    X(11, 64, 128, 1, 4, 2, 2, 16, 128)      \
    X(12, 32, 128, 2, 3, 1, 4, 16, 128)      \
    X(13, 128, 256, 1, 3, 2, 2, 32, 128)     \
    X(14, 128, 128, 1, 4, 2, 2, 32, 128)     \
    X(15, 64, 128, 1, 4, 2, 2, 32, 128)      \
    X(16, 256, 128, 1, 3, 2, 2, 32, 128)     \
    X(18, 64, 256, 1, 4, 1, 4, 32, 128)      \
    X(19, 32, 256, 1, 4, 1, 4, 32, 128)      \
    X(20, 256, 256, 1, 2, 2, 4, 16, 128)     \
    X(21, 256, 256, 1, 2, 2, 4, 32, 128)     \
    X(22, 128, 256, 1, 3, 2, 4, 16, 128)     \
    X(23, 256, 128, 1, 3, 4, 2, 16, 128)     \
    X(24, 256, 256, 1, 2, 4, 4, 32, 128)     \
    X(25, 256, 256, 1, 2, 4, 4, 16, 128)     \
    X(26, 128, 256, 1, 3, 4, 4, 32, 128)     \
    X(27, 256, 128, 1, 3, 4, 2, 32, 128)     \
    X(28, 128, 256, 1, 3, 2, 4, 32, 128)     \
    X(29, 256, 128, 1, 3, 4, 2, 16, 128) \
    X(30, 256, 256, 1, 4, 4, 4, 16, 64)  \
    X(31, 256, 256, 1, 4, 2, 4, 32, 64)  \
    X(32, 256, 256, 1, 4, 2, 4, 16, 64)  \
    X(33, 256, 256, 1, 5, 4, 4, 16, 64)  \
    X(34, 256, 256, 1, 5, 2, 4, 32, 64)  \
    X(35, 256, 128, 1, 5, 4, 2, 32, 64)  \
    X(36, 128, 256, 1, 5, 2, 4, 32, 64)  \
    X(37, 256, 128, 1, 3, 4, 4, 16, 128) \
    X(44, 128, 128, 1, 2, 2, 2, 16, 128) \
    X(45, 64, 256, 1, 2, 1, 4, 16, 128)
#define PIPE_FP8_TILES(X)               \
    X(7, 128, 256, 1, 3, 2, 2, 16, 128)      \
    X(8, 128, 128, 1, 4, 2, 2, 16, 128)      \
    X(9, 16, 128, 2, 4, 1, 4, 16, 128)       \
    X(10, 64, 128, 1, 4, 2, 2, 16, 128)      \
    X(11, 32, 128, 2, 3, 1, 4, 16, 128)      \
    X(12, 256, 256, 1, 2, 2, 4, 16, 128)     \
    X(13, 128, 256, 1, 3, 2, 4, 16, 128)     \
    X(14, 256, 256, 1, 2, 4, 4, 16, 128) \
    X(15, 256, 128, 1, 3, 4, 4, 16, 128) \
    X(16, 128, 256, 1, 3, 4, 4, 16, 128) \
    X(19, 128, 128, 1, 2, 2, 2, 16, 128) \
    X(20, 64, 256, 1, 2, 1, 4, 16, 128)
// tiles whose B (BX = 1) or A (BX = -1) runs a stage ahead of the other operand
//        id  BM   BN  KS ST WM WN MS  SB  BX
#define PIPE_BF16_TILES_BX(X) X(38, 256, 256, 1, 2, 4, 4, 16, 128, 1) X(39, 256, 256, 1, 2, 4, 4, 16, 128, -1)
#define PIPE_FP8_TILES_BX(X) X(17, 256, 256, 1, 2, 4, 4, 16, 128, 1) X(18, 256, 256, 1, 2, 4, 4, 16, 128, -1)
// deferred-epilogue twins (XT) of the large-T tiles
//        id  BM   BN  KS ST WM WN MS  SB  BX IL
#define PIPE_BF16_TILES_XT(X)                    \
    X(48, 256, 256, 1, 2, 4, 4, 16, 128, 0, 0)   \
    X(50, 256, 256, 1, 2, 4, 4, 16, 128, 1, 0)   \
    X(51, 128, 256, 1, 3, 2, 4, 16, 128, 0, 1)   \
    X(52, 256, 128, 1, 3, 4, 2, 16, 128, 0, 1)   \
    X(53, 128, 256, 1, 3, 2, 4, 16, 128, 0, 0)
#define PIPE_FP8_TILES_XT(X)                     \
    X(23, 128, 256, 1, 3, 4, 4, 16, 128, 0, 0)   \
    X(24, 128, 256, 1, 3, 2, 4, 16, 128, 0, 0)
// 8-wave tiles reading the next 32-K substep's fragments while the current MFMAs run (IL)
//        id  BM   BN  KS ST WM WN MS  SB
// (twins of tiles 22 and 23; a 128x64 wave tile with two fragment sets exceeds the 256
// registers a lane has at two waves per SIMD)
#define PIPE_BF16_TILES_IL(X)           \
    X(42, 128, 256, 1, 3, 2, 4, 16, 128)     \
    X(43, 256, 128, 1, 3, 4, 2, 16, 128)

template <class C, int WT, int KIND, bool PARTIAL>
hipError_t launch_one(const GemmArgs &a, int64_t max_tiles, hipStream_t s) {
    static int occ_cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    int occ = dev < 64 ? __atomic_load_n(&occ_cache[dev], __ATOMIC_RELAXED) : 0;
    if (occ == 0) {
        hipError_t err =
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, k_gemm_pipe<C, WT, KIND, PARTIAL>, C::NT, 0);
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
    // Large blocks: groups of an expert's blocks (at most 8) -- Mixtral T=4096 GEMM1 862 ->
    // 845 us, Scout T=8192 1520 -> 1460 us; the bf16 GEMM2 too (Scout T=4096 -1.4%, T=2048
    // -0.5%), while the fp8 GEMM2 of Qwen2 loses 5% with them and keeps group_m
    b.expert_groups = (KIND == GEMM_GATE_UP || WT == WT_BF16) && C::BM >= 128 ? 8 : 0;
    hipLaunchKernelGGL((k_gemm_pipe<C, WT, KIND, PARTIAL>), dim3((unsigned)grid), dim3(C::NT), 0, s, b);
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

bool pipe_tile_info(int wdtype, int tile, TileInfo *info) {
#define PINFO(WT, id, bm, bn, ks, st, wm, wn, ms, sb)                                      \
    if (tile == id) {                                                                      \
        *info = TileInfo{bm, bn, ks * (WT == WT_FP8 ? sb : sb / 2), wm, wn, st, ms};       \
        return true;                                                                       \
    }
#define PI_BF16(id, bm, bn, ks, st, wm, wn, ms, sb) PINFO(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PI_FP8(id, bm, bn, ks, st, wm, wn, ms, sb) PINFO(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PI_BF16_BX(id, bm, bn, ks, st, wm, wn, ms, sb, bx) PINFO(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PI_FP8_BX(id, bm, bn, ks, st, wm, wn, ms, sb, bx) PINFO(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PI_BF16_XT(id, bm, bn, ks, st, wm, wn, ms, sb, bx, il) PINFO(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PI_FP8_XT(id, bm, bn, ks, st, wm, wn, ms, sb, bx, il) PINFO(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb)
    if (wdtype == WT_BF16) {
        PIPE_BF16_TILES(PI_BF16) PIPE_BF16_TILES_BX(PI_BF16_BX) PIPE_BF16_TILES_IL(PI_BF16) PIPE_BF16_TILES_XT(PI_BF16_XT)
    }
    if (wdtype == WT_FP8) { PIPE_FP8_TILES(PI_FP8) PIPE_FP8_TILES_BX(PI_FP8_BX) PIPE_FP8_TILES_XT(PI_FP8_XT) }
    if (wdtype == WT_INT4) return i4_tile_info(tile, info);
    return false;
}

hipError_t launch_gemm_pipe(int wdtype, int tile, GemmKind kind, bool partial, const GemmArgs &a,
                            int64_t max_tiles, hipStream_t s) {
#define PLAUNCH(WT, id, bm, bn, ks, st, wm, wn, ms, sb) \
    if (tile == id) return launch_kind<PCfg<WT, bm, bn, ks, st, wm, wn, ms, sb>, WT>(kind, partial, a, max_tiles, s);
#define PL_BF16(id, bm, bn, ks, st, wm, wn, ms, sb) PLAUNCH(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PL_FP8(id, bm, bn, ks, st, wm, wn, ms, sb) PLAUNCH(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb)
#define PLAUNCH_BX(WT, id, bm, bn, ks, st, wm, wn, ms, sb, bx) \
    if (tile == id) return launch_kind<PCfg<WT, bm, bn, ks, st, wm, wn, ms, sb, bx>, WT>(kind, partial, a, max_tiles, s);
#define PL_BF16_BX(id, bm, bn, ks, st, wm, wn, ms, sb, bx) PLAUNCH_BX(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb, bx)
#define PL_FP8_BX(id, bm, bn, ks, st, wm, wn, ms, sb, bx) PLAUNCH_BX(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb, bx)
#define PL_BF16_IL(id, bm, bn, ks, st, wm, wn, ms, sb) \
    if (tile == id) return launch_kind<PCfg<WT_BF16, bm, bn, ks, st, wm, wn, ms, sb, 0, 1>, WT_BF16>(kind, partial, a, max_tiles, s);
#define PLAUNCH_XT(WT, id, bm, bn, ks, st, wm, wn, ms, sb, bx, il) \
    if (tile == id) return launch_kind<PCfg<WT, bm, bn, ks, st, wm, wn, ms, sb, bx, il, 1>, WT>(kind, partial, a, max_tiles, s);
#define PL_BF16_XT(id, bm, bn, ks, st, wm, wn, ms, sb, bx, il) PLAUNCH_XT(WT_BF16, id, bm, bn, ks, st, wm, wn, ms, sb, bx, il)
#define PL_FP8_XT(id, bm, bn, ks, st, wm, wn, ms, sb, bx, il) PLAUNCH_XT(WT_FP8, id, bm, bn, ks, st, wm, wn, ms, sb, bx, il)
    if (wdtype == WT_BF16) {
        PIPE_BF16_TILES(PL_BF16) PIPE_BF16_TILES_BX(PL_BF16_BX) PIPE_BF16_TILES_IL(PL_BF16_IL) PIPE_BF16_TILES_XT(PL_BF16_XT)
    }
    if (wdtype == WT_FP8) { PIPE_FP8_TILES(PL_FP8) PIPE_FP8_TILES_BX(PL_FP8_BX) PIPE_FP8_TILES_XT(PL_FP8_XT) }
    if (wdtype == WT_INT4) return launch_gemm_i4(tile, kind, partial, a, max_tiles, s);
    return hipErrorInvalidValue;
}

}  // namespace moe
