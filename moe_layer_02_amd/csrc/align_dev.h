// align_dev.h -- device code of the token/expert align (align.hip, prologue.hip).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {
namespace align_dev {

constexpr int kWaves = 16;
constexpr int kMaxE = 256;

// Inclusive prefix sum over the wave: four DPP row shifts (1, 2, 4, 8 lanes) scan each row
// of 16 lanes in registers, then the row totals (lanes 15, 31, 47) are added to the rows
// after them -- no LDS round trips (a shuffle is an LDS permute).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane_id() >> 4;
    return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// Lanes of the wave holding the same expert as this lane (only lanes with valid set).
__device__ __forceinline__ uint64_t match_mask(int e, bool valid, int nbits) {
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; b++) {
        const bool bit = (e >> b) & 1;
        const uint64_t bal = __ballot(valid && bit);
        same &= bit ? bal : ~bal;
    }
    return same;
}

// Scatter the pairs [beg, end) in order; cursor[e] (LDS) is the next row of expert e for
// this wave and advances by each piece's group sizes.
__device__ __forceinline__ void scatter_range(const int32_t *ids, int beg, int end, int E, int nbits,
                                              volatile int *cursor, int32_t *sorted, int32_t *inv_pos) {
    const int lane = lane_id();
    int e_next = beg + lane < end ? ids[beg + lane] : -1;   // the next piece loads while this one is placed
    for (int base = beg; base < end; base += kWave) {
        const int i = base + lane;
        int e = e_next;
        if (base + kWave < end) e_next = base + kWave + lane < end ? ids[base + kWave + lane] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (!valid) {
            if (i < end) inv_pos[i] = -1;
            e = 0;
        }
        const uint64_t same = match_mask(e, valid, nbits);
        if (valid) {
            const int rank = __popcll(same & lanemask_lt());
            const int cnt = __popcll(same);
            const int pos = cursor[e] + rank;
            sorted[pos] = i;
            inv_pos[i] = pos;
            if (rank == cnt - 1) cursor[e] = pos + 1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Exclusive scan of off_s[0..E) (padded counts) by wave 0; off_s[kMaxE] = total.
__device__ __forceinline__ void scan_experts(int *off_s, int E) {
    if (threadIdx.x >= kWave) return;
    const int lane = lane_id();
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int e = lane * 4 + q;
        v[q] = e < E ? off_s[e] : 0;
        sum += v[q];
    }
    const int incl = wave_inclusive_scan(sum);
    int run = incl - sum;
#pragma unroll
    for (int q = 0; q < 4; q++) {
        const int e = lane * 4 + q;
        if (e < E) off_s[e] = run;
        run += v[q];
    }
    if (lane == kWave - 1) off_s[kMaxE] = incl;
}

// Count the pairs [beg, end) per expert into hist (LDS) with one LDS atomic add per pair:
// the LDS serialises only the lanes that hit the same expert, where matching the lanes'
// experts first by ballots costs a few VALU operations per id bit and piece (four cycles
// each for a wave of 64).  kCountPieces pieces per step
// with their loads issued together, and the next step's loads issued before this step's
// pieces are counted (the order of the pieces does not matter to a count).  beg must be a
// multiple of 64; the wave strides by `step` pairs.
constexpr int kCountPieces = 8;

__device__ __forceinline__ void count_strided(const int32_t *ids, int beg, int end, int step, int E, int *hist) {
    const int lane = lane_id();
    int nxt[kCountPieces];
    auto load = [&](int base) {
#pragma unroll
        for (int q = 0; q < kCountPieces; q++) {
            const int i = base + q * kWave + lane;
            nxt[q] = i < end ? ids[i] : -1;
        }
    };
    if (beg < end) load(beg);
    for (int base = beg; base < end; base += step) {
        int e[kCountPieces];
#pragma unroll
        for (int q = 0; q < kCountPieces; q++) e[q] = nxt[q];
        if (base + step < end) load(base + step);
#pragma unroll
        for (int q = 0; q < kCountPieces; q++)
            if ((unsigned)e[q] < (unsigned)E) atomicAdd(&hist[e[q]], 1);
    }
}

// expert_ids for every block: the last expert whose first padded row is at or before the
// block's first padded row owns it (experts with no rows share their successor's offset).
// Without padding (blk_start non-null) also the block's first row among the unpadded rows,
// coff_s[e] + (its padded first row - off_s[e]), and P (the number of pairs) for the blocks
// past the last one, through blk_start[cap / BM].  Blocks first, first + stride, ... are
// written by the calling thread.
__device__ __forceinline__ void write_block_experts(const int *off_s, const int *coff_s, int E, int BM, int64_t cap,
                                                    int total, int P, int32_t *eids, int32_t *blk_start,
                                                    int64_t first, int64_t stride) {
    const int64_t nb = cap / BM;
    for (int64_t b = first; b <= nb; b += stride) {
        const int64_t r = b * BM;
        int e = -1;
        if (r < total) {
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off_s[mid] <= r) lo = mid; else hi = mid - 1;
            }
            e = lo;
        }
        if (b < nb) eids[b] = e;
        if (blk_start) blk_start[b] = e >= 0 ? coff_s[e] + (int)(r - off_s[e]) : P;
    }
}

// The whole align of at most kOneGroupPairs pairs by one workgroup of 1024 threads (every
// thread must call; the pairs must already be visible to the workgroup).
__device__ __forceinline__ void align_group(const AlignArgs &a) {
    __shared__ int hist[kWaves][kMaxE];   // per-wave counts, then per-wave write cursors
    __shared__ int off_s[kMaxE + 1];      // padded offsets
    __shared__ int coff_s[kMaxE + 1];     // unpadded offsets (the layout without padding)
    const int tid = threadIdx.x, w = tid >> 6;
    const int P = a.T * a.k, E = a.E, BM = a.BM;

    for (int i = tid; i < kWaves * kMaxE; i += 1024) hist[i / kMaxE][i % kMaxE] = 0;
    if (!a.blk_start)   // the padded layout's filler entries
        for (int64_t r = tid; r < a.cap; r += 1024) a.sorted[r] = P;
    __syncthreads();
    // each wave owns a contiguous segment of pairs, a multiple of 64 long
    const int seg = (P + kWaves * kWave - 1) / (kWaves * kWave) * kWave;
    const int beg = min(P, w * seg), end = min(P, beg + seg);
    count_strided(a.ids, beg, end, kCountPieces * kWave, E, hist[w]);
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int ww = 0; ww < kWaves; ww++) {
            const int c = hist[ww][tid];
            hist[ww][tid] = run;   // pairs of this expert in earlier waves
            run += c;
        }
        a.counts[tid] = run;
        off_s[tid] = (run + BM - 1) / BM * BM;
        coff_s[tid] = run;
    }
    __syncthreads();
    scan_experts(off_s, E);
    scan_experts(coff_s, E);
    __syncthreads();
    const int total = off_s[kMaxE];
    if (tid == 0) *a.npp = total;
    const int *base = a.blk_start ? coff_s : off_s;   // where each expert's rows start
    if (tid < E)
        for (int ww = 0; ww < kWaves; ww++) hist[ww][tid] += base[tid];
    write_block_experts(off_s, coff_s, E, BM, a.cap, total, P, a.eids, a.blk_start, tid, 1024);
    __syncthreads();
    scatter_range(a.ids, beg, end, E, a.nbits, hist[w], a.sorted, a.inv_pos);
}

// The align of one token's k pairs (a decode step): a top-k of one token names k distinct
// experts, so each selected expert holds one pair and the layout is the selected experts in
// ascending order -- what align_group produces for it, written directly.  my_id: on wave 0,
// lane j < k holds the expert of slot j (the route's result); every thread of the workgroup
// calls.  Returns false, having written nothing, when a slot holds no expert (the caller
// then runs align_group on the pairs in memory).
__device__ __forceinline__ bool align_one_token(const AlignArgs &a, int my_id) {
    __shared__ int sel_s[kWave];                  // expert of rank r (ascending)
    __shared__ int pair_s[kWave];                 // its pair (= slot)
    __shared__ uint32_t bits_s[kMaxE / 32];       // the selected experts
    __shared__ int ok_s;
    const int tid = threadIdx.x, k = a.k, E = a.E, BM = a.BM, P = k;
    if (tid < kMaxE / 32) bits_s[tid] = 0u;
    __syncthreads();
    if (tid < kWave) {
        const bool mine = tid < k;
        const bool ok = __ballot(mine && (unsigned)my_id < (unsigned)E) == __ballot(mine);
        if (tid == 0) ok_s = ok;
        if (ok && mine) {
            int rank = 0;
            for (int j = 0; j < k; j++) rank += __builtin_amdgcn_readlane(my_id, j) < my_id;
            sel_s[rank] = my_id;
            pair_s[rank] = tid;
            atomicOr(&bits_s[my_id >> 5], 1u << (my_id & 31));
        }
    }
    __syncthreads();
    if (!ok_s) return false;
    if (tid < E) a.counts[tid] = (int)((bits_s[tid >> 5] >> (tid & 31)) & 1u);
    if (tid == 0) *a.npp = k * BM;   // one block of padded rows per selected expert
    // block b < k belongs to the expert of rank b and starts at unpadded row b
    const int64_t nb = a.cap / BM;
    for (int64_t b = tid; b <= nb; b += 1024) {
        const int e = b < k ? sel_s[b] : -1;
        if (b < nb) a.eids[b] = e;
        if (a.blk_start) a.blk_start[b] = e >= 0 ? (int)b : P;
    }
    if (a.blk_start) {
        if (tid < k) {
            a.sorted[tid] = pair_s[tid];
            a.inv_pos[pair_s[tid]] = tid;
        }
    } else {   // the padded layout: filler entries except each block's first row
        for (int64_t r = tid; r < a.cap; r += 1024) {
            const int64_t b = r / BM;
            a.sorted[r] = (r == b * BM && b < k) ? pair_s[b] : P;
        }
        if (tid < k) a.inv_pos[pair_s[tid]] = tid * BM;
    }
    return true;
}

}  // namespace align_dev
}  // namespace moe
