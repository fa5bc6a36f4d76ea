// align.hip -- token/expert align and permute with no host round trip.
//
// The moe_align_block_size step of vLLM PR #12185 ("[Kernel] add triton fused moe kernel
// for gptq/awq", note 1: a shared-memory kernel that is CUDA-graph safe and handles large
// expert counts).  Here: per-wave LDS histograms, a prefix sum over the block-padded
// counts, then a stable scatter.  Positions never come from atomic tickets: a lane's rank
// among the lanes of its wave that hold the same expert is the popcount of a ballot match
// (one ballot per bit of the expert id), so the order inside an expert is the ascending
// flat index t*k + j and the layout is the same on every run.
//
// Up to kOneGroupPairs pairs one 1024-thread workgroup does everything (one launch, the
// small-T case).  Beyond that the pairs are cut into chunks of kChunk: k_align_count
// histograms every chunk in parallel, k_align_scan (one workgroup) turns the histograms
// into per-chunk write offsets, and k_align_scatter ranks and writes every chunk in
// parallel -- the same stable order, so both paths produce identical outputs.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int64_t kOneGroupPairs = 4096;   // up to this many pairs: the one-workgroup kernel

namespace {

constexpr int kWaves = 16;
constexpr int kMaxE = 256;

__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    return v;
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

// Count the pairs [beg, end) per expert into hist (LDS): per 64-pair piece, the lowest lane
// of each group of equal experts adds the group's size (no atomic contention per expert).
__device__ __forceinline__ void count_range(const int32_t *ids, int beg, int end, int E, int nbits, int *hist) {
    const int lane = lane_id();
    for (int base = beg; base < end; base += kWave) {
        const int i = base + lane;
        int e = i < end ? ids[i] : -1;
        const bool valid = (unsigned)e < (unsigned)E;   // other ids are dropped
        if (!valid) e = 0;
        const uint64_t same = match_mask(e, valid, nbits);
        if (valid && (same & lanemask_lt()) == 0) atomicAdd(&hist[e], __popcll(same));
    }
}

// Scatter the pairs [beg, end) in order; cursor[e] (LDS) is the next row of expert e for
// this wave and advances by each piece's group sizes.
__device__ __forceinline__ void scatter_range(const int32_t *ids, int beg, int end, int E, int nbits,
                                              volatile int *cursor, int32_t *sorted, int32_t *inv_pos) {
    const int lane = lane_id();
    for (int base = beg; base < end; base += kWave) {
        const int i = base + lane;
        int e = i < end ? ids[i] : -1;
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

// expert_ids for every block: the last expert whose first row is at or before the block's
// first row owns it (experts with no rows share their successor's offset).
__device__ __forceinline__ void write_block_experts(const int *off_s, int E, int BM, int64_t cap, int total,
                                                    int32_t *eids) {
    for (int64_t b = threadIdx.x; b < cap / BM; b += blockDim.x) {
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
        eids[b] = e;
    }
}

__global__ __launch_bounds__(1024) void k_align(AlignArgs a) {
    __shared__ int hist[kWaves][kMaxE];   // per-wave counts, then per-wave write cursors
    __shared__ int off_s[kMaxE + 1];
    const int tid = threadIdx.x, w = tid >> 6;
    const int P = a.T * a.k, E = a.E, BM = a.BM;

    for (int i = tid; i < kWaves * kMaxE; i += 1024) hist[i / kMaxE][i % kMaxE] = 0;
    for (int64_t r = tid; r < a.cap; r += 1024) a.sorted[r] = P;
    __syncthreads();
    // each wave owns a contiguous segment of pairs, a multiple of 64 long
    const int seg = (P + kWaves * kWave - 1) / (kWaves * kWave) * kWave;
    const int beg = min(P, w * seg), end = min(P, beg + seg);
    count_range(a.ids, beg, end, E, a.nbits, hist[w]);
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
    }
    __syncthreads();
    scan_experts(off_s, E);
    __syncthreads();
    const int total = off_s[kMaxE];
    if (tid == 0) *a.npp = total;
    if (tid < E)
        for (int ww = 0; ww < kWaves; ww++) hist[ww][tid] += off_s[tid];
    write_block_experts(off_s, E, BM, a.cap, total, a.eids);
    __syncthreads();
    scatter_range(a.ids, beg, end, E, a.nbits, hist[w], a.sorted, a.inv_pos);
}

// ---- the multi-workgroup path -------------------------------------------------------------

constexpr int kChunk = 2048;          // pairs per workgroup (8 waves x 256)
constexpr int kChunkWaves = 8;

__global__ __launch_bounds__(512) void k_align_count(AlignArgs a, int32_t *chunk_counts) {
    __shared__ int hist[kMaxE];
    const int P = a.T * a.k;
    for (int i = threadIdx.x; i < a.E; i += 512) hist[i] = 0;
    __syncthreads();
    const int c0 = blockIdx.x * kChunk, w = threadIdx.x >> 6;
    const int seg = kChunk / kChunkWaves;
    const int beg = min(P, c0 + w * seg), end = min(P, beg + seg);
    count_range(a.ids, beg, end, a.E, a.nbits, hist);
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += 512) chunk_counts[(int64_t)blockIdx.x * a.E + e] = hist[e];
}

// One workgroup: totals, padded offsets, expert_ids, fillers, and chunk_counts rewritten in
// place as each chunk's first row per expert.
__global__ __launch_bounds__(1024) void k_align_scan(AlignArgs a, int32_t *chunk_counts, int nchunks) {
    __shared__ int off_s[kMaxE + 1];
    const int tid = threadIdx.x, P = a.T * a.k, E = a.E, BM = a.BM;
    for (int64_t r = tid; r < a.cap; r += 1024) a.sorted[r] = P;
    if (tid < E) {
        int run = 0;
        for (int c = 0; c < nchunks; c++) run += chunk_counts[(int64_t)c * E + tid];
        a.counts[tid] = run;
        off_s[tid] = (run + BM - 1) / BM * BM;
    }
    __syncthreads();
    scan_experts(off_s, E);
    __syncthreads();
    const int total = off_s[kMaxE];
    if (tid == 0) *a.npp = total;
    if (tid < E) {
        int run = off_s[tid];
        for (int c = 0; c < nchunks; c++) {
            const int cnt = chunk_counts[(int64_t)c * E + tid];
            chunk_counts[(int64_t)c * E + tid] = run;
            run += cnt;
        }
    }
    write_block_experts(off_s, E, BM, a.cap, total, a.eids);
}

__global__ __launch_bounds__(512) void k_align_scatter(AlignArgs a, const int32_t *chunk_base) {
    __shared__ int hist[kChunkWaves][kMaxE];
    const int P = a.T * a.k, E = a.E;
    const int c0 = blockIdx.x * kChunk, w = threadIdx.x >> 6;
    const int seg = kChunk / kChunkWaves;
    const int beg = min(P, c0 + w * seg), end = min(P, beg + seg);
    for (int i = threadIdx.x; i < kChunkWaves * kMaxE; i += 512) hist[i / kMaxE][i % kMaxE] = 0;
    __syncthreads();
    count_range(a.ids, beg, end, E, a.nbits, hist[w]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 512) {
        int run = chunk_base[(int64_t)blockIdx.x * E + e];
        for (int ww = 0; ww < kChunkWaves; ww++) {
            const int c = hist[ww][e];
            hist[ww][e] = run;
            run += c;
        }
    }
    __syncthreads();
    scatter_range(a.ids, beg, end, E, a.nbits, hist[w], a.sorted, a.inv_pos);
}

}  // namespace

int64_t align_scratch_bytes(int64_t pairs, int E) {
    if (pairs <= kOneGroupPairs) return 0;
    return (pairs + kChunk - 1) / kChunk * E * 4;
}

hipError_t launch_align(const AlignArgs &a, int32_t *scratch, hipStream_t s) {
    const int64_t P = (int64_t)a.T * a.k;
    if (P <= kOneGroupPairs || !scratch) {
        hipLaunchKernelGGL(k_align, dim3(1), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
    const int nchunks = (int)((P + kChunk - 1) / kChunk);
    hipLaunchKernelGGL(k_align_count, dim3(nchunks), dim3(512), 0, s, a, scratch);
    hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(1024), 0, s, a, scratch, nchunks);
    hipLaunchKernelGGL(k_align_scatter, dim3(nchunks), dim3(512), 0, s, a, (const int32_t *)scratch);
    return hipGetLastError();
}

}  // namespace moe
