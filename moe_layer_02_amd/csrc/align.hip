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
// small-T case).  Up to kFusedMaxPairs, k_align_fused is still one launch: every workgroup
// scatters one chunk of kFusedChunk pairs, and to know where its rows go it counts all the
// batch's pairs itself (at most 256 KiB of ids, read from L2, with the next 512 ids per wave
// in flight while the current ones are counted), so no workgroup waits for another.  Beyond that the pairs are cut into chunks of kChunk: k_align_count histograms
// every chunk in parallel, k_align_scan (one workgroup) turns the histograms into per-chunk
// write offsets, and k_align_scatter ranks and writes every chunk in parallel.  All three
// paths give the same stable order, so their outputs are identical.
#include "align_dev.h"

namespace moe {

constexpr int64_t kOneGroupPairs = 4096;   // up to this many pairs: the one-workgroup kernel
constexpr int64_t kFusedMaxPairs = 65536;  // up to this many: one launch of k_align_fused

namespace {

using namespace align_dev;

__global__ __launch_bounds__(1024) void k_align(AlignArgs a) { align_group(a); }

// ---- one launch, many workgroups --------------------------------------------------------

constexpr int kFusedChunk = 2048;   // pairs scattered per workgroup: 16 waves x 128
constexpr int kFusedSeg = kFusedChunk / kWaves;
static_assert(kFusedChunk % (kCountPieces * kWave) == 0, "a count step never straddles a chunk edge");

__global__ __launch_bounds__(1024) void k_align_fused(AlignArgs a) {
    __shared__ int hist[kWaves][kMaxE];   // this chunk's per-wave counts, then write cursors
    __shared__ int before[kMaxE];         // pairs per expert in earlier chunks
    __shared__ int cnt_s[kMaxE];          // pairs per expert in later chunks, then in all
    __shared__ int off_s[kMaxE + 1];      // padded offsets
    __shared__ int coff_s[kMaxE + 1];     // unpadded offsets
    const int tid = threadIdx.x, w = tid >> 6, G = gridDim.x;
    const int P = a.T * a.k, E = a.E, BM = a.BM;
    const int c0 = blockIdx.x * kFusedChunk, c1 = c0 + kFusedChunk;

    for (int i = tid; i < kWaves * kMaxE; i += 1024) hist[i / kMaxE][i % kMaxE] = 0;
    for (int i = tid; i < kMaxE; i += 1024) before[i] = cnt_s[i] = 0;
    __syncthreads();
    constexpr int span = kCountPieces * kWave, step = kWaves * span;
    count_strided(a.ids, w * span, c0, step, E, before);
    count_strided(a.ids, c1 + w * span, P, step, E, cnt_s);
    const int beg = min(P, c0 + w * kFusedSeg), end = min(P, beg + kFusedSeg);
    count_strided(a.ids, beg, end, kCountPieces * kWave, E, hist[w]);
    __syncthreads();
    if (tid < E) {
        int run = before[tid];
        for (int ww = 0; ww < kWaves; ww++) {
            const int c = hist[ww][tid];
            hist[ww][tid] = run;   // pairs of this expert before this wave's segment
            run += c;
        }
        const int cnt = run + cnt_s[tid];
        cnt_s[tid] = cnt;
        if (blockIdx.x == 0) a.counts[tid] = cnt;
        off_s[tid] = (cnt + BM - 1) / BM * BM;
        coff_s[tid] = cnt;
    }
    __syncthreads();
    scan_experts(off_s, E);
    scan_experts(coff_s, E);
    __syncthreads();
    const int total = off_s[kMaxE];
    if (blockIdx.x == 0 && tid == 0) *a.npp = total;
    const int *base = a.blk_start ? coff_s : off_s;   // where each expert's rows start
    if (tid < E)
        for (int ww = 0; ww < kWaves; ww++) hist[ww][tid] += base[tid];
    if (!a.blk_start) {
        // rows no pair lands in: each expert's padding (experts dealt round the workgroups)
        // and every row past the last block
        for (int e = blockIdx.x; e < E; e += G) {
            const int r0 = off_s[e] + cnt_s[e], r1 = off_s[e] + (cnt_s[e] + BM - 1) / BM * BM;
            for (int r = r0 + tid; r < r1; r += 1024) a.sorted[r] = P;
        }
        for (int64_t r = total + (int64_t)blockIdx.x * 1024 + tid; r < a.cap; r += (int64_t)G * 1024) a.sorted[r] = P;
    }
    write_block_experts(off_s, coff_s, E, BM, a.cap, total, P, a.eids, a.blk_start, (int64_t)blockIdx.x * 1024 + tid,
                        (int64_t)G * 1024);
    __syncthreads();
    scatter_range(a.ids, beg, end, E, a.nbits, hist[w], a.sorted, a.inv_pos);
}

// ---- the multi-launch path -------------------------------------------------------------

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
    count_strided(a.ids, beg, end, kCountPieces * kWave, a.E, hist);
    __syncthreads();
    for (int e = threadIdx.x; e < a.E; e += 512) chunk_counts[(int64_t)blockIdx.x * a.E + e] = hist[e];
}

// One workgroup: totals, padded offsets, expert_ids, fillers, and chunk_counts rewritten in
// place as each chunk's first row per expert.
__global__ __launch_bounds__(1024) void k_align_scan(AlignArgs a, int32_t *chunk_counts, int nchunks) {
    __shared__ int off_s[kMaxE + 1];      // padded offsets
    __shared__ int coff_s[kMaxE + 1];     // unpadded offsets
    const int tid = threadIdx.x, P = a.T * a.k, E = a.E, BM = a.BM;
    if (!a.blk_start)   // the padded layout's filler entries
        for (int64_t r = tid; r < a.cap; r += 1024) a.sorted[r] = P;
    if (tid < E) {
        int run = 0;
        for (int c = 0; c < nchunks; c++) run += chunk_counts[(int64_t)c * E + tid];
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
    if (tid < E) {
        int run = a.blk_start ? coff_s[tid] : off_s[tid];
        for (int c = 0; c < nchunks; c++) {
            const int cnt = chunk_counts[(int64_t)c * E + tid];
            chunk_counts[(int64_t)c * E + tid] = run;
            run += cnt;
        }
    }
    write_block_experts(off_s, coff_s, E, BM, a.cap, total, P, a.eids, a.blk_start, tid, 1024);
}

__global__ __launch_bounds__(512) void k_align_scatter(AlignArgs a, const int32_t *chunk_base) {
    __shared__ int hist[kChunkWaves][kMaxE];
    const int P = a.T * a.k, E = a.E;
    const int c0 = blockIdx.x * kChunk, w = threadIdx.x >> 6;
    const int seg = kChunk / kChunkWaves;
    const int beg = min(P, c0 + w * seg), end = min(P, beg + seg);
    for (int i = threadIdx.x; i < kChunkWaves * kMaxE; i += 512) hist[i / kMaxE][i % kMaxE] = 0;
    __syncthreads();
    count_strided(a.ids, beg, end, kCountPieces * kWave, E, hist[w]);
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
    if (pairs <= kFusedMaxPairs) return 0;
    return (pairs + kChunk - 1) / kChunk * E * 4;
}

hipError_t launch_align(const AlignArgs &a, int32_t *scratch, hipStream_t s) {
    const int64_t P = (int64_t)a.T * a.k;
    if (P > kOneGroupPairs && P <= kFusedMaxPairs) {
        hipLaunchKernelGGL(k_align_fused, dim3((unsigned)((P + kFusedChunk - 1) / kFusedChunk)), dim3(1024), 0, s, a);
        return hipGetLastError();
    }
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
