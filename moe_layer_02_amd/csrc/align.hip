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
#include "align_dev.h"

namespace moe {

constexpr int64_t kOneGroupPairs = 4096;   // up to this many pairs: the one-workgroup kernel

namespace {

using namespace align_dev;

__global__ __launch_bounds__(1024) void k_align(AlignArgs a) { align_group(a); }

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
