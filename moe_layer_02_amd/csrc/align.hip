// align.hip -- token/expert align and permute in one workgroup, with no host round trip.
//
// The moe_align_block_size step of vLLM PR #12185 ("[Kernel] add triton fused moe kernel
// for gptq/awq", note 1: a shared-memory kernel that is CUDA-graph safe and handles large
// expert counts).  Here: an LDS histogram per wave, a prefix sum over the block-padded
// counts, then a stable scatter.  Positions never come from atomic tickets: a lane's rank
// among the lanes of its wave that hold the same expert is the popcount of a ballot match
// (one ballot per bit of the expert id), so the order inside an expert is the ascending
// flat index t*k + j and the layout is the same on every run.
#include "common.h"
#include "kernels.h"

namespace moe {
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

__global__ __launch_bounds__(1024) void k_align(AlignArgs a) {
    __shared__ int hist[kWaves][kMaxE];   // per-wave counts, then per-wave write cursors
    __shared__ int off_s[kMaxE + 1];      // exclusive prefix of padded counts; [256] = total
    const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6;
    const int P = a.T * a.k, E = a.E, BM = a.BM;

    for (int i = tid; i < kWaves * kMaxE; i += 1024) hist[i / kMaxE][i % kMaxE] = 0;
    for (int64_t r = tid; r < a.cap; r += 1024) a.sorted[r] = P;
    __syncthreads();

    // each wave owns a contiguous segment of pairs, a multiple of 64 long
    const int seg = (P + kWaves * kWave - 1) / (kWaves * kWave) * kWave;
    const int beg = min(P, w * seg), end = min(P, beg + seg);
    for (int i = beg + lane; i < end; i += kWave) {
        const int e = a.ids[i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[w][e], 1);   // others are dropped
    }
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
    if (w == 0) {
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
    __syncthreads();
    const int total = off_s[kMaxE];
    if (tid == 0) *a.npp = total;
    if (tid < E)
        for (int ww = 0; ww < kWaves; ww++) hist[ww][tid] += off_s[tid];
    for (int64_t b = tid; b < a.cap / BM; b += 1024) {
        const int64_t r = b * BM;
        int e = -1;
        if (r < total) {   // the last expert whose first row is at or before r owns r
            int lo = 0, hi = E - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off_s[mid] <= r) lo = mid; else hi = mid - 1;
            }
            e = lo;
        }
        a.eids[b] = e;
    }
    __syncthreads();

    // stable scatter: 64 pairs at a time, rank inside the chunk from matching ballots
    volatile int *cursor = hist[w];
    for (int base = beg; base < end; base += kWave) {
        const int i = base + lane;
        int e = i < end ? a.ids[i] : -1;
        const bool valid = (unsigned)e < (unsigned)E;
        if (!valid) e = 0;
        uint64_t same = __ballot(valid);
        for (int b = 0; b < a.nbits; b++) {
            const bool bit = (e >> b) & 1;
            const uint64_t bal = __ballot(valid && bit);
            same &= bit ? bal : ~bal;
        }
        if (valid) {
            const int rank = __popcll(same & lanemask_lt());
            const int cnt = __popcll(same);
            const int pos = cursor[e] + rank;
            a.sorted[pos] = i;
            a.inv_pos[i] = pos;
            if (rank == cnt - 1) cursor[e] = pos + 1;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

}  // namespace

hipError_t launch_align(const AlignArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_align, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
