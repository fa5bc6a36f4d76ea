// grouped.hip -- block layout of a grouped GEMM over pre-permuted contiguous segments.
//
// The EP-MoE grouped GEMM (aijishu article on FBGEMM's MoE grouped GEMM vs SGLang's: the
// kernel EP-MoE runs on tokens already grouped by expert) takes rows grouped by expert in
// contiguous segments of m_sizes[e] rows.  The GEMM kernels walk blocks of BM rows, one
// expert per block; this kernel lays the segments out as such blocks without moving data:
// block b of segment e covers its rows BM*(b - first block of e) ..., sorted[] names each
// block row's source row (M for the padding past a segment's end), expert_ids[] each
// block's segment, and num_post_pad the number of block rows.  Each 1024-thread workgroup
// takes the prefix sums of all sizes (at most 1024) itself and lays out its share of the
// rows, so the sizes stay on the device (no host synchronisation) and no workgroup waits
// for another.
#include <algorithm>

#include "kernels.h"

namespace moe {
namespace {

// inclusive prefix sum over the workgroup (1024 threads, one value each)
__device__ int block_scan(int v, int *buf) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int add = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    const int r = buf[t];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(1024) void k_segments(SegmentArgs a) {
    __shared__ int scan[1024], seg_start[1024], seg_len[1024], blk_end[1024];
    const int t = threadIdx.x;
    const int m = t < a.E ? max(a.m_sizes[t], 0) : 0;
    const int end = block_scan(m, scan);                      // rows through segment t
    // segments are clamped to the M rows of X (sizes past M are a caller error; their
    // rows are not read or written)
    const int start = min(end - m, a.M), len = min(end, a.M) - start;
    const int blocks = (len + a.BM - 1) >> a.bm_shift;
    const int bend = block_scan(blocks, scan);                // blocks through segment t
    seg_start[t] = start;
    seg_len[t] = len;
    blk_end[t] = bend;
    __syncthreads();
    const int total_blocks = blk_end[1023];
    if (blockIdx.x == 0 && t == 0) *a.npp = total_blocks << a.bm_shift;
    const int rows = total_blocks << a.bm_shift;
    // every workgroup computed the same prefix sums; each lays out its share of the rows
    for (int i = blockIdx.x * 1024 + t; i < rows; i += gridDim.x * 1024) {
        const int b = i >> a.bm_shift;
        int lo = 0, hi = a.E - 1;                             // the first segment ending past block b
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (blk_end[mid] > b) hi = mid;
            else lo = mid + 1;
        }
        const int r = i - ((blk_end[lo] - ((seg_len[lo] + a.BM - 1) >> a.bm_shift)) << a.bm_shift);
        a.sorted[i] = r < seg_len[lo] ? seg_start[lo] + r : a.M;
        if ((i & (a.BM - 1)) == 0) a.eids[b] = lo;
    }
}

}  // namespace

hipError_t launch_segments(const SegmentArgs &a, int64_t capacity, hipStream_t s) {
    // about two rows per thread, up to 128 workgroups
    const int64_t g = std::min<int64_t>(128, std::max<int64_t>(1, (capacity + 2047) / 2048));
    hipLaunchKernelGGL(k_segments, dim3((unsigned)g), dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
