// grouped.hip -- block layout of a grouped GEMM over pre-permuted contiguous segments.
//
// The EP-MoE grouped GEMM (aijishu article on FBGEMM's MoE grouped GEMM vs SGLang's: the
// kernel EP-MoE runs on tokens already grouped by expert) takes rows grouped by expert in
// contiguous segments of m_sizes[e] rows.  The GEMM kernels walk blocks of BM rows, one
// expert per block; this kernel lays the segments out as such blocks without moving data:
// block b of segment e covers its rows BM*(b - first block of e) ..., sorted[] names each
// block row's source row (M for the padding past a segment's end), expert_ids[] each
// block's segment, and num_post_pad the number of block rows.  One 1024-thread workgroup,
// so the sizes stay on the device (no host synchronisation).
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
    __shared__ int scan[1024], seg_start[1024], seg_len[1024], blk_start[1024];
    __shared__ int total_blocks;
    const int t = threadIdx.x;
    const int m = t < a.E ? max(a.m_sizes[t], 0) : 0;
    const int end = block_scan(m, scan);                      // rows through segment t
    // segments are clamped to the M rows of X (sizes past M are a caller error; their
    // rows are not read or written)
    const int start = min(end - m, a.M), len = min(end, a.M) - start;
    const int blocks = (len + a.BM - 1) / a.BM;
    const int bend = block_scan(blocks, scan);
    seg_start[t] = start;
    seg_len[t] = len;
    blk_start[t] = bend - blocks;
    if (t == 1023) total_blocks = bend;
    __syncthreads();
    for (int b = 0; b < blocks; b++) a.eids[blk_start[t] + b] = t;
    if (t == 0) *a.npp = total_blocks * a.BM;
    __syncthreads();                                          // expert_ids visible to the workgroup
    const int rows = total_blocks * a.BM;
    for (int i = t; i < rows; i += 1024) {
        const int e = a.eids[i / a.BM];
        const int r = i - blk_start[e] * a.BM;
        a.sorted[i] = r < seg_len[e] ? seg_start[e] + r : a.M;
    }
}

}  // namespace

hipError_t launch_segments(const SegmentArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_segments, dim3(1), dim3(1024), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
