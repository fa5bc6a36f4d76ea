// reduce.hip -- unpermute and reduce: each token's k weighted expert rows summed back to
// token order, in a fixed order, with no floating-point atomics.
//
// TensorRT-LLM's unpermute_and_reduce (named in the last review comment of SGLang PR #3191
// "Add deepseek_v3 fused gate") returns the permuted rows to their tokens.  Here each thread
// owns 8 consecutive columns of one token and adds, for j = 0..k-1 and then split s =
// 0..S-1, the row inv_pos[t*k + j] -- the same order on every run, so the result is bitwise
// reproducible; SGLang PR #2333 ("[kernel] introduce fused_moe_triton_splitk", Background)
// shows what an unordered atomic_add of the same partial sums did to the output.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void k_reduce(ReduceArgs a) {
    const int c8 = a.H / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t t = gid / c8;
    const int col = (int)(gid % c8) * 8;
    if (t >= a.T) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < a.k; j++) {
        const int64_t row = a.inv_pos[t * a.k + j];
        if (a.split == 0) {
            const uint4 v = *(const uint4 *)((const uint16_t *)a.Y + row * a.H + col);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[2 * i] += __uint_as_float(w[i] << 16);
                acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
            }
        } else {
            for (int s = 0; s < a.split; s++) {
                const float *p = (const float *)a.Y + s * a.partial_stride + row * a.H + col;
                const float4 lo = *(const float4 *)p, hi = *(const float4 *)(p + 4);
                acc[0] += lo.x; acc[1] += lo.y; acc[2] += lo.z; acc[3] += lo.w;
                acc[4] += hi.x; acc[5] += hi.y; acc[6] += hi.z; acc[7] += hi.w;
            }
        }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *(uint4 *)(a.out + t * a.H + col) = o;
}

}  // namespace

hipError_t launch_reduce(const ReduceArgs &a, hipStream_t s) {
    const int64_t threads = (int64_t)a.T * (a.H / 8);
    hipLaunchKernelGGL(k_reduce, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
