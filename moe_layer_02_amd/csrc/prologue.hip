// prologue.hip -- route, align and the activation pass of a small batch in one launch.
//
// With a few tokens each of these steps is a few microseconds of launch and memory
// latency, comparable to the whole weight-streaming time of a small layer.  One launch of
// 1024-thread workgroups does them all, with the same results as the separate kernels:
//   workgroup 0: wave w routes tokens w, w + 16, ... (route_dev.h), a barrier makes the
//                pairs visible, then the one-workgroup align (align_dev.h) lays them out
//                (one token: its k distinct experts are laid out directly);
//   workgroups 1..: the activation pass, independent of the routing --
//                fp8 (one workgroup): the batch into registers, its largest |x| (reduced
//                inside the workgroup, no atomics), then every code with that scale
//                (quant_dev.h), and the scale; int4: the hidden states to fp16 in the packed-nibble order.
#include <algorithm>

#include "align_dev.h"
#include "kernels.h"
#include "quant_dev.h"
#include "route_dev.h"

namespace moe {
namespace {

template <int EPL, int V>
__global__ __launch_bounds__(1024) void k_prologue(PrologueArgs p) {
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0 && p.h_amax) *p.h_amax = 0u;   // GEMM1's |h| maximum starts at 0
        if (p.route.T == 1) {   // one token: its distinct experts lay out directly
            const int id = threadIdx.x < kWave ? route_dev::route_token<EPL, V>(p.route, 0) : 0;
            if (align_dev::align_one_token(p.align, id)) return;
        } else {
            for (int t = threadIdx.x >> 6; t < p.route.T; t += 16) route_dev::route_token<EPL, V>(p.route, t);
        }
        __syncthreads();
        align_dev::align_group(p.align);
        return;
    }
    const int64_t n8 = p.n / 8;
    const int tid = threadIdx.x;
    if (p.act == PROLOGUE_ACT_BF16_PERM) {   // workgroups 1 .. G-1 share the permutation
        const int64_t stride = (int64_t)(gridDim.x - 1) * 1024;
        for (int64_t i = (int64_t)(blockIdx.x - 1) * 1024 + tid; i < n8; i += stride)
            ((uint4 *)p.xperm)[i] = bf16x8_perm(((const uint4 *)p.x)[i]);
        return;
    }
    // fp8: the batch is read once into registers (every load in flight at once), its
    // largest |x| reduced in the workgroup, and the codes written from the registers.
    // Groups beyond kPrologueActRegs per thread (none for the sizes the host sends here)
    // are read again from memory.
    // (past the end a thread reads the last group again: no effect on the maximum)
    if (n8 <= 0) return;
    const uint4 *xv = (const uint4 *)p.x;
    const int last = (int)min<int64_t>(n8, (int64_t)kPrologueActRegs * 1024) - 1;
    uint4 v[kPrologueActRegs];
#pragma unroll
    for (int j = 0; j < kPrologueActRegs; j++) v[j] = xv[min(tid + j * 1024, last)];
    float m = 0.0f;
    auto fold = [&](const uint4 &g) {
        const uint32_t wv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
            m = fmaxf(m, fabsf(__uint_as_float(wv[q] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(wv[q] & 0xFFFF0000u)));
        }
    };
#pragma unroll
    for (int j = 0; j < kPrologueActRegs; j++) fold(v[j]);
    for (int64_t i = tid + (int64_t)kPrologueActRegs * 1024; i < n8; i += 1024) fold(((const uint4 *)p.x)[i]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    __shared__ float wmax[16];
    if (lane_id() == 0) wmax[tid >> 6] = m;
    __syncthreads();
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) amax = fmaxf(amax, wmax[i]);
    float scale, inv;
    quant_dev::scales_from_amax(__float_as_uint(amax), &scale, &inv);
    if (tid == 0) {
        *p.x_amax = __float_as_uint(amax);
        *p.x_scale = scale;
    }
    // the codes are derived from v again, not from values kept since the maximum (which
    // would hold eight floats per group through the reduction)
#pragma unroll
    for (int j = 0; j < kPrologueActRegs; j++) asm volatile("" : "+v"(v[j].x), "+v"(v[j].y), "+v"(v[j].z), "+v"(v[j].w));
    auto codes = [&](const uint4 &g) {
        uint2 out;
        out.x = quant_dev::e4m3x4(__uint_as_float(g.x << 16), __uint_as_float(g.x & 0xFFFF0000u),
                                  __uint_as_float(g.y << 16), __uint_as_float(g.y & 0xFFFF0000u), inv);
        out.y = quant_dev::e4m3x4(__uint_as_float(g.z << 16), __uint_as_float(g.z & 0xFFFF0000u),
                                  __uint_as_float(g.w << 16), __uint_as_float(g.w & 0xFFFF0000u), inv);
        return out;
    };
#pragma unroll
    for (int j = 0; j < kPrologueActRegs; j++)
        if (tid + j * 1024 <= last) ((uint2 *)p.xq)[tid + j * 1024] = codes(v[j]);
    for (int64_t i = tid + (int64_t)kPrologueActRegs * 1024; i < n8; i += 1024)
        ((uint2 *)p.xq)[i] = codes(((const uint4 *)p.x)[i]);
}

template <int EPL>
void launch_epl(const PrologueArgs &p, dim3 grid, dim3 block, hipStream_t s) {
    switch (route_dev::route_variant(p.route.kind, p.route.E, p.route.n_group)) {
    case route_dev::V_SOFTMAX: hipLaunchKernelGGL((k_prologue<EPL, route_dev::V_SOFTMAX>), grid, block, 0, s, p); break;
    case route_dev::V_SIGMOID: hipLaunchKernelGGL((k_prologue<EPL, route_dev::V_SIGMOID>), grid, block, 0, s, p); break;
    case route_dev::V_GROUPED_POW2: hipLaunchKernelGGL((k_prologue<EPL, route_dev::V_GROUPED_POW2>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((k_prologue<EPL, route_dev::V_GROUPED_ANY>), grid, block, 0, s, p); break;
    }
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs &p, hipStream_t s) {
    // fp8: one workgroup for the pass; fp16 conversion: one per 4096 16-byte groups, up to 32
    int g = 1;
    if (p.act == PROLOGUE_ACT_FP8) g = 2;
    if (p.act == PROLOGUE_ACT_BF16_PERM) g = 1 + (int)std::min<int64_t>(32, std::max<int64_t>(1, (p.n / 8 + 4095) / 4096));
    const dim3 grid(g), block(1024);
    if (p.route.E <= 64)
        launch_epl<1>(p, grid, block, s);
    else if (p.route.E <= 128)
        launch_epl<2>(p, grid, block, s);
    else
        launch_epl<4>(p, grid, block, s);
    return hipGetLastError();
}

}  // namespace moe
