// quant.hip -- dynamic per-tensor E4M3 quantisation of activations for the w8a8 layer.
//
// fp8 w8a8 with per-tensor scales is how SGLang PR #2333 serves Qwen2-57B-A14B-FP8 and what
// the FBGEMM article's grouped GEMM supports.  A tensor's scale is its largest magnitude
// over 448 (the largest E4M3 value), so the largest element lands on +-448.  Two kernels:
//   absmax: largest |x| over the tensor, combined across workgroups with an integer
//           atomicMax on the fp32 bit pattern (non-negative floats order like their bits;
//           max is order-independent, so the result is exact and reproducible);
//   quant:  code = RNE_E4M3(x * (448 / amax)) (the product in fp32, clamped to +-448), and
//           block 0 publishes scale = amax / 448 (1 when amax is 0) for the GEMM epilogue.
#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

namespace moe {
namespace {

using namespace quant_dev;

// Same-address atomics serialise (about 16 ns each here), so the pass runs as at most one
// 1024-thread workgroup per CU, each with one atomic, and keeps four 16-byte loads in
// flight per thread (the maximum does not depend on the order).
constexpr int kAbsmaxThreads = 1024;

__global__ __launch_bounds__(kAbsmaxThreads) void k_absmax(AbsmaxArgs a) {
    float m = 0.0f;
    const int64_t n8 = a.n / 8, stride = (int64_t)gridDim.x * kAbsmaxThreads;
    constexpr int U = 4;
    for (int64_t i0 = (int64_t)blockIdx.x * kAbsmaxThreads + threadIdx.x; i0 < n8; i0 += U * stride) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int64_t i = i0 + u * stride;
            v[u] = i < n8 ? ((const uint4 *)a.x)[i] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                m = fmaxf(m, fabsf(__uint_as_float(w[q] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
            }
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
    __shared__ float wmax[kAbsmaxThreads / kWave];
    if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = 0.0f;
        for (int w = 0; w < kAbsmaxThreads / kWave; w++) b = fmaxf(b, wmax[w]);
        amax_raise(a.amax, amax_peek(a.amax), b);
    }
}

// 8 elements (bf16 or fp32) per thread -> 8 codes (one 8-byte store)
__global__ __launch_bounds__(256) void k_quant(QuantArgs a) {
    float scale, inv;
    scales_from_amax(*a.amax, &scale, &inv);
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.scale_out = scale;
    const int64_t c8 = a.cols / 8;
    int64_t rows = a.rows;
    if (a.npp) rows = min(rows, (int64_t)*a.npp);
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < rows * c8; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / c8;
        uint2 out = make_uint2(0, 0);
        if (!a.row_valid || a.row_valid[r] < a.pairs) {
            if (a.x_f32) {
                const float4 lo = ((const float4 *)a.x)[2 * i], hi = ((const float4 *)a.x)[2 * i + 1];
                out.x = e4m3x4(lo.x, lo.y, lo.z, lo.w, inv);
                out.y = e4m3x4(hi.x, hi.y, hi.z, hi.w, inv);
            } else {
                const uint4 v = ((const uint4 *)a.x)[i];
                out.x = e4m3x4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u), inv);
                out.y = e4m3x4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xFFFF0000u),
                               __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xFFFF0000u), inv);
            }
        }
        ((uint2 *)a.q)[i] = out;
    }
}

// int4 GEMM1's A: each 8 bf16 reordered into the packed-nibble order, one 16-byte load and
// store
__global__ __launch_bounds__(256) void k_bf16_perm(const uint16_t *x, uint16_t *y, int64_t n8) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256)
        ((uint4 *)y)[i] = bf16x8_perm(((const uint4 *)x)[i]);
}

}  // namespace

hipError_t launch_bf16_perm(const uint16_t *x, uint16_t *y, int64_t n8, hipStream_t s) {
    int64_t blocks = (n8 + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_bf16_perm, dim3((unsigned)blocks), dim3(256), 0, s, x, y, n8);
    return hipGetLastError();
}

hipError_t launch_absmax(const AbsmaxArgs &a, hipStream_t s) {
    int64_t blocks = (a.n / 8 + kAbsmaxThreads - 1) / kAbsmaxThreads;
    const int64_t cap = device_cu_count();
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_absmax, dim3((unsigned)blocks), dim3(kAbsmaxThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    int64_t blocks = (a.rows * (a.cols / 8) + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_quant, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
