// quant.hip -- dynamic per-tensor E4M3 quantisation of activations for the w8a8 layer.
//
// fp8 w8a8 with per-tensor scales is how SGLang PR #2333 serves Qwen2-57B-A14B-FP8 and what
// the FBGEMM article's grouped GEMM supports.  A tensor's scale is its largest magnitude
// over 448 (the largest E4M3 value), so the largest element lands on +-448.  The largest
// |x| comes from the pass before this one: for the hidden states as one partial maximum per
// route workgroup (reduced here by every workgroup; non-negative floats order like their
// bits, and max is order-independent, so the result is exact and reproducible), for the
// intermediate h from GEMM1's epilogue atomics.  quant: code = RNE_E4M3(x * (448 / amax))
// (the product in fp32, clamped to +-448), and block 0 publishes scale = amax / 448 (1 when
// amax is 0) for the GEMM epilogue.
#include "common.h"
#include "kernels.h"
#include "quant_dev.h"

namespace moe {
namespace {

using namespace quant_dev;

// 8 elements (bf16 or fp32) per thread -> 8 codes (one 8-byte store)
__global__ __launch_bounds__(256) void k_quant(QuantArgs a) {
    float scale, inv;
    uint32_t amax_bits;
    if (a.amax_parts) {   // the largest of the partial maxima, by every workgroup
        float m = 0.0f;
        for (int i = threadIdx.x; i < a.n_parts; i += 256) m = fmaxf(m, __uint_as_float(a.amax_parts[i]));
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        __shared__ float wmax[4];
        if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
        __syncthreads();
        amax_bits = __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
        if (blockIdx.x == 0 && threadIdx.x == 0 && a.amax_out) *a.amax_out = amax_bits;
    } else {
        amax_bits = *a.amax;
    }
    scales_from_amax(amax_bits, &scale, &inv);
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

}  // namespace

hipError_t launch_quant(const QuantArgs &a, hipStream_t s) {
    int64_t blocks = (a.rows * (a.cols / 8) + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_quant, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
