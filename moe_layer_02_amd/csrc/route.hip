// route.hip -- router top-k, one wavefront per token (the selection itself: route_dev.h); the
// same waves read their tokens' hidden rows for the activation pass of the fp8 and int4 layers.
#include "route_dev.h"

namespace moe {
namespace {

template <int EPL, int V>
__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
    if (blockIdx.x == 0 && a.zero_ptr && (int)threadIdx.x < a.zero_n) a.zero_ptr[threadIdx.x] = 0u;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    // fp8 and int4: the token's hidden row is requested before the routing, which runs under
    // its latency
    constexpr int XP = 8;   // 16-byte groups of the row per lane held from before the routing
    uint4 xv[XP];
    const uint4 *row = (const uint4 *)(a.x + (int64_t)(t < a.T ? t : 0) * a.x_cols);
    const int64_t n8 = (a.x_parts || a.x_perm) && t < a.T ? a.x_cols / 8 : 0;
#pragma unroll
    for (int j = 0; j < XP; j++) {
        const int64_t i = lane_id() + (int64_t)j * kWave;
        xv[j] = i < n8 ? row[i] : make_uint4(0, 0, 0, 0);
    }
    if (t < a.T) route_dev::route_token<EPL, V>(a, t);
    if (a.x_perm) {   // int4: the row with each 8 values in the nibble order (bf16x8_perm)
        uint4 *out = (uint4 *)(a.x_perm + (int64_t)t * a.x_cols);
#pragma unroll
        for (int j = 0; j < XP; j++) {
            const int64_t i = lane_id() + (int64_t)j * kWave;
            if (i < n8) out[i] = bf16x8_perm(xv[j]);
        }
        // the rest of the row in batches of XP groups, each batch's loads in flight together
        for (int64_t b = (int64_t)XP * kWave; b < n8; b += (int64_t)XP * kWave) {
            uint4 v[XP];
#pragma unroll
            for (int j = 0; j < XP; j++) {
                const int64_t i = b + lane_id() + (int64_t)j * kWave;
                v[j] = i < n8 ? row[i] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < XP; j++) {
                const int64_t i = b + lane_id() + (int64_t)j * kWave;
                if (i < n8) out[i] = bf16x8_perm(v[j]);
            }
        }
    }
    if (a.x_parts) {   // the largest |x| of this workgroup's tokens (the quantisation reduces the parts)
        float m = 0.0f;
        auto fold = [&](const uint4 &g) {
            const uint32_t w[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
                m = fmaxf(m, fabsf(__uint_as_float(w[q] << 16)));
                m = fmaxf(m, fabsf(__uint_as_float(w[q] & 0xFFFF0000u)));
            }
        };
#pragma unroll
        for (int j = 0; j < XP; j++) fold(xv[j]);
        for (int64_t b = (int64_t)XP * kWave; b < n8; b += (int64_t)XP * kWave) {   // the rest, XP at a time
            uint4 v[XP];
#pragma unroll
            for (int j = 0; j < XP; j++) {
                const int64_t i = b + lane_id() + (int64_t)j * kWave;
                v[j] = i < n8 ? row[i] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < XP; j++) fold(v[j]);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
        __shared__ float wmax[4];
        if (lane_id() == 0) wmax[threadIdx.x >> 6] = m;
        __syncthreads();
        if (threadIdx.x == 0)
            a.x_parts[blockIdx.x] = __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    }
}

// one instantiation per (experts per lane, routing variant): each holds only its own path
template <int EPL>
void launch_epl(const RouteArgs &a, dim3 grid, dim3 block, hipStream_t s) {
    switch (route_dev::route_variant(a.kind, a.E, a.n_group)) {
    case route_dev::V_SOFTMAX: hipLaunchKernelGGL((k_route<EPL, route_dev::V_SOFTMAX>), grid, block, 0, s, a); break;
    case route_dev::V_SIGMOID: hipLaunchKernelGGL((k_route<EPL, route_dev::V_SIGMOID>), grid, block, 0, s, a); break;
    case route_dev::V_GROUPED_POW2: hipLaunchKernelGGL((k_route<EPL, route_dev::V_GROUPED_POW2>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((k_route<EPL, route_dev::V_GROUPED_ANY>), grid, block, 0, s, a); break;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
    const dim3 grid((a.T + 3) / 4 > 0 ? (a.T + 3) / 4 : 1), block(256);
    if (a.E <= 64)
        launch_epl<1>(a, grid, block, s);
    else if (a.E <= 128)
        launch_epl<2>(a, grid, block, s);
    else
        launch_epl<4>(a, grid, block, s);
    return hipGetLastError();
}

}  // namespace moe
