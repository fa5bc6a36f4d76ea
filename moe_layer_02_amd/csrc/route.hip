// route.hip -- router top-k, one wavefront per token (the selection itself: route_dev.h).
#include "route_dev.h"

namespace moe {
namespace {

template <int EPL>
__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
    if (blockIdx.x == 0 && a.zero_ptr && (int)threadIdx.x < a.zero_n) a.zero_ptr[threadIdx.x] = 0u;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < a.T) route_dev::route_token<EPL>(a, t);
}

}  // namespace

hipError_t launch_route(const RouteArgs &a, hipStream_t s) {
    const dim3 grid((a.T + 3) / 4 > 0 ? (a.T + 3) / 4 : 1), block(256);
    if (a.E <= 64)
        hipLaunchKernelGGL(k_route<1>, grid, block, 0, s, a);
    else if (a.E <= 128)
        hipLaunchKernelGGL(k_route<2>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(k_route<4>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
