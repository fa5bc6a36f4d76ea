// route.hip -- router top-k, one wavefront per token (the selection itself: route_dev.h).
#include "route_dev.h"

namespace moe {
namespace {

template <int EPL, int V>
__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
    if (blockIdx.x == 0 && a.zero_ptr && (int)threadIdx.x < a.zero_n) a.zero_ptr[threadIdx.x] = 0u;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t < a.T) route_dev::route_token<EPL, V>(a, t);
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
