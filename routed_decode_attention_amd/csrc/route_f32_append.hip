// Router kernels for fp32 storage, fused with the append.
#include "route_kernel.hpp"

namespace bkv {

hipError_t launch_route_f32_append(const RouteArgs& a, hipStream_t st) { return launch_d<float, true>(a, st); }

}  // namespace bkv
