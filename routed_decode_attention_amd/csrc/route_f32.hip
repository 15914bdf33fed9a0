// Router kernels for fp32 storage.
#include "route_kernel.hpp"

namespace bkv {

hipError_t launch_route_f32(const RouteArgs& a, hipStream_t st) { return launch_d<float, false>(a, st); }

}  // namespace bkv
