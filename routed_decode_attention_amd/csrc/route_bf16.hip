// Router kernels for bf16 storage.
#include "route_kernel.hpp"

namespace bkv {

hipError_t launch_route_bf16(const RouteArgs& a, hipStream_t st) { return launch_d<uint16_t, false>(a, st); }

}  // namespace bkv
