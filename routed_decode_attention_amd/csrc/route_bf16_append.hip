// Router kernels for bf16 storage, fused with the append.
#include "route_kernel.hpp"

namespace bkv {

hipError_t launch_route_bf16_append(const RouteArgs& a, hipStream_t st) { return launch_d<uint16_t, true>(a, st); }

}  // namespace bkv
