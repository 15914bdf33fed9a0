// Router host side: cluster sizing, LDS limits and the launch, dispatched to
// the per-dtype translation units that instantiate the kernel
// (route_kernel.hpp).
#include "route_kernel.hpp"

namespace bkv {

int route_cluster(const Shape& s, bool append, bool counters) {
  if (!counters) return 1;
  int per = 512;  // pages per scoring workgroup: one load group of its quads
  if (const char* e = getenv("BASISKV_ROUTE_PAGES_PER_WG")) per = std::max(1, std::min(8192, atoi(e)));
  else if (s.max_pages <= 128) return 1;  // one workgroup scores while it appends
  const int nsc = (s.max_pages + per - 1) / per;
  return std::min(nsc + (append ? 1 : 0), 32);
}

bool route_fits(const Shape& s, bool append) {
  // the kernel's static arrays take under 24 KiB; gfx950 has 160 KiB per CU
  return route_lds_bytes(s, append) + 24 * 1024 <= 160 * 1024;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const bool append = a.pos != nullptr;
  if (a.s.dtype == 0) return append ? launch_route_f32_append(a, st) : launch_route_f32(a, st);
  return append ? launch_route_bf16_append(a, st) : launch_route_bf16(a, st);
}

}  // namespace bkv
