// Router scores, host side: the cluster plan, the LDS limit and the launch,
// dispatched to the per-dtype translation units that instantiate the kernel
// (score_kernel.hpp).
#include <algorithm>
#include <cstdlib>

#include "score_kernel.hpp"

namespace bkv {

void score_plan(const Shape& s, bool append, int* cluster, int* per) {
  // Pages per scoring workgroup: few, so that a pair's sums load over many
  // CUs at once (each workgroup is two memory round trips, whatever its
  // share); at most 256 (four pages per quad).
  int p = 64;
  if (const char* e = getenv("BASISKV_SCORE_PAGES_PER_WG")) p = std::max(1, std::min(256, atoi(e)));
  const int scorers = (s.max_pages + p - 1) / p;
  *per = p;
  *cluster = scorers + (append ? 1 : 0);
}

bool score_fits(const Shape& s, bool append) {
  // the kernel's static arrays take under 14 KiB; gfx950 has 160 KiB per CU
  const size_t lds = score_lds(s.head_dim, s.rank_v, s.rank_k, s.group, s.page_size, s.dtype == 0 ? 4 : 2,
                               append).total;
  return lds + 14 * 1024 <= 160 * 1024;
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  return a.s.dtype == 0 ? launch_score_f32(a, st) : launch_score_bf16(a, st);
}

}  // namespace bkv
