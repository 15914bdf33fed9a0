// Router scores, host side: the cluster plan, the LDS limit and the launch,
// dispatched to the per-dtype translation units that instantiate the kernel
// (score_kernel.hpp).
#include <algorithm>
#include <cstdlib>

#include "score_kernel.hpp"

namespace bkv {

// Workgroups of the scoring launch that are resident at once: four per CU
// (about 40 KiB of LDS and at most 128 VGPRs each) on 256 CUs.
constexpr long SC_RESIDENT = 4 * 256;

void score_plan(const Shape& s, bool append, int* cluster, int* per) {
  // Pages per scoring workgroup: few, so that a pair's sums load over many
  // CUs at once (each workgroup is two memory round trips, whatever its
  // share), but not so few that the grid needs a second round of residency
  // (long contexts: 70B 128K share, 2048 pages, 32 pairs -> 67 a workgroup);
  // at most 256 (four pages per quad).
  const long pairs = (long)s.batch * s.n_kv_heads;
  const long room = SC_RESIDENT - pairs * (append ? 1 : 0);  // the appenders take one each
  int p = 64;
  if (room > 0) p = (int)std::max<long>(64, (pairs * s.max_pages + room - 1) / room);
  p = std::min(p, 256);
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
