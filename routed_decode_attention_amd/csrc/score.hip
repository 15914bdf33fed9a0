// Router scores, host side: the cluster plan, the LDS limit and the launch,
// dispatched to the per-dtype translation units that instantiate the kernel
// (score_kernel.hpp).
#include <algorithm>
#include <cstdlib>

#include "score_kernel.hpp"

namespace bkv {

// The kernel's static LDS (the projected queries, the token's buffers) is
// under 14 KiB; gfx950 has 160 KiB of LDS per CU and 256 CUs.
constexpr size_t SC_STATIC_LDS = 14 * 1024, CU_LDS = 160 * 1024;

void score_plan(const Shape& s, bool append, int* cluster, int* per) {
  // Pages per scoring workgroup: few, so that a pair's sums load over many
  // CUs at once (each workgroup is two memory round trips, whatever its
  // share), but not so few that the grid needs a second round of residency
  // (long contexts: 70B 128K share, 2048 pages, 32 pairs); at most 256 (four
  // pages per quad).  Resident workgroups: at most four per CU (VGPRs), fewer
  // when LDS decides (every workgroup of a launch reserves the appender's
  // regions too).
  const size_t lds = score_lds(s.head_dim, s.rank_v, s.rank_k, s.group, s.page_size, s.dtype == 0 ? 4 : 2,
                               append).total + SC_STATIC_LDS;
  const long resident = (long)std::min<size_t>(4, CU_LDS / lds) * 256;
  const long pairs = (long)s.batch * s.n_kv_heads;
  const long room = resident - pairs * (append ? 1 : 0);  // the appenders take one each
  int p = 64;
  if (room > 0) p = (int)std::max<long>(64, (pairs * s.max_pages + room - 1) / room);
  p = std::min(p, 256);
  if (const char* e = getenv("BASISKV_SCORE_PAGES_PER_WG")) p = std::max(1, std::min(256, atoi(e)));
  const int scorers = (s.max_pages + p - 1) / p;
  *per = p;
  *cluster = scorers + (append ? 1 : 0);
}

bool score_fits(const Shape& s, bool append) {
  const size_t lds = score_lds(s.head_dim, s.rank_v, s.rank_k, s.group, s.page_size, s.dtype == 0 ? 4 : 2,
                               append).total;
  return lds + SC_STATIC_LDS <= CU_LDS;
}

hipError_t launch_score(const ScoreArgs& a, hipStream_t st) {
  return a.s.dtype == 0 ? launch_score_f32(a, st) : launch_score_bf16(a, st);
}

}  // namespace bkv
