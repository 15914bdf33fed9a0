// Router score kernels for bf16 storage (split from score.hip to keep each
// translation unit's compile short).
#include "score_kernel.hpp"

namespace bkv {
hipError_t launch_score_bf16(const ScoreArgs& a, hipStream_t st) { return launch_score_t<uint16_t>(a, st); }
}  // namespace bkv
