// Router score kernels for fp32 storage (split from score.hip to keep each
// translation unit's compile short).
#include "score_kernel.hpp"

namespace bkv {
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t st) { return launch_score_t<float>(a, st); }
}  // namespace bkv
