// Combining split-K attention partials (flash decoding): a split holds the
// running max m, the denominator l = sum_t 2^(s_t - m) and the unnormalised
// latent sum acc = sum_t 2^(s_t - m) z~_t over its tokens (scores s_t in log2
// units).  The softmax over all tokens is recovered exactly by rescaling each
// split to the common max M (machinelearning.ru "KV-кэширование",
// "Математическая формализация": softmax(q.k / sqrt(d_h)) weights on the
// cached values; here the values are the stored latents).
#pragma once

#include "common.hpp"

namespace bkv {

constexpr int MERGE_CHUNK = 16;  // splits whose partials are requested together

// z[r0 .. r0+3] of query head h of one (sequence, KV head) pair:
//   M = max_s m_s,  L = sum_s 2^(m_s - M) l_s,  A = sum_s 2^(m_s - M) acc_s,
//   z = A / L (0 when the pair has no token).
// acc: the pair's [n_wsplit][G][R]; ml: the pair's [n_wsplit][G][2].  The
// splits are taken in chunks of MERGE_CHUNK whose loads are issued together
// (load), then folded into a running (M, L, A) rescaled to each chunk's new
// max, splits in order within a chunk (fold); finish() normalises.
// (CH: splits requested together, MERGE_CHUNK unless a kernel needs fewer
// registers for it.)
template <int CH>
struct SplitMergeT {
  static constexpr int MERGE_CHUNK = CH;
  const float *acc, *ml;
  int nws, G, R, h, r0;
  float M = -__builtin_huge_valf(), L = 0.f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  float2 p[MERGE_CHUNK];
  f32x4 a4[MERGE_CHUNK];

  __device__ __forceinline__ void load(int s0) {
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i) {
      const int s = s0 + i < nws ? s0 + i : nws - 1;
      p[i] = *reinterpret_cast<const float2*>(ml + (s * G + h) * 2);
      a4[i] = *reinterpret_cast<const f32x4*>(acc + ((size_t)s * G + h) * R + r0);
    }
  }
  __device__ __forceinline__ void fold(int s0) {
    constexpr float NEG = -__builtin_huge_valf();
    float Mc = M;
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i)
      if (s0 + i < nws) Mc = fmaxf(Mc, p[i].x);
    // branch-free: with nothing attended yet (Mc = -inf) every weight is 0
    const float base = Mc == NEG ? 0.f : Mc;
    const float c = M == NEG ? 0.f : exp2f(M - base);
    L *= c;
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] *= c;
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i) {
      const float e = s0 + i < nws ? exp2f(p[i].x - base) : 0.f;
      L = fmaf(e, p[i].y, L);
#pragma unroll
      for (int k = 0; k < 4; ++k) A[k] = fmaf(e, a4[i][k], A[k]);
    }
    M = Mc;
  }
  __device__ __forceinline__ f32x4 finish() const {
    f32x4 z = A;
    if (L > 0.f) {
      const float inv = 1.f / L;
#pragma unroll
      for (int k = 0; k < 4; ++k) z[k] *= inv;
    }
    return z;
  }
};

using SplitMerge = SplitMergeT<MERGE_CHUNK>;

__device__ __forceinline__ f32x4 merge_splits4(const float* acc, const float* ml, int nws, int G, int R, int h,
                                               int r0) {
  SplitMerge m{acc, ml, nws, G, R, h, r0};
  for (int s0 = 0; s0 < nws; s0 += MERGE_CHUNK) {
    m.load(s0);
    __builtin_amdgcn_sched_barrier(0);
    m.fold(s0);
  }
  return m.finish();
}

}  // namespace bkv
