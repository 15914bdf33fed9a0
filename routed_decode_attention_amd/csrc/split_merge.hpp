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
// splits are taken in chunks of MERGE_CHUNK, every load of a chunk issued at
// once; a running (M, L, A) is rescaled to each chunk's new max, and within
// a chunk the splits are added in order.
__device__ __forceinline__ f32x4 merge_splits4(const float* acc, const float* ml, int nws, int G, int R, int h,
                                               int r0) {
  constexpr float NEG = -__builtin_huge_valf();
  float M = NEG, L = 0.f;
  f32x4 A = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nws; s0 += MERGE_CHUNK) {
    float2 p[MERGE_CHUNK];
    f32x4 a4[MERGE_CHUNK];
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i) {
      const int s = s0 + i < nws ? s0 + i : nws - 1;
      p[i] = *reinterpret_cast<const float2*>(ml + (s * G + h) * 2);
      a4[i] = *reinterpret_cast<const f32x4*>(acc + ((size_t)s * G + h) * R + r0);
    }
    float Mc = M;
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i)
      if (s0 + i < nws) Mc = fmaxf(Mc, p[i].x);
    if (Mc == NEG) continue;  // nothing attended so far
    const float c = exp2f(M - Mc);  // 0 while M is -inf
    L *= c;
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] *= c;
#pragma unroll
    for (int i = 0; i < MERGE_CHUNK; ++i)
      if (s0 + i < nws) {
        const float e = exp2f(p[i].x - Mc);
        L = fmaf(e, p[i].y, L);
#pragma unroll
        for (int k = 0; k < 4; ++k) A[k] = fmaf(e, a4[i][k], A[k]);
      }
    M = Mc;
  }
  if (L > 0.f) {
    const float inv = 1.f / L;
#pragma unroll
    for (int k = 0; k < 4; ++k) A[k] *= inv;
  }
  return A;
}

}  // namespace bkv
