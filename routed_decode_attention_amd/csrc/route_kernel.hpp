// Router: page scores predicted from the Value latents plus the Key residual,
// then top-k page selection per (sequence, KV head); optionally fused with
// the decode-step append of the new token.
//
// weekinpapers "BasisKV: Value Latents for Communication and Key Routing",
// Abstract: the compressed Value cache predicts part of the Key information
// needed for routing and a Key-specific residual stores the rest; kongchang
// article, section on Value-latent Key routing (cheap coarse routing, exact
// scoring afterwards).  With the predicted Key k~_t = z~_t.P + s~_t.R_dec the
// score of page j for query head h is scale * q_h . mean_t k~_t, which by
// linearity is scale * ((P.q_h) . sumz_j + (R_dec.q_h) . sums_j) / cnt_j.
// The group's score is the max over its query heads; the min(top_k, n_pg)
// best pages are kept (ties to the smaller page) and listed in ascending order.
// Decode appends the new token before attending (machinelearning.ru
// "KV-кэширование", "Фаза Decode"), so the fused variant writes it first.
//
// A cluster of 512-thread workgroups per (sequence, KV head) when a
// workspace provides arrival counters: with an append, workgroup 0 writes
// the new token and scores its page while the others score the remaining
// pages (up to 512 each) and select among them; the appending workgroup and
// the selecting one meet at a 64-bit word, and the second to arrive adds the
// appended page to the selection.  Without counters one workgroup does
// everything.  The kernel is a short chain of memory round trips, and its
// serial parts are kept to few instructions:
//   1. the page-table row, the factors, the query and the new token are
//      copied straight into LDS together (16-byte direct loads);
//   2. every scoring lane requests the sums of its pages; the waves project
//      the query through P and R_dec (four lanes per output) and, when
//      appending, split the new token's three products between them
//      (partials added in LDS in the chunk writer's order);
//   3. when appending, wave 0 stores the token and rebuilds its page's sums
//      from the page's LDS image, then scores that page; a quad of lanes
//      scores one page from its fp32 sums held in registers;
//   4. up to 512 pages and 64 selected: a sorting network on 64-bit
//      (key, ~page) values (a wave per 64 keys, three merge levels through
//      LDS), each selected page's slot in page order counted by its lane;
//      larger selections: an MSB-first 8-bit radix select over
//      order-preserving keys in LDS (per-wave histograms, scanned by every
//      wave, one barrier a pass) finds the k-th score, and ballots plus
//      per-wave counts compact the selection in page order.
#pragma once

#include <algorithm>
#include <cstdlib>

#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int RT = 512;
constexpr int NW = RT / 64;
constexpr int VMAX = 64;                      // page-sum channels held in registers per pass
constexpr int XMAX = MAX_RANK + MAX_RESID;    // projected-query width bound

// Sum over the four lanes of a quad (every lane gets the total).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lanes ^1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lanes ^2
  return x;
}

// Wave-wide max / min of a 32-bit key (every lane gets the result).
// (lanes without a source, e.g. past a row end for row_shl, read 0)
#define BKV_DPPU(x, ctrl) (uint32_t) __builtin_amdgcn_mov_dpp((int)(x), ctrl, 0xF, 0xF, true)
__device__ __forceinline__ uint32_t wave_umax(uint32_t x) {
  x = max(x, BKV_DPPU(x, 0xB1));
  x = max(x, BKV_DPPU(x, 0x4E));
  x = max(x, BKV_DPPU(x, 0x124));  // row_ror:4
  x = max(x, BKV_DPPU(x, 0x128));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t x) {
  x = min(x, BKV_DPPU(x, 0xB1));
  x = min(x, BKV_DPPU(x, 0x4E));
  x = min(x, BKV_DPPU(x, 0x124));
  x = min(x, BKV_DPPU(x, 0x128));
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min(r[0], r[1]);
}
__device__ __forceinline__ uint32_t wave_uadd(uint32_t x) {
  x += BKV_DPPU(x, 0xB1);
  x += BKV_DPPU(x, 0x4E);
  x += BKV_DPPU(x, 0x124);
  x += BKV_DPPU(x, 0x128);
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = r[0] + r[1];
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return r[0] + r[1];
}

// The value lane (lane ^ J) holds, J in {1, 2, 4, 8, 16, 32}: DPP within a
// 16-lane row, gfx950's lane-half swaps across rows.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (J == 1) {
    return BKV_DPPU(x, 0xB1);
  } else if constexpr (J == 2) {
    return BKV_DPPU(x, 0x4E);
  } else if constexpr (J == 4) {
    const uint32_t up = BKV_DPPU(x, 0x104), dn = BKV_DPPU(x, 0x114);  // row_shl:4 (lane + 4), row_shr:4
    return (lane & 4) ? dn : up;
  } else if constexpr (J == 8) {
    return BKV_DPPU(x, 0x128);  // row_ror:8
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
#undef BKV_DPPU

// the same for a 64-bit value, one half at a time
template <int J>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t x, int lane) {
  return (uint64_t)lane_xor<J>((uint32_t)(x >> 32), lane) << 32 | lane_xor<J>((uint32_t)x, lane);
}

// Bitonic sorting network over the 64 lanes of a wave on 64-bit values: one
// compare-exchange with lane ^ J inside blocks of K lanes; a whole sort
// (descending unless `up`), and the final merge of a bitonic sequence.
template <int J>
__device__ __forceinline__ void bitonic_step(uint64_t& x, int lane, int K, bool up) {
  const bool keep_max = (((lane & J) == 0) == ((lane & K) == 0)) != up;
  const uint64_t p = lane_xor64<J>(x, lane);
  if (keep_max == (p > x)) x = p;
}
__device__ __forceinline__ void bitonic_merge(uint64_t& x, int lane, bool up) {
  bitonic_step<32>(x, lane, 64, up);
  bitonic_step<16>(x, lane, 64, up);
  bitonic_step<8>(x, lane, 64, up);
  bitonic_step<4>(x, lane, 64, up);
  bitonic_step<2>(x, lane, 64, up);
  bitonic_step<1>(x, lane, 64, up);
}
__device__ __forceinline__ void bitonic_sort(uint64_t& x, int lane, bool up) {
  bitonic_step<1>(x, lane, 2, up);
  bitonic_step<2>(x, lane, 4, up);
  bitonic_step<1>(x, lane, 4, up);
  bitonic_step<4>(x, lane, 8, up);
  bitonic_step<2>(x, lane, 8, up);
  bitonic_step<1>(x, lane, 8, up);
  bitonic_step<8>(x, lane, 16, up);
  bitonic_step<4>(x, lane, 16, up);
  bitonic_step<2>(x, lane, 16, up);
  bitonic_step<1>(x, lane, 16, up);
  bitonic_step<16>(x, lane, 32, up);
  bitonic_step<8>(x, lane, 32, up);
  bitonic_step<4>(x, lane, 32, up);
  bitonic_step<2>(x, lane, 32, up);
  bitonic_step<1>(x, lane, 32, up);
  bitonic_merge(x, lane, up);
}


// best[i] = max over the group's heads h of qc[h] . sums(page i), each dot
// split over the four lanes of a quad (NG 16-byte channel granules per lane,
// granule part + 4u) and summed by the quad; the group's max (MEAN: mean)
// over its query heads.
template <int NG, int PPL, bool MEAN>
__device__ __forceinline__ void score_group(const f32x4 (&sv)[PPL][NG], const float (*qc)[XMAX], int G, int part,
                                            float (&best)[PPL]) {
#pragma unroll
  for (int i = 0; i < PPL; ++i) best[i] = MEAN ? 0.f : -__builtin_huge_valf();
  for (int h = 0; h < G; ++h) {
    f32x4 qg[NG];
#pragma unroll
    for (int u = 0; u < NG; ++u) qg[u] = *reinterpret_cast<const f32x4*>(&qc[h][4 * (part + 4 * u)]);
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < NG; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = fmaf(qg[u][e], sv[i][u][e], acc);
      if constexpr (MEAN) best[i] += quad_sum(acc);
      else best[i] = fmaxf(best[i], quad_sum(acc));
    }
  }
  if constexpr (MEAN)
#pragma unroll
    for (int i = 0; i < PPL; ++i) best[i] /= (float)G;
}

// Four consecutive storage-dtype elements from LDS as fp32.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// Dynamic LDS layout (bytes, every part 16-byte aligned).
struct RouteLds {
  size_t pid, P, Rd, q, B, Re, vk, img, keys, total;
};
__host__ __device__ inline size_t a16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ inline RouteLds route_lds(int maxp, int D, int R, int RK, int G, int ps, int es, bool append) {
  RouteLds L;
  L.pid = 0;
  L.P = a16((size_t)maxp * 4);
  L.Rd = L.P + (size_t)R * D * 4;
  L.q = L.Rd + (size_t)RK * D * 4;
  L.B = L.q + a16((size_t)G * D * es);
  L.Re = L.B + (append ? (size_t)D * R * 4 : 0);
  L.vk = L.Re + (append ? (size_t)D * RK * 4 : 0);
  L.img = L.vk + (append ? (size_t)2 * D * es : 0);
  L.total = L.img + (append ? (size_t)(R * ps + ps * RK) * es : 0);
  // the score keys reuse the factors' space (written once the query
  // projections are done), unless they would reach the appended token and
  // page image, which are still in use while the pages are scored
  L.keys = L.P;
  if (!append) {
    if (L.total < L.P + (size_t)maxp * 4) L.total = L.P + (size_t)maxp * 4;
  } else if (L.P + (size_t)maxp * 4 > L.vk) {
    L.keys = a16(L.total);
    L.total = L.keys + (size_t)maxp * 4;
  }
  return L;
}

// NG: 16-byte channel granules per scoring lane, at least ceil((r + r_k) / 16)
// FORCE: pages kept at either end of the sequence (sink_pages, local_pages);
// MEAN: a page's score is the mean over the group's query heads, not the
// max.  Each compiled in only when a call asks for it.
template <typename T, bool APPEND, int D, int NG, bool FORCE, bool MEAN>
__global__ __launch_bounds__(RT) void route_kernel(RouteArgs a) {
  constexpr int PPL = 4;  // pages per scoring quad and load group
  extern __shared__ __attribute__((aligned(16))) float lds[];
  static_assert(NW == CW, "one real wave per virtual wave of the token arithmetic");
  __shared__ __attribute__((aligned(16))) float s_qc[MAX_GROUP][XMAX];   // scale * (P.q_h | R_dec.q_h), zero past r + r_k
  __shared__ __attribute__((aligned(16))) float s_e[128];              // appended token's Key remainder
  __shared__ __attribute__((aligned(16))) float s_st[XMAX];            // appended token's stored values (latent, residual)
  __shared__ __attribute__((aligned(16))) float s_newsum[XMAX];        // the appended page's sums
  __shared__ __attribute__((aligned(16))) float s_work[NW * 256];      // token partials, then the radix histograms

  const int H = a.s.n_kv_heads, G = a.s.group;
  const int C = gridDim.x / (a.s.batch * H);  // workgroups per (sequence, KV head)
  // a pair's workgroups on one XCD, the one the attention kernel gives the
  // pair's splits, so the selection it reads back is in that XCD's L2
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = L / C, c = L - pair * C;
  const int R = a.s.rank_v, RK = a.s.rank_k, RR = R + RK, ps = a.s.page_size;
  const int maxp = a.s.max_pages;
  const int b = pair / H, g = pair % H;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int32_t* pt = a.page_table + (size_t)b * maxp;
  char* base = reinterpret_cast<char*>(lds);
  const RouteLds lay = route_lds(maxp, D, R, RK, G, ps, (int)sizeof(T), APPEND);
  int32_t* s_pid = reinterpret_cast<int32_t*>(base + lay.pid);  // [maxp] the page-table row
  float* sP = reinterpret_cast<float*>(base + lay.P);            // [R][D] rotated
  float* sRd = reinterpret_cast<float*>(base + lay.Rd);          // [RK][D] rotated
  T* sq = reinterpret_cast<T*>(base + lay.q);                    // [G][D] the group's query heads
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(base + lay.keys);  // [maxp], once the projections are done

  // ---- round trip 1: page-table row, sequence length, append position,
  // factors, query and new token, all requested together ----
  const int n = a.seq_lens[b];
  int pos = -1;
  if (APPEND) {
    pos = a.pos[b];
    if (pos < 0 || pos >= maxp * ps) pos = -1;
  }
  const bool app = APPEND && pos >= 0;
  const bool app0 = app && c == 0;  // this workgroup appends the token
  const int apage = app ? pos / ps : 0, slot = app ? pos % ps : 0;
  const int npg = n > 0 ? min((n + ps - 1) / ps, maxp) : 0;
  // pages [lo, hi) scored here: with an append in a cluster, workgroup 0
  // appends (and scores the appended page) and the others share the pages
  const int nsc = APPEND && C > 1 ? C - 1 : C, sidx = APPEND && C > 1 ? c - 1 : c;
  const int per = (npg + nsc - 1) / nsc;
  const int lo = sidx < 0 ? 0 : min(npg, sidx * per), hi = sidx < 0 ? 0 : min(npg, lo + per);
  const bool in_regs = RR <= VMAX;  // a page's sums fit one lane's registers
  const bool pt16 = (maxp & 3) == 0 && (reinterpret_cast<uintptr_t>(pt) & 15) == 0;
  {
    const char* P = reinterpret_cast<const char*>(a.P + (size_t)g * R * D);
    const char* Rd = reinterpret_cast<const char*>(a.R_dec + (size_t)g * RK * D);
    const char* q = reinterpret_cast<const char*>(static_cast<const T*>(a.q) + ((size_t)b * a.s.n_q_heads + g * G) * D);
    const char* ptc = reinterpret_cast<const char*>(pt);
    int first = dma_stage(sP, R * D / 4, [&](int G_) { return P + 16 * rot_source(G_, D); }, 0, NW, wave, lane);
    first = dma_stage(sRd, RK * D / 4, [&](int G_) { return Rd + 16 * rot_source(G_, D); }, first, NW, wave, lane);
    first = dma_stage(sq, (int)(G * D * sizeof(T) / 16), [&](int G_) { return q + 16 * G_; }, first, NW, wave, lane);
    if (pt16) first = dma_stage(s_pid, maxp / 4, [&](int G_) { return ptc + 16 * G_; }, first, NW, wave, lane);
    if (app0) {
      const char* B = reinterpret_cast<const char*>(a.B + (size_t)g * D * R);
      const char* Re = reinterpret_cast<const char*>(a.R_enc + (size_t)g * D * RK);
      const size_t tok = ((size_t)b * H + g) * D;
      const char* vn = reinterpret_cast<const char*>(static_cast<const T*>(a.v_new) + tok);
      const char* kn = reinterpret_cast<const char*>(static_cast<const T*>(a.k_new) + tok);
      const int tc = (int)(D * sizeof(T) / 16);
      first = dma_stage(base + lay.B, D * R / 4, [&](int G_) { return B + 16 * G_; }, first, NW, wave, lane);
      first = dma_stage(base + lay.Re, D * RK / 4, [&](int G_) { return Re + 16 * G_; }, first, NW, wave, lane);
      dma_stage(base + lay.vk, 2 * tc, [&](int G_) { return G_ < tc ? vn + 16 * G_ : kn + 16 * (G_ - tc); }, first,
                NW, wave, lane);
    }
  }
  if (!pt16)
    for (int j = tid; j < maxp; j += RT) s_pid[j] = pt[j];
  __syncthreads();

  // ---- round trip 2: page sums for scoring, requested now.  Four lanes
  // per page: lane `part` of a quad holds channel granules part + 4u of its
  // page's row (contiguous 64 bytes per quad and load); quad q of nq takes
  // pages lo + q + nq m, PPL of them per group.  In the appending workgroup
  // wave 0 writes the token while waves 1.. score ----
  const int nq = app0 ? 16 * (NW - 1) : 16 * NW;
  const int quad = (app0 ? wave - 1 : wave) * 16 + (lane >> 2), part = lane & 3;
  const bool scorer = !(app0 && wave == 0);
  f32x4 sv[PPL][NG];
  // The loads are unconditional (a page past the sequence reads page 0, a
  // granule past the row reads the row's last one), so all of a group's
  // requests are in flight together; mask_group() zeroes the extra ones
  // right before the scores need them.
  uint32_t svok = 0;  // bit 4 i + u: sv[i][u] holds real sums
  auto load_group = [&](int m0) {
    if (npg == 0) return;
    svok = 0;
#pragma unroll
    for (int i = 0; i < PPL; ++i) {
      const int jj = quad + nq * (m0 + i);  // negative on the appending wave
      const bool ok = (unsigned)jj < (unsigned)(hi - lo);
      const f32x4* row = reinterpret_cast<const f32x4*>(a.summ + ((size_t)s_pid[ok ? lo + jj : 0] * H + g) * RR);
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int gr = part + 4 * u;
        sv[i][u] = row[min(gr, RR / 4 - 1)];
        svok |= (uint32_t)(ok && 4 * gr < RR) << (4 * i + u);
      }
    }
  };
  auto mask_group = [&]() {
#pragma unroll
    for (int i = 0; i < PPL; ++i)
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const uint32_t keep = 0u - ((svok >> (4 * i + u)) & 1u);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[i][u][e] = __uint_as_float(__float_as_uint(sv[i][u][e]) & keep);
      }
  };
  auto score = [&](float (&best)[PPL]) { score_group<NG, PPL, MEAN>(sv, s_qc, G, part, best); };
  // (in a cluster the scores are read back by another workgroup: stored
  // coherently at device scope)
  auto finish = [&](int j, float best) {
    const float sc = best / (float)min(ps, n - j * ps);
    if (C > 1) __hip_atomic_store(a.scores + (size_t)pair * maxp + j, sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else a.scores[(size_t)pair * maxp + j] = sc;
    s_keys[j] = float_key(sc);
  };

  // the appended page and its LDS image (wave 0)
  const int aphys = app0 ? s_pid[apage] : 0;
  T* Kp = static_cast<T*>(a.K) + ((size_t)aphys * H + g) * ps * D;
  T* Zp = static_cast<T*>(a.Z) + ((size_t)aphys * H + g) * R * ps;
  T* Sp = static_cast<T*>(a.S) + ((size_t)aphys * H + g) * ps * RK;
  T* img = reinterpret_cast<T*>(base + lay.img);
  PageImage pg;
  if (app0 && wave == 0) pg.load(Zp, Sp, (int)(R * ps * sizeof(T) / 16), (int)(ps * RK * sizeof(T) / 16), lane);
  // ---- the query seen through the latent predictor P and the residual
  // decoder R_dec: one task per (output row x, quarter c) for every head,
  // lane c taking 16-byte pieces 4u + c of the row; a quad sums the
  // quarters.  Outputs past r + r_k (up to VMAX) are zero.  The appending
  // workgroup of a cluster needs them only for its last score, so it
  // computes them later, beside the page sums ----
  auto qproj = [&](int t0, int stride) {
    for (int t = t0; t < RR * 4; t += stride) {
      const int x = t >> 2, c = t & 3;
      const int xr = x < R ? x : x - R;
      const float* row = (x < R ? sP : sRd) + xr * D;
      f32x4 pr[D / 16];
#pragma unroll
      for (int u = 0; u < D / 16; ++u) pr[u] = lds4(row + rot_granule(xr, 4 * u + c, D) * 4);
      for (int h = 0; h < G; ++h) {
        const T* qh = sq + h * D;
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
          const f32x4 q4 = lds4(qh + 16 * u + 4 * c);
          acc = fmaf(pr[u][0], q4[0], acc);
          acc = fmaf(pr[u][1], q4[1], acc);
          acc = fmaf(pr[u][2], q4[2], acc);
          acc = fmaf(pr[u][3], q4[3], acc);
        }
        acc = quad_sum(acc);
        if (c == 0) s_qc[h][x] = acc * a.s.scale;
      }
    }
    if (RR < VMAX)
      for (int t = t0; t < G * (VMAX - RR); t += stride) s_qc[t / (VMAX - RR)][RR + t % (VMAX - RR)] = 0.f;
  };
  // The waves holding query-projection tasks project first and request
  // their pages after (their requests would otherwise wait in the CU's
  // address queue behind everyone's, holding the projection back).
  const bool late_qproj = app0 && C > 1;
  const int QT = (RR * 4 + 63) & ~63;  // threads with a projection task
  const bool q_first = !late_qproj && tid < QT;
  if (q_first) qproj(tid, QT);
  // every wave requests a group (unused on the appending wave), which keeps
  // the registers of the two kinds of request apart
  if (in_regs) load_group(0);

  // the new token's three products, each split over the NW waves (wave w
  // takes the w-th eighth of the contraction); the partials meet in LDS and
  // are added in wave order, the chunk writer's order for the same split
  const T* vn = reinterpret_cast<const T*>(base + lay.vk);
  const T* kn = vn + D;
  const float* sB = reinterpret_cast<const float*>(base + lay.B);
  const float* sRe = reinterpret_cast<const float*>(base + lay.Re);
  float* s_lr = s_work;            // [NW][64] latent, later residual partials
  float* s_kp = s_work + NW * 64;  // [NW][128] Key-estimate partials
  if (app0) {
    f32x4 acc;
    int gq;
    if (part_matvec<D>(vn, sB, R, wave, lane, acc, gq))
      *reinterpret_cast<f32x4*>(s_lr + wave * 64 + 4 * gq) = acc;
  }

  lds_barrier();  // the scoring loads stay in flight

  if (app0) {
    // z~ rows of this wave, then its part of z~.P
    const int RW = R / NW;
    if (lane < RW) {
      const int x = wave * RW + lane;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += s_lr[w * 64 + x];
      s_st[x] = round_only(sum, static_cast<const T*>(nullptr));
    }
    wave_sync();
    const f32x4 kh = part_remainder<D>(s_st, sP, R, wave, lane);
    if (lane < D / 4) *reinterpret_cast<f32x4*>(s_kp + wave * 128 + 4 * lane) = kh;
    lds_barrier();
    // Key remainder rows of this wave, then its part of e.R_enc
    if (lane < D / NW) {
      const int i = wave * (D / NW) + lane;
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += s_kp[w * 128 + i];
      s_e[i] = lds_elem(kn, i) - sum;
    }
    wave_sync();
    f32x4 acc;
    int gq;
    if (part_matvec<D>(s_e, sRe, RK, wave, lane, acc, gq))
      *reinterpret_cast<f32x4*>(s_lr + wave * 64 + 4 * gq) = acc;
    lds_barrier();
  }

  if (app0 && wave != 0 && late_qproj) qproj(tid - 64, RT - 64);
  if (app0 && wave == 0) {
    // ---- wave 0: s~, the page image with the new slot, the page's sums
    // from scratch over slots [0, slot], the appended page's score, then
    // the memory writes: the token, then the page's sums ----
    if (lane < RK) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += s_lr[w * 64 + lane];
      s_st[R + lane] = round_only(sum, static_cast<const T*>(nullptr));
    }
    pg.store(img, lane);
    wave_sync();
    for (int x = lane; x < RR; x += 64) {
      if (x < R) store_elem(img, (size_t)x * ps + slot, s_st[x]);
      else store_elem(img, (size_t)R * ps + (size_t)slot * RK + (x - R), s_st[x]);
    }
    wave_sync();
    wave_page_sums(img, img + (size_t)R * ps, R, RK, ps, slot + 1, s_newsum, lane);
    wave_sync();
  }
  if (late_qproj) lds_barrier();  // the query projections of waves 1..
  if (app0 && wave == 0) {
    if (in_regs) {
      // quad 0 scores the page from its new sums
#pragma unroll
      for (int i = 0; i < PPL; ++i)
#pragma unroll
        for (int u = 0; u < NG; ++u) {
          const int gr = part + 4 * u;
          sv[i][u] = (i == 0 && lane < 4 && 4 * gr < RR) ? *reinterpret_cast<const f32x4*>(s_newsum + 4 * gr)
                                                         : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      float best[PPL];
      score(best);
      if (lane == 0 && apage < npg) finish(apage, best[0]);
    }
    const TokenLds<T> L{vn, kn, sB, sP, sRe, s_e, s_st};
    wave_token_store<T, D>(L, R, RK, ps, slot, Kp + (size_t)slot * D, Zp, Sp, lane);
    for (int x = lane; x < RR; x += 64) a.summ[((size_t)aphys * H + g) * RR + x] = s_newsum[x];
  }

  // ---- one quad per page: score from the page's fp32 sums ----
  if (in_regs) {
    if (scorer)
      for (int m0 = 0; lo + nq * m0 < hi; m0 += PPL) {
        if (m0 > 0) load_group(m0);
        mask_group();
        float best[PPL];
        score(best);
#pragma unroll
        for (int i = 0; i < PPL; ++i) {
          const int j = lo + quad + nq * (m0 + i);
          if (part == 0 && j < hi && !(app && j == apage)) finish(j, best[i]);
        }
      }
  } else {
    // wide sums (r + r_k > 64): 64 channels at a time, every head's dot
    // kept; the appending workgroup scores the appended page from its new
    // sums, the others skip it
    if (app0) lds_barrier();  // the appended page's sums are in s_newsum
    float v[VMAX];
    float d[MAX_GROUP];
    const int cnt = hi - lo + (app0 && (apage < lo || apage >= hi) && apage < npg ? 1 : 0);
    for (int t = tid; t < cnt; t += RT) {
      const int j = t < hi - lo ? lo + t : apage;
      if (app && !app0 && j == apage) continue;
      const float* sm = a.summ + ((size_t)s_pid[j] * H + g) * RR;
#pragma unroll
      for (int h = 0; h < MAX_GROUP; ++h) d[h] = 0.f;
      for (int x0 = 0; x0 < RR; x0 += VMAX) {
#pragma unroll
        for (int u = 0; u < VMAX / 4; ++u) {
          float4 t4 = {0.f, 0.f, 0.f, 0.f};
          if (x0 + 4 * u < RR) t4 = *reinterpret_cast<const float4*>(sm + x0 + 4 * u);
          v[4 * u] = t4.x;
          v[4 * u + 1] = t4.y;
          v[4 * u + 2] = t4.z;
          v[4 * u + 3] = t4.w;
        }
        if (app0 && j == apage) {
#pragma unroll
          for (int x = 0; x < VMAX; ++x)
            if (x0 + x < RR) v[x] = s_newsum[x0 + x];
        }
#pragma unroll
        for (int h = 0; h < MAX_GROUP; ++h)
          if (h < G) {
#pragma unroll
            for (int x = 0; x < VMAX; ++x)
              if (x0 + x < RR) d[h] = fmaf(s_qc[h][x0 + x], v[x], d[h]);
          }
      }
      float best = MEAN ? 0.f : -__builtin_huge_valf();
#pragma unroll
      for (int h = 0; h < MAX_GROUP; ++h)
        if (h < G) best = MEAN ? best + d[h] : fmaxf(best, d[h]);
      if constexpr (MEAN) best /= (float)G;
      finish(j, best);
    }
  }
  lds_barrier();  // the keys are in LDS; the score stores stay in flight

  // ---- selection ----
  const int top_k = a.s.top_k;
  int32_t* sel = a.sel + (size_t)pair * top_k;
  int32_t* selp = a.sel_phys ? a.sel_phys + (size_t)pair * top_k : nullptr;
  const float* scp = a.scores + (size_t)pair * maxp;
  // With an append in a cluster, the scorers select among every page but
  // the appended one and leave that partial selection in the workspace; the
  // appending workgroup and the scorers' last one then meet, and the second
  // to arrive adds the appended page (one candidate more).
  const bool split = APPEND && C > 1;
  const int excl = split && app && apage < npg ? apage : -1;
  uint32_t* pkeys = split ? a.part_keys + (size_t)pair * top_k : nullptr;
  int32_t* ppages = split ? a.part_pages + (size_t)pair * top_k : nullptr;
  auto put = [&](int p, int j) {
    sel[p] = j;
    if (selp) selp[p] = s_pid[j];
  };
  auto agent_load = [](const auto* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };

  // Data handed between the cluster's workgroups is stored with device-scope
  // atomic stores; once complete (vmcnt) they are visible to device-scope
  // loads anywhere, so the counters need no release/acquire (which would
  // write back and invalidate the L2).
  // whole workgroup: arrive at a counter, true for the n-th arrival (which
  // resets it); the workgroup's earlier device-scope stores are visible to it
  __shared__ int s_flag;
  auto last_of = [&](uint32_t* cnt, uint32_t n) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
    __syncthreads();
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = old == n - 1;
      if (s_flag) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    return s_flag != 0;
  };

  // whole workgroup: the final selection from the partial one in the
  // workspace (nS entries in page order) plus the appended page.  When
  // there are top_k entries already, the worst of them and the appended
  // page goes: the smallest key, then the largest page (the latest entry).
  __shared__ uint32_t s_wred[NW][4];
  // the scorers' copy of their partial selection, up to 1024 entries
  uint32_t* s_Sk = reinterpret_cast<uint32_t*>(s_work);
  int32_t* s_Sp = reinterpret_cast<int32_t*>(s_work) + 1024;
  auto merge_appended = [&](bool local, uint32_t ka) {
    auto part_key = [&](int p) { return local ? s_Sk[p] : agent_load(pkeys + p); };
    auto part_page = [&](int p) { return local ? s_Sp[p] : agent_load(ppages + p); };
    const int k = min(top_k, npg);
    const int nS = min(top_k, npg - (excl >= 0 ? 1 : 0));
    for (int p = k + tid; p < top_k; p += RT) {
      sel[p] = -1;
      if (selp) selp[p] = -1;
    }
    if (tid == 0) a.n_sel[pair] = k;
    if (excl < 0) {
      for (int p = tid; p < nS; p += RT) put(p, part_page(p));
      return;
    }
    const bool drop = nS == top_k;
    // per thread: entries p = tid + RT i; the first one's page kept
    int j0 = -1;
    uint32_t hk = ~0u, hl = ~0u;  // (smallest key, then largest index) as (key, ~index)
    int hj = -1, before = 0;      // its page; entries with a page below the appended one
    for (int p = tid; p < nS; p += RT) {
      const uint32_t kp = part_key(p);
      const int jp = part_page(p);
      if (p == tid) j0 = jp;
      before += jp < excl;
      if (kp < hk || (kp == hk && ~(uint32_t)p < hl)) {
        hk = kp;
        hl = ~(uint32_t)p;
        hj = jp;
      }
    }
    // workgroup reductions: the worst entry and the count before the appended page
    const uint32_t wk = wave_umin(hk);
    const uint32_t wl = wave_umin(hk == wk ? hl : ~0u);
    const unsigned long long own = __ballot(hk == wk && hl == wl);
    const int wj = __builtin_amdgcn_readlane(hj, own ? __ffsll((long long)own) - 1 : 0);
    const int wb = (int)wave_uadd((uint32_t)before);
    if (lane == 0) {
      s_wred[wave][0] = wk;
      s_wred[wave][1] = wl;
      s_wred[wave][2] = (uint32_t)wj;
      s_wred[wave][3] = (uint32_t)wb;
    }
    __syncthreads();
    uint32_t bk = ~0u, bl = ~0u;
    int bj = -1, ins = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const uint32_t kv = s_wred[v][0], lv = s_wred[v][1];
      if (kv < bk || (kv == bk && lv < bl)) {
        bk = kv;
        bl = lv;
        bj = (int)s_wred[v][2];
      }
      ins += (int)s_wred[v][3];
    }
    const bool drop_appended = drop && (ka < bk || (ka == bk && excl > bj));
    const int w = drop && !drop_appended ? (int)~bl : -1;  // index of the dropped entry
    for (int p = tid; p < nS; p += RT) {
      if (p == w) continue;
      const int jp = p == tid ? j0 : part_page(p);
      put(drop_appended ? p : p - (w >= 0 && p > w ? 1 : 0) + (jp > excl ? 1 : 0), jp);
    }
    if (tid == 0 && !drop_appended) put(ins - (w >= 0 && bj < excl ? 1 : 0), excl);
  };

  // ---- top-k of the keys s_keys[j], j < nk, j != excl: emit(p, j) for the
  // selected j in increasing order, p = 0, 1, ...
  // An MSB-first 8-bit radix select over the workgroup, starting at the
  // highest bit where the keys differ; a pass stops the search when the
  // bucket holding the k-th key is exactly what remains to be taken.  The
  // selected keys are then those whose masked value exceeds the found
  // prefix, plus the first `take_eq` (in order) of those equal to it.  Every
  // wave scans the per-wave histograms itself (they alternate between two
  // buffers), so a pass takes one barrier. ----
  const unsigned long long below = (1ull << lane) - 1ull;
  int* const s_hbuf0 = reinterpret_cast<int*>(s_work);        // [NW][256]
  int* const s_hbuf1 = reinterpret_cast<int*>(&s_qc[0][0]);  // [NW][256], free once the scores are done
  __shared__ int s_wcnt[NW][2];
  __shared__ uint32_t s_red[NW][2];
  auto select = [&](int nk, int ks, auto&& emit) {
    const int present = nk - (excl >= 0 && excl < nk ? 1 : 0);
    const bool all = ks == present;
    uint32_t prefix = 0, mask = 0;
    int take_eq = 0;
    if (!all) {
      uint32_t kmax = 0u, kmin = 0xffffffffu;
      for (int j = tid; j < nk; j += RT) {
        if (j == excl) continue;
        const uint32_t key = s_keys[j];
        kmax = max(kmax, key);
        kmin = min(kmin, key);
      }
      kmax = wave_umax(kmax);
      kmin = wave_umin(kmin);
      if (lane == 0) {
        s_red[wave][0] = kmax;
        s_red[wave][1] = kmin;
      }
      lds_barrier();
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        kmax = max(kmax, s_red[w][0]);
        kmin = min(kmin, s_red[w][1]);
      }
      const uint32_t diff = kmax ^ kmin;
      int hi = diff ? 31 - __builtin_clz(diff) : -1;
      mask = hi >= 0 ? ~((2u << hi) - 1u) : ~0u;
      prefix = kmax & mask;
      int krem = ks;
      for (int pass = 0; hi >= 0; ++pass) {
        int* hb = pass & 1 ? s_hbuf1 : s_hbuf0;
        const int shift = hi >= 7 ? hi - 7 : 0;
        const uint32_t dmask = (2u << (hi - shift)) - 1u;  // digit bits [shift, hi]
        *reinterpret_cast<int4*>(hb + wave * 256 + 4 * lane) = int4{0, 0, 0, 0};
        __builtin_amdgcn_wave_barrier();
        for (int j = tid; j < nk; j += RT) {
          const uint32_t key = s_keys[j];
          if (j != excl && (key & mask) == prefix) atomicAdd(hb + wave * 256 + ((key >> shift) & dmask), 1);
        }
        lds_barrier();
        // lane owns digits 255-4*lane .. 252-4*lane (descending)
        int cd[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const int4 h4 = *reinterpret_cast<const int4*>(hb + w * 256 + 252 - 4 * lane);
          cd[0] += h4.w;
          cd[1] += h4.z;
          cd[2] += h4.y;
          cd[3] += h4.x;
        }
        const int owns = cd[0] + cd[1] + cd[2] + cd[3];
        int run = wave_incl_scan(owns) - owns;  // keys with a larger digit than this lane's
        int digit = 0, nrem = 0, done = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (run < krem && run + cd[u] >= krem) {
            digit = 255 - 4 * lane - u;
            nrem = krem - run;
            done = cd[u] == krem - run;
          }
          run += cd[u];
        }
        const unsigned long long hit = __ballot(nrem > 0);
        const int src = __ffsll((long long)hit) - 1;
        digit = __builtin_amdgcn_readlane(digit, src);
        krem = __builtin_amdgcn_readlane(nrem, src);
        done = __builtin_amdgcn_readlane(done, src);
        prefix |= (uint32_t)digit << shift;
        mask |= dmask << shift;
        if (done || shift == 0) break;
        hi = shift - 1;
      }
      take_eq = krem;
    }
    // compaction in order: a taken key's slot is the count of taken keys
    // before it, i.e. greater keys before it plus min(equal keys before it,
    // take_eq)
    int gt_seen = 0, eq_seen = 0;
    for (int base0 = 0; base0 < nk; base0 += RT) {
      if (base0 > 0) lds_barrier();  // the previous round's counts are read
      const int j = base0 + tid;
      const bool in = j < nk && j != excl;
      const uint32_t mk = in ? (s_keys[j] & mask) : 0u;
      const bool gt = in && (all || mk > prefix);
      const bool eq = in && !all && mk == prefix;
      const unsigned long long gtm = __ballot(gt), eqm = __ballot(eq);
      if (lane == 0) {
        s_wcnt[wave][0] = __popcll(gtm);
        s_wcnt[wave][1] = __popcll(eqm);
      }
      lds_barrier();
      int gt_before = gt_seen + __popcll(gtm & below), eq_before = eq_seen + __popcll(eqm & below);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cg = s_wcnt[w][0], ce = s_wcnt[w][1];
        if (w < wave) {
          gt_before += cg;
          eq_before += ce;
        }
        gt_seen += cg;
        eq_seen += ce;
      }
      if (gt || (eq && eq_before < take_eq)) emit(gt_before + min(eq_before, take_eq), j);
    }
  };

  // the appending and the selecting workgroup meet at a 64-bit word: the
  // appender sets bit 63 and leaves its page's key in the low half, the
  // selector sets bit 62; the second to arrive (which clears the word)
  // finishes the selection
  __shared__ unsigned long long s_met;
  auto meet = [&](unsigned long long mine) {
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's stores are complete
    __syncthreads();
    if (tid == 0) {
      const unsigned long long old =
          __hip_atomic_fetch_or(a.meet + pair, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old) __hip_atomic_store(a.meet + pair, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_met = old;
    }
    __syncthreads();
    return s_met;
  };
  // ---- small selections (at most 512 pages, 2 <= top_k <= 64): a sorting
  // network.  Every wave sorts 64 keys as 64-bit values (key, ~page) —
  // larger key first, then smaller page, the selection's own order — then
  // three merge levels through LDS leave the top 64 in wave 0, one per lane;
  // each lane counts the selected pages below its own for its position in
  // page order.  The appended page is merged in by wave 0 alone: with top_k
  // candidates already, the worst of them (kept from the key order) and the
  // appended page compete. ----
  const bool fast = npg <= 512 && top_k >= 2 && top_k <= 64;
  __shared__ __attribute__((aligned(16))) uint32_t s_fpage[64];
  // wave 0: a selected page, its position in page order, the worst (hi, lo)
  uint32_t f_page = 0xffffffffu, f_rank = 0u, f_whi = 0u, f_wlo = 0u;
  auto select_fast = [&](int ks) {
    const int j = 64 * wave + lane;
    uint64_t x = 0u;
    if (j < npg && j != excl) x = (uint64_t)s_keys[j] << 32 | ~(uint32_t)j;
    bitonic_sort(x, lane, false);
    uint64_t* xs = reinterpret_cast<uint64_t*>(s_work);  // [NW][64]
#pragma unroll
    for (int lv = 1; lv < NW; lv <<= 1) {
      if (wave % (2 * lv) == lv) xs[wave * 64 + lane] = x;
      lds_barrier();
      if (wave % (2 * lv) == 0) {
        x = max(x, xs[(wave + lv) * 64 + 63 - lane]);
        bitonic_merge(x, lane, false);
      }
    }
    if (wave == 0 && ks > 0) {
      f_whi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), ks - 1);
      f_wlo = __builtin_amdgcn_readlane((uint32_t)x, ks - 1);
      f_page = lane < ks ? ~(uint32_t)x : 0xffffffffu;
      s_fpage[lane] = f_page;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint4* fp = reinterpret_cast<const uint4*>(s_fpage);
      uint32_t r = 0u;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const uint4 q = fp[m];
        r += (q.x < f_page) + (q.y < f_page) + (q.z < f_page) + (q.w < f_page);
      }
      f_rank = r;
    }
  };
  // wave 0: the final selection from the partial one (lane p < nS holds page
  // jp at position rank, worst (whi, wlo)) and the appended page with key ka
  auto merge_fast = [&](uint32_t ka, int jp, int rank) {
    const int k = min(top_k, npg);
    const int nS = min(top_k, npg - (excl >= 0 ? 1 : 0));
    if (lane == 0) a.n_sel[pair] = k;
    for (int p = k + lane; p < top_k; p += 64) {
      sel[p] = -1;
      if (selp) selp[p] = -1;
    }
    if (excl < 0 || (nS == top_k && (ka < f_whi || (ka == f_whi && ~(uint32_t)excl < f_wlo)))) {
      if (lane < nS) put(rank, jp);  // the appended page stays out
      return;
    }
    const int jw = nS == top_k ? (int)~f_wlo : -1;  // the entry it displaces
    const bool keep = lane < nS && jp != jw;
    if (keep) put(rank - (jw >= 0 && jp > jw ? 1 : 0) + (jp > excl ? 1 : 0), jp);
    const int ins = __popcll(__ballot(keep && jp < excl));
    if (lane == 0) put(ins, excl);
  };

  // pages kept whatever their score -- the first sink_pages and the last
  // local_pages of the sequence -- take a key above every score
  auto forced = [&](int j) { return j < a.sink_pages || j >= npg - a.local_pages; };
  if (split && c == 0) {  // the appending workgroup: its page's score is in
    uint32_t ka = excl >= 0 ? s_keys[excl] : 0u;
    if constexpr (FORCE)
      if (excl >= 0 && forced(excl)) ka = 0xFFFFFFFFu;
    if (meet((1ull << 63) | ka)) {
      if (!fast) {
        merge_appended(false, ka);
      } else if (wave == 0) {
        const int nS = min(top_k, npg - (excl >= 0 ? 1 : 0));
        const int jp = lane < nS ? agent_load(ppages + lane) : -1;
        f_whi = agent_load(pkeys);
        f_wlo = agent_load(pkeys + 1);
        merge_fast(ka, jp, lane);
      }
    }
    return;
  }
  if (nsc > 1) {
    // the scorers' last workgroup takes every score back (but the appended
    // page's, when split)
    if (!last_of(a.arrive + pair, (uint32_t)nsc)) return;
    for (int j = tid; j < npg; j += RT)
      if (j != excl) s_keys[j] = float_key(agent_load(scp + j));
    __syncthreads();
  }
  if constexpr (FORCE) {
    for (int j = tid; j < npg; j += RT)
      if (forced(j)) s_keys[j] = 0xFFFFFFFFu;
    lds_barrier();
  }
  const int ks = min(top_k, npg - (excl >= 0 ? 1 : 0));
  if (fast) {
    select_fast(ks);
    if (!split) {
      if (wave == 0) {
        if (lane == 0) a.n_sel[pair] = ks;
        if (lane < ks) put((int)f_rank, (int)f_page);
        for (int p = ks + lane; p < top_k; p += 64) {
          sel[p] = -1;
          if (selp) selp[p] = -1;
        }
      }
      return;
    }
    if (wave != 0) return;
    // wave 0 alone: should the appending workgroup have come and gone (its
    // bit is in the word), finish here without handing the partial
    // selection over; else hand it over and meet
    unsigned long long met = __hip_atomic_load(a.meet + pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (!(met >> 63)) {
      if (lane < ks) __hip_atomic_store(ppages + f_rank, (int)f_page, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) {
        __hip_atomic_store(pkeys, f_whi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(pkeys + 1, f_wlo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the hand-over is complete
      unsigned long long old = 0ull;
      if (lane == 0) old = __hip_atomic_fetch_or(a.meet + pair, 1ull << 62, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      met = (unsigned long long)(uint32_t)__builtin_amdgcn_readfirstlane((int)(old >> 32)) << 32 |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)old);
    }
    if (met) {
      if (lane == 0) __hip_atomic_store(a.meet + pair, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      merge_fast((uint32_t)met, (int)f_page, (int)f_rank);
    }
    return;
  }
  const bool keep_local = top_k <= 1024;
  auto emit = [&](int p, int j) {
    if (split) {
      __hip_atomic_store(ppages + p, j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(pkeys + p, s_keys[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (keep_local) {
        s_Sp[p] = j;
        s_Sk[p] = s_keys[j];
      }
    } else {
      put(p, j);
    }
  };
  if (!split) {
    for (int p = ks + tid; p < top_k; p += RT) {
      sel[p] = -1;
      if (selp) selp[p] = -1;
    }
    if (tid == 0) a.n_sel[pair] = ks;
  }
  if (ks > 0) select(npg, ks, emit);
  if (split) {
    const unsigned long long met = meet(1ull << 62);
    if (met) merge_appended(keep_local, (uint32_t)met);
  }
}

size_t route_lds_bytes(const Shape& s, bool append) {
  return route_lds(s.max_pages, s.head_dim, s.rank_v, s.rank_k, s.group, s.page_size, s.dtype == 0 ? 4 : 2, append)
      .total;
}

template <typename T, bool APPEND, int D, int NG, bool FORCE, bool MEAN>
hipError_t launch_f(const RouteArgs& a, hipStream_t st) {
  const size_t lds = route_lds_bytes(a.s, APPEND);
  const hipError_t e = allow_lds((const void*)route_kernel<T, APPEND, D, NG, FORCE, MEAN>, lds);
  if (e != hipSuccess) return e;
  const int cl = route_cluster(a.s, APPEND, a.arrive != nullptr);
  hipLaunchKernelGGL((route_kernel<T, APPEND, D, NG, FORCE, MEAN>), dim3(a.s.batch * a.s.n_kv_heads * cl), dim3(RT),
                     lds, st, a);
  return hipGetLastError();
}

template <typename T, bool APPEND, int D, int NG>
hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  const bool force = a.sink_pages > 0 || a.local_pages > 0;
  if (a.group_mean) {
    if (force) return launch_f<T, APPEND, D, NG, true, true>(a, st);
    return launch_f<T, APPEND, D, NG, false, true>(a, st);
  }
  if (force) return launch_f<T, APPEND, D, NG, true, false>(a, st);
  return launch_f<T, APPEND, D, NG, false, false>(a, st);
}

template <typename T, bool APPEND, int D>
hipError_t launch_g(const RouteArgs& a, hipStream_t st) {
  const int ng = (a.s.rank_v + a.s.rank_k + 15) / 16;
  if (ng <= 2) return launch_t<T, APPEND, D, 2>(a, st);
  if (ng == 3) return launch_t<T, APPEND, D, 3>(a, st);
  return launch_t<T, APPEND, D, 4>(a, st);  // also wide rows, which do not use it
}

template <typename T, bool APPEND>
hipError_t launch_d(const RouteArgs& a, hipStream_t st) {
  return a.s.head_dim == 64 ? launch_g<T, APPEND, 64>(a, st) : launch_g<T, APPEND, 128>(a, st);
}

}  // namespace

}  // namespace bkv
