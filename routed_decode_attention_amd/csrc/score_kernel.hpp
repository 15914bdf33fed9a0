// Page scores for Key routing, predicted from the Value latents plus the Key
// residual; optionally fused with the decode-step append of the new token.
//
// weekinpapers "BasisKV: Value Latents for Communication and Key Routing",
// Abstract: the compressed Value cache predicts part of the Key information
// needed for routing and a Key-specific residual stores the rest; kongchang
// article, section on Value-latent Key routing (cheap coarse routing, exact
// scoring afterwards).  With the predicted Key k~_t = z~_t.P + s~_t.R_dec the
// score of page j for query head h is scale * q_h . mean_t k~_t, which by
// linearity is scale * ((P.q_h) . sumz_j + (R_dec.q_h) . sums_j) / cnt_j.
// A page's group score is the max over the KV head's query heads (their mean
// with group_mean); with per-query-head selection every head keeps its own.  Decode appends the new token before attending
// (machinelearning.ru "KV-кэширование", "Фаза Decode"), so the appended page
// is scored from its sums after the write.
//
// Each (sequence, KV head) gets a cluster of 256-thread workgroups that never
// wait for one another: with an append, workgroup 0 writes the new token
// (wave 0) while waves 1-3 project the query, then scores the appended page;
// the others each score up to `per` pages (every page but the appended one).
// The top-k selection reads the scores afterwards (the attention kernel's
// prologue, or the selection kernel).  A scoring workgroup is two memory round
// trips: (1) P, R_dec and the query copied straight into LDS beside its
// pages' page-table entries; (2) the pages' fp32 sums, four lanes per page,
// in flight while the waves project the query.
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int SC_T = 256;
constexpr int SC_NW = SC_T / 64;
constexpr int SC_VMAX = 64;                       // page-sum channels held in registers (quad path)
constexpr int SC_XMAX = MAX_RANK + MAX_RESID;     // projected-query width bound
constexpr int SC_PPL = 4;                         // pages per quad: up to 256 pages per workgroup

// Sum over the four lanes of a quad (every lane gets the total).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lanes ^1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lanes ^2
  return x;
}

// Four consecutive storage-dtype elements from LDS as fp32.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// How a unit's page score combines the group's query heads: the max, the
// mean, or every head its own score (per-query-head selection).
enum { AGG_MAX = 0, AGG_MEAN = 1, AGG_HEAD = 2 };

// d[i] = qh . sums(page i), each dot split over the four lanes of a quad (NG
// 16-byte channel granules per lane: granule part + 4u) and summed by the quad.
template <int NG, int PPL>
__device__ __forceinline__ void head_dots(const f32x4 (&sv)[PPL][NG], const float* qh, int part, float (&d)[PPL]) {
  f32x4 qg[NG];
#pragma unroll
  for (int u = 0; u < NG; ++u) qg[u] = *reinterpret_cast<const f32x4*>(&qh[4 * (part + 4 * u)]);
#pragma unroll
  for (int i = 0; i < PPL; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < NG; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = fmaf(qg[u][e], sv[i][u][e], acc);
    d[i] = quad_sum(acc);
  }
}

// best[i] = max (AGG_MEAN: mean) over the group's heads h of qc[h] . sums(page i).
template <int NG, int PPL, int AGG>
__device__ __forceinline__ void score_group(const f32x4 (&sv)[PPL][NG], const float (*qc)[SC_XMAX], int G, int part,
                                            float (&best)[PPL]) {
#pragma unroll
  for (int i = 0; i < PPL; ++i) best[i] = AGG == AGG_MEAN ? 0.f : -__builtin_huge_valf();
  for (int h = 0; h < G; ++h) {
    float d[PPL];
    head_dots<NG, PPL>(sv, qc[h], part, d);
#pragma unroll
    for (int i = 0; i < PPL; ++i) best[i] = AGG == AGG_MEAN ? best[i] + d[i] : fmaxf(best[i], d[i]);
  }
  if constexpr (AGG == AGG_MEAN)
#pragma unroll
    for (int i = 0; i < PPL; ++i) best[i] /= (float)G;
}

// Dynamic LDS layout (bytes, every part 16-byte aligned): P and R_dec
// rotated, the group's queries; for the appending workgroup also B, R_enc,
// the new token (v then k) and the appended page's image (Z then S).
struct ScoreLds {
  size_t P, Rd, q, B, Re, vk, img, total;
};
__host__ __device__ inline size_t sc_a16(size_t x) { return (x + 15) & ~(size_t)15; }
__host__ __device__ inline ScoreLds score_lds(int D, int R, int RK, int G, int ps, int es, bool append) {
  ScoreLds L;
  L.P = 0;
  L.Rd = L.P + (size_t)R * D * 4;
  L.q = L.Rd + (size_t)RK * D * 4;
  L.B = L.q + sc_a16((size_t)G * D * es);
  L.Re = L.B + (append ? (size_t)D * R * 4 : 0);
  L.vk = L.Re + (append ? (size_t)D * RK * 4 : 0);
  L.img = L.vk + (append ? sc_a16((size_t)2 * D * es) : 0);
  L.total = L.img + (append ? sc_a16((size_t)(R * ps + ps * RK) * es) : 0);
  return L;
}

// The query seen through P and R_dec, times the softmax scale, on the matrix
// cores (fp32 products, v_mfma_f32_16x16x4f32): the rows of P and R_dec (r + r_k, in 16-row tiles) times the group's
// queries (up to 16 heads as the columns).  Waves wave0, wave0 + nwaves, ...
// take a tile each; lane (n, qd) supplies row 16 t + n and head n over dims
// 32 qd + s at step s (the contraction's order permuted so that each lane
// reads 32 consecutive values), two accumulators for the even and odd steps.
// qc[h][x] = scale * (P.q_h | R_dec.q_h)[x]; outputs past r + r_k (up to
// SC_VMAX) are zero (the threads of waves >= wave0 write them).
template <typename T, int D>
__device__ __forceinline__ void project_query(const float* sP, const float* sRd, const T* sq,
                                                   float (*qc)[SC_XMAX], int R, int RK, int G, float scale, int wave0,
                                                   int nwaves, int wave, int lane) {
  static_assert(D == 128 || D == 64, "head_dim");
  constexpr int KQ = D / 4;  // dims per lane group
  const int RR = R + RK, n = lane & 15, qd = lane >> 4;
  // this lane's head: its KQ consecutive query values as fp32
  float qv[KQ];
  {
    const T* qh = sq + min(n, G - 1) * D + KQ * qd;
#pragma unroll
    for (int u = 0; u < KQ / 4; ++u) {
      const f32x4 q4 = lds4(qh + 4 * u);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * u + e] = n < G ? q4[e] : 0.f;
    }
  }
  for (int t = wave - wave0; 16 * t < RR; t += nwaves) {
    const int x = min(16 * t + n, RR - 1);
    const int xr = x < R ? x : x - R;
    const float* row = (x < R ? sP : sRd) + xr * D;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KQ / 4; ++u) {
      // granule KQ/4 qd + u of the row, rotated by the row in LDS
      const f32x4 p4 = lds4(row + rot_granule(xr, (KQ / 4) * qd + u, D) * 4);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[0], qv[4 * u], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[1], qv[4 * u + 1], acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[2], qv[4 * u + 2], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(p4[3], qv[4 * u + 3], acc1, 0, 0, 0);
    }
    // lane (n, qd) holds rows 16 t + 4 qd + i of head n
    if (n < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int xo = 16 * t + 4 * qd + i;
        if (xo < RR) qc[n][xo] = (acc0[i] + acc1[i]) * scale;
      }
    }
  }
  if (RR < SC_VMAX) {
    const int t0 = (wave - wave0) * 64 + lane, stride = nwaves * 64;
    for (int t = t0; t < G * (SC_VMAX - RR); t += stride) qc[t / (SC_VMAX - RR)][RR + t % (SC_VMAX - RR)] = 0.f;
  }
}

// NG: 16-byte channel granules per scoring lane, ceil((r + r_k) / 16); 0 for
// wide page sums (r + r_k > 64), scored by a plain per-thread path; AGG: how
// the query heads' scores combine (AGG_HEAD: scores [b][query head][page]).
template <typename T, bool APPEND, int D, int NG, int AGG>
__global__ __launch_bounds__(SC_T) void score_kernel(ScoreArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  __shared__ __attribute__((aligned(16))) float s_qc[MAX_GROUP][SC_XMAX];
  __shared__ __attribute__((aligned(16))) float s_st[SC_XMAX];    // the appended token's stored values
  __shared__ __attribute__((aligned(16))) float s_e[128];          // its Key remainder
  __shared__ __attribute__((aligned(16))) float s_newsum[SC_XMAX]; // its page's new sums
  __shared__ __attribute__((aligned(16))) float s_pre[SC_XMAX];    // the sums of its page's earlier slots
  __shared__ __attribute__((aligned(16))) float s_parts[TP * (64 + 128 + 64)];  // its products' parts

  const int H = a.s.n_kv_heads, G = a.s.group, C = a.cluster;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = L / C, c = L - pair * C;
  const int b = pair / H, g = pair % H;
  const int R = a.s.rank_v, RK = a.s.rank_k, RR = R + RK, ps = a.s.page_size, maxp = a.s.max_pages;
  const int tid = threadIdx.x, wave = uniform(tid >> 6), lane = tid & 63;
  const int n = load_uniform(a.seq_lens, b);
  const int npg = n > 0 ? min((n + ps - 1) / ps, maxp) : 0;
  int pos = -1;
  if (APPEND) {
    pos = load_uniform(a.pos, b);
    if (pos < 0 || pos >= maxp * ps) pos = -1;
  }
  const int apage = pos >= 0 ? pos / ps : -1;
  const bool appender = APPEND && c == 0;
  const int32_t* pt = a.page_table + (size_t)b * maxp;
  char* base = reinterpret_cast<char*>(lds);
  const ScoreLds lay = score_lds(D, R, RK, G, ps, (int)sizeof(T), APPEND);
  float* sP = reinterpret_cast<float*>(base + lay.P);    // [R][D] rotated
  float* sRd = reinterpret_cast<float*>(base + lay.Rd);  // [RK][D] rotated
  T* sq = reinterpret_cast<T*>(base + lay.q);            // [G][D]
  // scores of the unit(s): [pair][page], or with AGG_HEAD [pair][head][page]
  float* out = a.scores + (size_t)pair * (AGG == AGG_HEAD ? G : 1) * maxp;

  // pages [lo, hi) of a scoring workgroup (the appender scores only its page)
  const int sidx = APPEND ? c - 1 : c;
  const int lo = appender ? 0 : min(npg, sidx * a.per), hi = appender ? 0 : min(npg, lo + a.per);
  if (appender ? pos < 0 : lo >= hi) return;  // the whole workgroup

  // ---- round trip 1: factors and queries straight into LDS (and for the
  // appender its factors, the token and, once its page is known, the page
  // image); scorers load their pages' page-table entries ----
  {
    const char* P = reinterpret_cast<const char*>(a.P + (size_t)g * R * D);
    const char* Rd = reinterpret_cast<const char*>(a.R_dec + (size_t)g * RK * D);
    const char* q = reinterpret_cast<const char*>(static_cast<const T*>(a.q) + ((size_t)b * a.s.n_q_heads + g * G) * D);
    // the appender's wave 0 copies nothing: it requests the appended page's
    // image into its registers instead and so never waits for the copies
    // (vmcnt counts a wave's loads in issue order)
    const int cw = appender ? SC_NW - 1 : SC_NW, cwave = appender ? wave - 1 : wave;
    if (cwave >= 0) {
      int first = dma_stage(sP, R * D / 4, [&](int G_) { return P + 16 * rot_source(G_, D); }, 0, cw, cwave, lane);
      first = dma_stage(sRd, RK * D / 4, [&](int G_) { return Rd + 16 * rot_source(G_, D); }, first, cw, cwave, lane);
      first = dma_stage(sq, (int)(G * D * sizeof(T) / 16), [&](int G_) { return q + 16 * G_; }, first, cw, cwave,
                        lane);
      if (appender) {
        const char* B = reinterpret_cast<const char*>(a.B + (size_t)g * D * R);
        const char* Re = reinterpret_cast<const char*>(a.R_enc + (size_t)g * D * RK);
        const size_t tok = ((size_t)b * H + g) * D;
        const char* vn = reinterpret_cast<const char*>(static_cast<const T*>(a.v_new) + tok);
        const char* kn = reinterpret_cast<const char*>(static_cast<const T*>(a.k_new) + tok);
        const int tc = (int)(D * sizeof(T) / 16);
        first = dma_stage(base + lay.B, D * R / 4, [&](int G_) { return B + 16 * G_; }, first, cw, cwave, lane);
        first = dma_stage(base + lay.Re, D * RK / 4, [&](int G_) { return Re + 16 * G_; }, first, cw, cwave, lane);
        dma_stage(base + lay.vk, 2 * tc, [&](int G_) { return G_ < tc ? vn + 16 * G_ : kn + 16 * (G_ - tc); },
                  first, cw, cwave, lane);
      }
    }
  }

  if (appender) {
    // wave 0 requests the appended page's stored latents and residuals into
    // registers while waves 1-3's copies land; they wait for their copies
    const int aphys = load_uniform(pt, apage);
    const int slot = pos - apage * ps;
    T* Zp = static_cast<T*>(a.Z) + ((size_t)aphys * H + g) * R * ps;
    T* Sp = static_cast<T*>(a.S) + ((size_t)aphys * H + g) * ps * RK;
    // (bf16: the operands of the page's sums themselves, in the layout the
    // sums' products take, so the sums need no LDS copy of the page; fp32:
    // the raw image, summed through LDS)
    constexpr bool BF16 = sizeof(T) == 2;
    PageImage pg;
    PageSumRegs pr;
    if (wave == 0) {
      if constexpr (BF16) {
        pr.load(reinterpret_cast<const uint16_t*>(Zp), reinterpret_cast<const uint16_t*>(Sp), R, RK, ps, lane);
        // the page arrives before waves 1-3's copies: the sums of the slots
        // before the token are taken meanwhile (the token's own values are
        // added once it exists: wave_page_sums' order)
        wait_vmem();
        pr.prefix(R, RK, ps, slot, s_pre, lane);
      } else {
        pg.load(Zp, Sp, (int)(R * ps * sizeof(T) / 16), (int)(ps * RK * sizeof(T) / 16), lane);
      }
    } else {
      wait_vmem();
    }
    lds_barrier();
    const T* vn = reinterpret_cast<const T*>(base + lay.vk);
    const T* kn = vn + D;
    T* img = reinterpret_cast<T*>(base + lay.img);
    // the token's three products, each split over the four waves (wave w
    // takes part w); each wave finishes the rows its next part needs
    const TokenLds<T> Lt{vn, kn, reinterpret_cast<const float*>(base + lay.B), sP,
                         reinterpret_cast<const float*>(base + lay.Re), s_e, s_st,
                         s_parts, s_parts + TP * 64, s_parts + TP * 192};
    token_latent_part<T, D>(Lt, R, wave, lane);
    lds_barrier();
    token_latent_finish(Lt, wave * (R / TP), R / TP, lane);
    wave_sync();
    token_keyest_part<T, D>(Lt, R, wave, lane);
    lds_barrier();
    token_remainder_finish(Lt, wave * (D / TP), D / (4 * TP), lane);
    wave_sync();
    token_residual_part<T, D>(Lt, RK, wave, lane);
    lds_barrier();
    if (wave == 0) {
      token_residual_finish(Lt, R, RK, lane);
      // (fp32) the page image, long since in: waiting for it here, before
      // the token's stores, keeps its use below from waiting for the stores
      // (vmcnt counts both in issue order); bf16 waited for it above
      wait_vmem();
      wave_sync();
      // the token's stores first: they complete while the sums are formed
      T* Kp = static_cast<T*>(a.K) + ((size_t)aphys * H + g) * ps * D;
      wave_token_store<T, D>(Lt, R, RK, ps, slot, Kp + (size_t)slot * D, Zp, Sp, lane);
      if constexpr (BF16) {
        for (int x = lane; x < RR; x += 64) s_newsum[x] = s_pre[x] + s_st[x];
      } else {
        pg.store(img, lane);
        wave_sync();
        for (int x = lane; x < RR; x += 64) {
          if (x < R) store_elem(img, (size_t)x * ps + slot, s_st[x]);
          else store_elem(img, (size_t)R * ps + (size_t)slot * RK + (x - R), s_st[x]);
        }
        wave_sync();
        wave_page_sums(img, img + (size_t)R * ps, R, RK, ps, slot + 1, s_newsum, lane);
      }
    } else {
      project_query<T, D>(sP, sRd, sq, s_qc, R, RK, G, a.s.scale, 1, SC_NW - 1, wave, lane);
    }
    lds_barrier();
    if (wave == 0) {
      // the page's sums, then (quad 0) the page's score
      for (int x = lane; x < RR; x += 64) a.summ[((size_t)aphys * H + g) * RR + x] = s_newsum[x];
      if (apage < npg) {
        const float cnt = (float)min(ps, n - apage * ps);
        float best = AGG == AGG_MEAN ? 0.f : -__builtin_huge_valf();
        if constexpr (NG > 0) {
          const int part = lane & 3;
          f32x4 sv[1][NG];
#pragma unroll
          for (int u = 0; u < NG; ++u) {
            const int gr = part + 4 * u;
            sv[0][u] = 4 * gr < RR ? *reinterpret_cast<const f32x4*>(s_newsum + 4 * gr) : f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if constexpr (AGG == AGG_HEAD) {
            for (int h = 0; h < G; ++h) {
              float d[1];
              head_dots<NG, 1>(sv, s_qc[h], part, d);
              if (lane == 0) out[(size_t)h * maxp + apage] = d[0] / cnt;
            }
          } else {
            float bst[1];
            score_group<NG, 1, AGG>(sv, s_qc, G, part, bst);
            best = bst[0];
          }
        } else if (lane == 0) {
          for (int h = 0; h < G; ++h) {
            float d = 0.f;
            for (int x = 0; x < RR; ++x) d = fmaf(s_qc[h][x], s_newsum[x], d);
            if constexpr (AGG == AGG_HEAD) out[(size_t)h * maxp + apage] = d / cnt;
            best = AGG == AGG_MEAN ? best + d : fmaxf(best, d);
          }
          if constexpr (AGG == AGG_MEAN) best /= (float)G;
        }
        if (AGG != AGG_HEAD && lane == 0) out[apage] = best / cnt;
      }
    }
    return;
  }

  // ---- scorer.  Quad q (64 per workgroup) takes pages lo + q + 64 i ----
  const int quad = tid >> 2, part = tid & 3;
  int phys[SC_PPL];
#pragma unroll
  for (int i = 0; i < SC_PPL; ++i) {
    const int j = lo + quad + 64 * i;
    phys[i] = j < hi ? pt[j] : 0;
  }
  wait_vmem();  // this wave's direct copies and page-table loads are in
  if constexpr (NG > 0) {
    // ---- round trip 2: the page sums, requested before the query
    // projection so that they are in flight while it runs.  Unconditional
    // loads (a granule past the row re-reads its last one), masked below ----
    f32x4 sv[SC_PPL][NG];
#pragma unroll
    for (int i = 0; i < SC_PPL; ++i) {
      const f32x4* row = reinterpret_cast<const f32x4*>(a.summ + ((size_t)phys[i] * H + g) * RR);
#pragma unroll
      for (int u = 0; u < NG; ++u) sv[i][u] = row[min(part + 4 * u, RR / 4 - 1)];
    }
    lds_barrier();  // every wave's direct copies are complete (waited above); the sums stay in flight
    project_query<T, D>(sP, sRd, sq, s_qc, R, RK, G, a.s.scale, 0, SC_NW, wave, lane);
    lds_barrier();
#pragma unroll
    for (int i = 0; i < SC_PPL; ++i)
#pragma unroll
      for (int u = 0; u < NG; ++u)
        if (4 * (part + 4 * u) >= RR) sv[i][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (AGG == AGG_HEAD) {
      for (int h = 0; h < G; ++h) {
        float d[SC_PPL];
        head_dots<NG, SC_PPL>(sv, s_qc[h], part, d);
#pragma unroll
        for (int i = 0; i < SC_PPL; ++i) {
          const int j = lo + quad + 64 * i;
          if (part == 0 && j < hi && j != apage) out[(size_t)h * maxp + j] = d[i] / (float)min(ps, n - j * ps);
        }
      }
    } else {
      float best[SC_PPL];
      score_group<NG, SC_PPL, AGG>(sv, s_qc, G, part, best);
#pragma unroll
      for (int i = 0; i < SC_PPL; ++i) {
        const int j = lo + quad + 64 * i;
        if (part == 0 && j < hi && j != apage) out[j] = best[i] / (float)min(ps, n - j * ps);
      }
    }
  } else {
    // wide sums (r + r_k > 64): a thread per page, 64 channels at a time
    lds_barrier();
    project_query<T, D>(sP, sRd, sq, s_qc, R, RK, G, a.s.scale, 0, SC_NW, wave, lane);
    lds_barrier();
    float d[MAX_GROUP];
    for (int j = lo + tid; j < hi; j += SC_T) {
      if (j == apage) continue;
      const float* sm = a.summ + ((size_t)pt[j] * H + g) * RR;
#pragma unroll
      for (int h = 0; h < MAX_GROUP; ++h) d[h] = 0.f;
      for (int x0 = 0; x0 < RR; x0 += SC_VMAX) {
        float v[SC_VMAX];
#pragma unroll
        for (int u = 0; u < SC_VMAX / 4; ++u) {
          float4 t4 = {0.f, 0.f, 0.f, 0.f};
          if (x0 + 4 * u < RR) t4 = *reinterpret_cast<const float4*>(sm + x0 + 4 * u);
          v[4 * u] = t4.x;
          v[4 * u + 1] = t4.y;
          v[4 * u + 2] = t4.z;
          v[4 * u + 3] = t4.w;
        }
#pragma unroll
        for (int h = 0; h < MAX_GROUP; ++h)
          if (h < G) {
#pragma unroll
            for (int x = 0; x < SC_VMAX; ++x)
              if (x0 + x < RR) d[h] = fmaf(s_qc[h][x0 + x], v[x], d[h]);
          }
      }
      const float cnt = (float)min(ps, n - j * ps);
      if constexpr (AGG == AGG_HEAD) {
#pragma unroll
        for (int h = 0; h < MAX_GROUP; ++h)
          if (h < G) out[(size_t)h * maxp + j] = d[h] / cnt;
      } else {
        float best = AGG == AGG_MEAN ? 0.f : -__builtin_huge_valf();
#pragma unroll
        for (int h = 0; h < MAX_GROUP; ++h)
          if (h < G) best = AGG == AGG_MEAN ? best + d[h] : fmaxf(best, d[h]);
        if constexpr (AGG == AGG_MEAN) best /= (float)G;
        out[j] = best / cnt;
      }
    }
  }
}

template <typename T, bool APPEND, int D, int NG, int AGG>
hipError_t launch_sc(const ScoreArgs& a, hipStream_t st) {
  const size_t lds = score_lds(a.s.head_dim, a.s.rank_v, a.s.rank_k, a.s.group, a.s.page_size,
                               (int)sizeof(T), APPEND).total;
  const hipError_t e = allow_lds((const void*)score_kernel<T, APPEND, D, NG, AGG>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((score_kernel<T, APPEND, D, NG, AGG>), dim3(a.s.batch * a.s.n_kv_heads * a.cluster),
                     dim3(SC_T), lds, st, a);
  return hipGetLastError();
}

template <typename T, bool APPEND, int D, int AGG>
hipError_t launch_sc_n(const ScoreArgs& a, hipStream_t st) {
  const int rr = a.s.rank_v + a.s.rank_k;
  const int ng = (rr + 15) / 16;
  if (rr > SC_VMAX) return launch_sc<T, APPEND, D, 0, AGG>(a, st);  // wide page sums
  if (ng <= 2) return launch_sc<T, APPEND, D, 2, AGG>(a, st);
  if (ng == 3) return launch_sc<T, APPEND, D, 3, AGG>(a, st);
  return launch_sc<T, APPEND, D, 4, AGG>(a, st);
}

template <typename T, bool APPEND, int D>
hipError_t launch_sc_g(const ScoreArgs& a, hipStream_t st) {
  if (a.s.head_select) return launch_sc_n<T, APPEND, D, AGG_HEAD>(a, st);
  return a.group_mean ? launch_sc_n<T, APPEND, D, AGG_MEAN>(a, st) : launch_sc_n<T, APPEND, D, AGG_MAX>(a, st);
}

template <typename T>
hipError_t launch_score_t(const ScoreArgs& a, hipStream_t st) {
  const bool app = a.pos != nullptr;
  if (a.s.head_dim == 64) return app ? launch_sc_g<T, true, 64>(a, st) : launch_sc_g<T, false, 64>(a, st);
  return app ? launch_sc_g<T, true, 128>(a, st) : launch_sc_g<T, false, 128>(a, st);
}

}  // namespace

}  // namespace bkv
