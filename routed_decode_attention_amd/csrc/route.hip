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
// One 512-thread workgroup per (sequence, KV head), no cross-workgroup
// traffic.  The kernel is a short chain of memory round trips, and its
// serial parts are kept to few instructions:
//   1. the page-table row, the factors, the query and the new token are
//      copied straight into LDS together (16-byte direct loads);
//   2. every lane requests the sums of its first page; meanwhile wave 0
//      appends the new token (the writer's wave functions, then the page's
//      sums from scratch over its LDS image) and the other waves project
//      the query through P and R_dec, four lanes per output;
//   3. one lane scores one page from its fp32 sums held in registers;
//   4. an MSB-first 8-bit radix select over order-preserving keys in LDS
//      (per-wave histograms merged once per pass) finds the k-th score, and
//      ballots plus per-wave counts compact the selection in page order.
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

// Four consecutive storage-dtype elements from LDS as fp32.
__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// Dynamic LDS layout (bytes, every part 16-byte aligned).
struct RouteLds {
  size_t pid, P, Rd, q, B, Re, vk, img, total;
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
  // the score keys reuse the space from P on
  if (L.total < L.P + (size_t)maxp * 4) L.total = L.P + (size_t)maxp * 4;
  return L;
}

template <typename T, bool APPEND, int D>
__global__ __launch_bounds__(RT) void route_kernel(RouteArgs a) {
  extern __shared__ float lds[];
  __shared__ float s_qc[MAX_GROUP][XMAX];   // scale * (P.q_h | R_dec.q_h), zero past r + r_k
  __shared__ float s_tok[4][128];           // appended token: v, k, Key remainder; stored values
  __shared__ float s_newsum[XMAX];          // the appended page's sums

  const int pair = blockIdx.x;
  const int H = a.s.n_kv_heads, G = a.s.group;
  const int R = a.s.rank_v, RK = a.s.rank_k, RR = R + RK, ps = a.s.page_size;
  const int maxp = a.s.max_pages;
  const int b = pair / H, g = pair % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int32_t* pt = a.page_table + (size_t)b * maxp;
  char* base = reinterpret_cast<char*>(lds);
  const RouteLds lay = route_lds(maxp, D, R, RK, G, ps, (int)sizeof(T), APPEND);
  int32_t* s_pid = reinterpret_cast<int32_t*>(base + lay.pid);  // [maxp] the page-table row
  float* sP = reinterpret_cast<float*>(base + lay.P);            // [R][D] rotated
  float* sRd = reinterpret_cast<float*>(base + lay.Rd);          // [RK][D] rotated
  T* sq = reinterpret_cast<T*>(base + lay.q);                    // [G][D] the group's query heads
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(sP);            // [maxp], once the projections are done

  // ---- round trip 1: page-table row, sequence length, append position,
  // factors, query and new token, all requested together ----
  const int pid0 = tid < maxp ? pt[tid] : 0;  // this lane's first page, for its sums below
  const int n = a.seq_lens[b];
  int pos = -1;
  if (APPEND) {
    pos = a.pos[b];
    if (pos < 0 || pos >= maxp * ps) pos = -1;
  }
  const bool app = APPEND && pos >= 0;
  const int apage = app ? pos / ps : 0, slot = app ? pos % ps : 0;
  const int npg = n > 0 ? min((n + ps - 1) / ps, maxp) : 0;
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
    if (app) {
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

  // ---- round trip 2: this lane's first page sums (lane j scores page j)
  float v[VMAX];
  auto load_row = [&](float (&dst)[VMAX], int phys) {
    const float* sm = a.summ + ((size_t)phys * H + g) * RR;
#pragma unroll
    for (int u = 0; u < VMAX / 4; ++u) {
      float4 t4 = {0.f, 0.f, 0.f, 0.f};
      if (4 * u < RR) t4 = *reinterpret_cast<const float4*>(sm + 4 * u);
      dst[4 * u] = t4.x;
      dst[4 * u + 1] = t4.y;
      dst[4 * u + 2] = t4.z;
      dst[4 * u + 3] = t4.w;
    }
  };
  if (in_regs && tid < npg) load_row(v, pid0);

  if (app && wave == 0) {
    // ---- the new token (wave 0): exact Key, rounded latent and residual,
    // then its page's sums from scratch over slots [0, slot] ----
    const int aphys = s_pid[apage];
    T* Kp = static_cast<T*>(a.K) + ((size_t)aphys * H + g) * ps * D;
    T* Zp = static_cast<T*>(a.Z) + ((size_t)aphys * H + g) * R * ps;
    T* Sp = static_cast<T*>(a.S) + ((size_t)aphys * H + g) * ps * RK;
    T* img = reinterpret_cast<T*>(base + lay.img);
    PageImage pg;
    pg.load(Zp, Sp, (int)(R * ps * sizeof(T) / 16), (int)(ps * RK * sizeof(T) / 16), lane);
    const T* vk = reinterpret_cast<const T*>(base + lay.vk);
#pragma unroll
    for (int i = lane; i < D; i += 64) {
      s_tok[0][i] = ld_elem(vk, i);
      s_tok[1][i] = ld_elem(vk, D + i);
    }
    wave_sync();
    const TokenLds L{s_tok[0], s_tok[1], reinterpret_cast<const float*>(base + lay.B), sP,
                     reinterpret_cast<const float*>(base + lay.Re), s_tok[2], s_tok[3]};
    wave_write_token<T, D>(L, R, RK, ps, slot, Kp + (size_t)slot * D, Zp, Sp, lane);
    pg.store(img, lane);
    wave_sync();
    // the new token's values replace what the page held in its slot
    for (int x = lane; x < RR; x += 64) {
      if (x < R) store_elem(img, (size_t)x * ps + slot, L.st[x]);
      else store_elem(img, (size_t)R * ps + (size_t)slot * RK + (x - R), L.st[x]);
    }
    wave_sync();
    wave_page_sums(img, img + (size_t)R * ps, R, RK, ps, slot + 1, s_newsum, lane);
    wave_sync();
    for (int x = lane; x < RR; x += 64) a.summ[((size_t)aphys * H + g) * RR + x] = s_newsum[x];
  } else {
    // ---- the query seen through the latent predictor P and the residual
    // decoder R_dec: four lanes per output, lane c taking 16-byte pieces
    // 4u + c of the rows; outputs past r + r_k (up to VMAX) are zero ----
    const int q0 = app ? 64 : 0;
    const int XP = RR > VMAX ? RR : VMAX;
    for (int t = tid - q0; t < G * XP * 4; t += RT - q0) {
      const int o = t >> 2, c = t & 3;
      const int h = o / XP, x = o % XP;
      float acc = 0.f;
      if (x < RR) {
        const int xr = x < R ? x : x - R;
        const float* row = (x < R ? sP : sRd) + xr * D;
        const T* qh = sq + h * D;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
          const f32x4 p4 = lds4(row + rot_granule(xr, 4 * u + c, D) * 4);
          const f32x4 q4 = lds4(qh + 16 * u + 4 * c);
          acc = fmaf(p4[0], q4[0], acc);
          acc = fmaf(p4[1], q4[1], acc);
          acc = fmaf(p4[2], q4[2], acc);
          acc = fmaf(p4[3], q4[3], acc);
        }
      }
      acc = quad_sum(acc);
      if (c == 0) s_qc[h][x] = acc * a.s.scale;
    }
  }
  __syncthreads();

  // ---- one lane per page: score from the page's fp32 sums ----
  auto finish = [&](int j, float best) {
    const float sc = best / (float)min(ps, n - j * ps);
    a.scores[(size_t)pair * maxp + j] = sc;
    s_keys[j] = float_key(sc);
  };
  if (in_regs) {
    // max over the group's heads of (q_h seen through P | R_dec) . sums, over
    // VMAX channels (both zero past r + r_k)
    auto score_row = [&](const float (&vv)[VMAX]) {
      float best = -__builtin_huge_valf();
      for (int h = 0; h < G; ++h) {
        const f32x4* qc = reinterpret_cast<const f32x4*>(s_qc[h]);
        float acc = 0.f;
#pragma unroll
        for (int u = 0; u < VMAX / 4; ++u) {
          const f32x4 c4 = qc[u];
          acc = fmaf(c4[0], vv[4 * u], acc);
          acc = fmaf(c4[1], vv[4 * u + 1], acc);
          acc = fmaf(c4[2], vv[4 * u + 2], acc);
          acc = fmaf(c4[3], vv[4 * u + 3], acc);
        }
        best = fmaxf(best, acc);
      }
      return best;
    };
    // lanes with several pages request the next page's sums before scoring
    // the current one
    float w[VMAX];
    for (int j = tid; j < npg; j += RT) {
      if (j + RT < npg) load_row(w, s_pid[j + RT]);
      if (app && j == apage) {
#pragma unroll
        for (int x = 0; x < VMAX; ++x) v[x] = x < RR ? s_newsum[x] : 0.f;
      }
      finish(j, score_row(v));
#pragma unroll
      for (int x = 0; x < VMAX; ++x) v[x] = w[x];
    }
  } else {
    // wide sums (r + r_k > 64): 64 channels at a time, every head's dot kept
    float d[MAX_GROUP];
    for (int j = tid; j < npg; j += RT) {
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
        if (app && j == apage) {
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
      float best = -__builtin_huge_valf();
#pragma unroll
      for (int h = 0; h < MAX_GROUP; ++h)
        if (h < G) best = fmaxf(best, d[h]);
      finish(j, best);
    }
  }
  __syncthreads();

  // ---- top-k selection: per-wave histograms, one merge per radix pass ----
  __shared__ int s_whist[NW][256];
  __shared__ int s_tot[256];
  __shared__ int s_wcnt[NW][2];
  __shared__ int s_digit, s_krem;
  const int k = min(a.s.top_k, npg);
  int32_t* sel = a.sel + (size_t)pair * a.s.top_k;
  int32_t* selp = a.sel_phys ? a.sel_phys + (size_t)pair * a.s.top_k : nullptr;
  for (int p = k + tid; p < a.s.top_k; p += RT) {
    sel[p] = -1;
    if (selp) selp[p] = -1;
  }
  if (tid == 0) a.n_sel[pair] = k;
  if (k == 0) return;

  uint32_t thr = 0;
  int take_eq = 0;
  const bool all = k == npg;
  if (!all) {
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) s_whist[wave][lane + 64 * u] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int j = tid; j < npg; j += RT) {
        const uint32_t key = s_keys[j];
        if ((key & mask) == prefix) atomicAdd(&s_whist[wave][(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 256) {
        int t = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) t += s_whist[w][tid];
        s_tot[tid] = t;
      }
      __syncthreads();
      if (wave == 0) {
        // lane owns digits 255-4*lane .. 252-4*lane (descending)
        int c[4], own = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          c[u] = s_tot[255 - 4 * lane - u];
          own += c[u];
        }
        int run = wave_incl_scan(own) - own;  // keys with a larger digit than this lane's
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (run < krem && run + c[u] >= krem) {
            s_digit = 255 - 4 * lane - u;
            s_krem = krem - run;
          }
          run += c[u];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)s_digit << shift;
      mask |= 0xffu << shift;
      krem = s_krem;
    }
    thr = prefix;
    take_eq = krem;
  }

  // compaction in page order: ballots within a wave, counts across waves
  const unsigned long long below = (1ull << lane) - 1ull;
  int eq_seen = 0, taken = 0;
  for (int base = 0; base < npg; base += RT) {
    const int j = base + tid;
    const uint32_t key = j < npg ? s_keys[j] : 0u;
    const bool eq = !all && j < npg && key == thr;
    const unsigned long long eqm = __ballot(eq);
    if (lane == 0) s_wcnt[wave][0] = __popcll(eqm);
    __syncthreads();
    int eq_before = 0, eq_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      eq_before += w < wave ? s_wcnt[w][0] : 0;
      eq_total += s_wcnt[w][0];
    }
    const bool take =
        j < npg && (all || key > thr || (eq && eq_seen + eq_before + __popcll(eqm & below) < take_eq));
    const unsigned long long tm = __ballot(take);
    if (lane == 0) s_wcnt[wave][1] = __popcll(tm);
    __syncthreads();
    int take_before = 0, take_total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      take_before += w < wave ? s_wcnt[w][1] : 0;
      take_total += s_wcnt[w][1];
    }
    if (take) {
      const int p = taken + take_before + __popcll(tm & below);
      if (p < k) {
        sel[p] = j;
        if (selp) selp[p] = s_pid[j];
      }
    }
    eq_seen += eq_total;
    taken += take_total;
    __syncthreads();
  }
}

size_t route_lds_bytes(const Shape& s, bool append) {
  return route_lds(s.max_pages, s.head_dim, s.rank_v, s.rank_k, s.group, s.page_size, s.dtype == 0 ? 4 : 2, append)
      .total;
}

template <typename T, bool APPEND, int D>
hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  const size_t lds = route_lds_bytes(a.s, APPEND);
  const hipError_t e = allow_lds((const void*)route_kernel<T, APPEND, D>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((route_kernel<T, APPEND, D>), dim3(a.s.batch * a.s.n_kv_heads), dim3(RT), lds, st, a);
  return hipGetLastError();
}

template <typename T, bool APPEND>
hipError_t launch_d(const RouteArgs& a, hipStream_t st) {
  return a.s.head_dim == 64 ? launch_t<T, APPEND, 64>(a, st) : launch_t<T, APPEND, 128>(a, st);
}

}  // namespace

bool route_fits(const Shape& s, bool append) {
  // the kernel's static arrays take under 24 KiB; gfx950 has 160 KiB per CU
  return route_lds_bytes(s, append) + 24 * 1024 <= 160 * 1024;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const bool append = a.pos != nullptr;
  if (a.s.dtype == 0) return append ? launch_d<float, true>(a, st) : launch_d<float, false>(a, st);
  return append ? launch_d<uint16_t, true>(a, st) : launch_d<uint16_t, false>(a, st);
}

}  // namespace bkv
