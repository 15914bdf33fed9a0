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
// traffic: the factors are staged in LDS (P and R_dec rows padded to 16-byte
// aligned strides for float4 dot products), one lane scores one page from its
// fp32 sums with every load of the kernel's front in flight at once; an
// MSB-first 8-bit radix select over order-preserving keys in LDS (per-wave
// histograms merged once per pass) finds the k-th score, and ballots plus
// per-wave counts compact the selection in page order.
#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int RT = 512;
constexpr int VMAX = 64;  // page-sum channels held in registers per pass

// One staging round: every 16-byte chunk of every item is loaded before the
// first LDS store, so the whole front of the kernel costs one memory round
// trip.  Items: fp32 matrices (rows padded to ld floats), storage-dtype
// vectors (converted to fp32), and a latent page (channel rows padded to
// ps+1 floats).
enum ChunkKind { CK_F32_MATRIX = 0, CK_VECTOR = 1, CK_ZPAGE = 2 };
struct ChunkItem {
  const void* src;
  float* dst;
  int n16;    // 16-byte chunks
  int kind;
  int cols;   // CK_F32_MATRIX: row length; CK_ZPAGE: page size
  int ld;     // CK_F32_MATRIX: LDS row stride
};
constexpr int MAX_ITEMS = 9;
constexpr int CHUNKS_PER_THREAD = 8;

template <typename T>
__device__ __forceinline__ void stage_chunks(const ChunkItem (&it)[MAX_ITEMS], int n_items) {
  constexpr int PER = 16 / sizeof(T);
  int start[MAX_ITEMS + 1];
  start[0] = 0;
#pragma unroll
  for (int m = 0; m < MAX_ITEMS; ++m) start[m + 1] = start[m] + (m < n_items ? it[m].n16 : 0);
  const int total = start[MAX_ITEMS];
  for (int base = threadIdx.x; base < total; base += RT * CHUNKS_PER_THREAD) {
    u32x4 v[CHUNKS_PER_THREAD];
#pragma unroll
    for (int u = 0; u < CHUNKS_PER_THREAD; ++u) {
      const int c = base + u * RT;
      if (c < total) {
        const u32x4* src = reinterpret_cast<const u32x4*>(it[0].src) + c;
#pragma unroll
        for (int m = 1; m < MAX_ITEMS; ++m)
          if (c >= start[m]) src = reinterpret_cast<const u32x4*>(it[m].src) + (c - start[m]);
        v[u] = *src;
      }
    }
#pragma unroll
    for (int u = 0; u < CHUNKS_PER_THREAD; ++u) {
      const int c = base + u * RT;
      if (c >= total) continue;
      int m = 0;
#pragma unroll
      for (int mm = 1; mm < MAX_ITEMS; ++mm)
        if (c >= start[mm]) m = mm;
      int cc = c, kind = it[0].kind, cols = it[0].cols, ld = it[0].ld;
      float* dst = it[0].dst;
#pragma unroll
      for (int mm = 1; mm < MAX_ITEMS; ++mm)
        if (mm == m) {
          cc = c - start[mm];
          kind = it[mm].kind;
          cols = it[mm].cols;
          ld = it[mm].ld;
          dst = it[mm].dst;
        }
      if (kind == CK_F32_MATRIX) {
        const int e = cc * 4;
        float* d = dst + (e / cols) * ld + e % cols;
#pragma unroll
        for (int k = 0; k < 4; ++k) d[k] = __uint_as_float(v[u][k]);
      } else {
#pragma unroll
        for (int k = 0; k < PER; ++k) {
          const uint32_t w = v[u][k * sizeof(T) / 4];
          const float f = sizeof(T) == 2 ? __uint_as_float(((k & 1) ? (w >> 16) : (w & 0xffffu)) << 16)
                                         : __uint_as_float(w);
          const int e = cc * PER + k;
          if (kind == CK_VECTOR) dst[e] = f;
          else dst[(e / cols) * (cols + 1) + e % cols] = f;
        }
      }
    }
  }
}

template <typename T, bool APPEND>
__global__ __launch_bounds__(RT) void route_kernel(RouteArgs a) {
  extern __shared__ float lds[];
  __shared__ float s_q[MAX_GROUP * 128];  // [G][D]
  __shared__ float s_qc[MAX_GROUP][MAX_RANK + MAX_RESID];
  __shared__ float s_tok[3][128];  // appended token: v, k, Key remainder
  __shared__ float s_zt[MAX_RANK];
  __shared__ float s_newsum[MAX_RANK + MAX_RESID];  // the appended page's sums

  const int pair = blockIdx.x;
  const int H = a.s.n_kv_heads, G = a.s.group, D = a.s.head_dim;
  const int R = a.s.rank_v, RK = a.s.rank_k, RR = R + RK, ps = a.s.page_size;
  const int b = pair / H, g = pair % H;
  const int tid = threadIdx.x;
  const int32_t* pt = a.page_table + (size_t)b * a.s.max_pages;

  const int LDP = lds_row(D);
  float* sP = lds;                 // [R][LDP]
  float* sRd = sP + R * LDP;       // [RK][LDP]
  float* sB = sRd + RK * LDP;      // [D][R]   (append)
  float* sRe = sB + D * R;         // [D][RK]  (append)
  float* sZp = sRe + D * RK;       // [R][ps+1] the appended page's stored latents
  float* sSp = sZp + R * (ps + 1); // [ps][RK] ... and residuals
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(lds);  // [max_pages], after the projections

  int pos = -1;
  if (APPEND) {
    pos = a.pos[b];
    if (pos >= a.s.max_pages * ps) pos = -1;
  }
  const int apage = pos >= 0 ? pos / ps : -1, slot = pos >= 0 ? pos % ps : 0;
  const int aphys = pos >= 0 ? pt[apage] : 0;
  T* Kp = static_cast<T*>(a.K);
  T* Zp = static_cast<T*>(a.Z);
  T* Sp = static_cast<T*>(a.S);
  const size_t zbase = ((size_t)aphys * H + g) * R * ps;
  const size_t sbase = ((size_t)aphys * H + g) * ps * RK;

  // ---- one round of loads: factors, query, the new token and the appended
  // page into LDS; each scoring lane's page sums into registers ----
  {
    const T* q = static_cast<const T*>(a.q) + ((size_t)b * a.s.n_q_heads + g * G) * D;
    const bool app = APPEND && pos >= 0;
    const size_t tok = ((size_t)b * H + g) * D;
    const int tchunks = (int)(D * sizeof(T) / 16);
    // fixed slots (the append's items carry no chunks when there is no append)
    ChunkItem it[MAX_ITEMS] = {
        {a.P + (size_t)g * R * D, sP, R * D / 4, CK_F32_MATRIX, D, LDP},
        {a.R_dec + (size_t)g * RK * D, sRd, RK * D / 4, CK_F32_MATRIX, D, LDP},
        {q, s_q, (int)(G * D * sizeof(T) / 16), CK_VECTOR, 0, 0},
        {a.B + (size_t)g * D * R, sB, app ? D * R / 4 : 0, CK_F32_MATRIX, R, R},
        {a.R_enc + (size_t)g * D * RK, sRe, app ? D * RK / 4 : 0, CK_F32_MATRIX, RK, RK},
        {static_cast<const T*>(a.v_new) + tok, s_tok[0], app ? tchunks : 0, CK_VECTOR, 0, 0},
        {static_cast<const T*>(a.k_new) + tok, s_tok[1], app ? tchunks : 0, CK_VECTOR, 0, 0},
        {Zp + zbase, sZp, app ? (int)(R * ps * sizeof(T) / 16) : 0, CK_ZPAGE, ps, 0},
        {Sp + sbase, sSp, app ? (int)(ps * RK * sizeof(T) / 16) : 0, CK_VECTOR, 0, 0}};
    stage_chunks<T>(it, MAX_ITEMS);
  }
  const int n = a.seq_lens[b];
  const int npg = n > 0 ? min((n + ps - 1) / ps, a.s.max_pages) : 0;
  // this lane's page sums (lane j scores page j; npg <= 512 and r + r_k <= 64
  // take the prefetched one-pass path)
  float v[VMAX];
  const bool one_pass = npg <= RT && RR <= VMAX;
  if (one_pass && tid < npg) {
    const float* sm = a.summ + ((size_t)pt[tid] * H + g) * RR;
#pragma unroll
    for (int u = 0; u < VMAX / 4; ++u) {
      float4 t4 = {0.f, 0.f, 0.f, 0.f};
      if (4 * u < RR) t4 = *reinterpret_cast<const float4*>(sm + 4 * u);
      v[4 * u] = t4.x;
      v[4 * u + 1] = t4.y;
      v[4 * u + 2] = t4.z;
      v[4 * u + 3] = t4.w;
    }
  }
  __syncthreads();

  if (APPEND && pos >= 0) {
    // the new token: exact Key, rounded latent and residual, then its page's sums
    const size_t kbase = ((size_t)aphys * H + g) * ps * D;
    if (tid < R) {
      const float zt = round_store(Zp, zbase + (size_t)tid * ps + slot, latent_dot(s_tok[0], sB, D, R, tid));
      s_zt[tid] = zt;
      sZp[tid * (ps + 1) + slot] = zt;
    }
    if (tid >= RT - D)
      Kp[kbase + (size_t)slot * D + (tid - (RT - D))] =
          static_cast<const T*>(a.k_new)[((size_t)b * H + g) * D + (tid - (RT - D))];
    __syncthreads();
    if (tid < D) s_tok[2][tid] = key_remainder(s_tok[1][tid], s_zt, sP, LDP, R, tid);
    __syncthreads();
    if (tid < RK) sSp[slot * RK + tid] = round_store(Sp, sbase + (size_t)slot * RK + tid, residual_dot(s_tok[2], sRe, D, RK, tid));
    __syncthreads();
    if (tid < RR) {
      const float sum = page_channel_sum(sZp, sSp, R, RK, ps, tid, slot + 1);
      a.summ[((size_t)aphys * H + g) * RR + tid] = sum;
      s_newsum[tid] = sum;
    }
    __syncthreads();
  }

  // the query seen through the latent predictor P and the residual decoder R_dec
  for (int o = tid; o < G * 128; o += RT) {
    const int h = o / 128, x = o % 128;
    float acc = 0.f;
    if (x < RR) {
      const float4* row = reinterpret_cast<const float4*>(x < R ? sP + x * LDP : sRd + (x - R) * LDP);
      const float4* qv = reinterpret_cast<const float4*>(s_q + h * D);
      for (int i = 0; i < D / 4; ++i) {
        const float4 p4 = row[i], q4 = qv[i];
        acc = fmaf(p4.x, q4.x, acc);
        acc = fmaf(p4.y, q4.y, acc);
        acc = fmaf(p4.z, q4.z, acc);
        acc = fmaf(p4.w, q4.w, acc);
      }
    }
    s_qc[h][x] = acc * a.s.scale;
  }
  __syncthreads();

  // one lane per page: score from the page's fp32 sums
  // one lane per page; the page sums in registers, 64 channels at a time
  float d[MAX_GROUP];
  auto accumulate = [&](const float (&vv)[VMAX], int x0) {
#pragma unroll
    for (int h = 0; h < MAX_GROUP; ++h)
      if (h < G) {
#pragma unroll
        for (int x = 0; x < VMAX; ++x)
          if (x0 + x < RR) d[h] = fmaf(s_qc[h][x0 + x], vv[x], d[h]);
      }
  };
  auto finish = [&](int j) {
    const int cnt = min(ps, n - j * ps);
    float best = -__builtin_huge_valf();
#pragma unroll
    for (int h = 0; h < MAX_GROUP; ++h)
      if (h < G) best = fmaxf(best, d[h]);
    const float sc = best / (float)cnt;
    a.scores[(size_t)pair * a.s.max_pages + j] = sc;
    s_keys[j] = float_key(sc);
  };
  if (one_pass) {
    if (tid < npg) {
      if (APPEND && tid == apage) {
#pragma unroll
        for (int x = 0; x < VMAX; ++x) v[x] = x < RR ? s_newsum[x] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < MAX_GROUP; ++h) d[h] = 0.f;
      accumulate(v, 0);
      finish(tid);
    }
  } else {
    for (int j = tid; j < npg; j += RT) {
      const float* sm = a.summ + ((size_t)pt[j] * H + g) * RR;
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
        accumulate(v, x0);
      }
      finish(j);
    }
  }
  __syncthreads();

  // ---- top-k selection: per-wave histograms, one merge per radix pass ----
  constexpr int NW = RT / 64;
  __shared__ int s_whist[NW][256];
  __shared__ int s_tot[256];
  __shared__ int s_wcnt[NW][2];
  __shared__ int s_digit, s_krem;
  const int wave = tid >> 6, lane = tid & 63;
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
        if (selp) selp[p] = pt[j];
      }
    }
    eq_seen += eq_total;
    taken += take_total;
    __syncthreads();
  }
}

size_t route_lds_bytes(const Shape& s, bool append) {
  const size_t D = s.head_dim, R = s.rank_v, RK = s.rank_k, ps = s.page_size;
  size_t f = (R + RK) * lds_row(s.head_dim);
  if (append) f += D * R + D * RK + R * (ps + 1) + ps * RK;
  if (f < (size_t)s.max_pages) f = s.max_pages;
  return f * sizeof(float);
}

template <typename T, bool APPEND>
hipError_t launch_t(const RouteArgs& a, hipStream_t st) {
  const size_t lds = route_lds_bytes(a.s, APPEND);
  const hipError_t e = allow_lds((const void*)route_kernel<T, APPEND>, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((route_kernel<T, APPEND>), dim3(a.s.batch * a.s.n_kv_heads), dim3(RT), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const bool append = a.pos != nullptr;
  if (a.s.dtype == 0) return append ? launch_t<float, true>(a, st) : launch_t<float, false>(a, st);
  return append ? launch_t<uint16_t, true>(a, st) : launch_t<uint16_t, false>(a, st);
}

}  // namespace bkv
