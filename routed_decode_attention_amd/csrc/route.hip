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
// One 1024-thread workgroup per (sequence, KV head), no cross-workgroup
// traffic: the factors are staged in LDS (P and R_dec rows padded to 16-byte
// aligned strides for float4 dot products), one lane scores one page from its
// fp32 sums with every load of the page in flight at once, and one wave then
// selects without workgroup barriers: an MSB-first 8-bit radix select over
// order-preserving keys in LDS finds the k-th score, and ballots compact the
// selection in page order.
#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int RT = 1024;

template <typename T, bool APPEND>
__global__ __launch_bounds__(RT) void route_kernel(RouteArgs a) {
  extern __shared__ float lds[];
  __shared__ float s_q[MAX_GROUP][128];
  __shared__ float s_qc[MAX_GROUP][MAX_RANK + MAX_RESID];
  __shared__ float s_tok[3][128];  // appended token: v, k, Key remainder
  __shared__ float s_zt[MAX_RANK];
  __shared__ int s_hist[256];

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
  uint32_t* s_keys = reinterpret_cast<uint32_t*>(lds);  // [max_pages], after the projections

  stage_matrix(sP, LDP, a.P + (size_t)g * R * D, R, D);
  stage_matrix(sRd, LDP, a.R_dec + (size_t)g * RK * D, RK, D);
  const T* q = static_cast<const T*>(a.q);
  for (int o = tid; o < G * D; o += RT)
    s_q[o / D][o % D] = ld_elem(q, ((size_t)b * a.s.n_q_heads + g * G + o / D) * D + o % D);
  int pos = -1;
  if (APPEND) {
    stage_matrix(sB, R, a.B + (size_t)g * D * R, D, R);
    stage_matrix(sRe, RK, a.R_enc + (size_t)g * D * RK, D, RK);
    pos = a.pos[b];
    if (pos >= a.s.max_pages * ps) pos = -1;
    if (pos >= 0) {
      const T* kin = static_cast<const T*>(a.k_new);
      const T* vin = static_cast<const T*>(a.v_new);
      for (int i = tid; i < D; i += RT) {
        const size_t src = ((size_t)b * H + g) * D + i;
        s_tok[0][i] = ld_elem(vin, src);
        s_tok[1][i] = ld_elem(kin, src);
      }
    }
  }
  __syncthreads();

  if (APPEND && pos >= 0) {
    // the new token: exact Key, rounded latent and residual, then its page's sums
    const int page = pos / ps, slot = pos % ps;
    const int phys = pt[page];
    T* Kp = static_cast<T*>(a.K);
    T* Zp = static_cast<T*>(a.Z);
    T* Sp = static_cast<T*>(a.S);
    const size_t kbase = ((size_t)phys * H + g) * ps * D;
    const size_t zbase = ((size_t)phys * H + g) * R * ps;
    const size_t sbase = ((size_t)phys * H + g) * ps * RK;
    if (tid < R) s_zt[tid] = round_store(Zp, zbase + (size_t)tid * ps + slot, latent_dot(s_tok[0], sB, D, R, tid));
    if (tid >= 512 && tid < 512 + D)
      Kp[kbase + (size_t)slot * D + (tid - 512)] =
          static_cast<const T*>(a.k_new)[((size_t)b * H + g) * D + (tid - 512)];
    __syncthreads();
    if (tid < D) s_tok[2][tid] = key_remainder(s_tok[1][tid], s_zt, sP, LDP, R, tid);
    __syncthreads();
    if (tid < RK) round_store(Sp, sbase + (size_t)slot * RK + tid, residual_dot(s_tok[2], sRe, D, RK, tid));
    __threadfence_block();
    __syncthreads();
    // the page's stored latents and residuals (B and R_enc are no longer needed)
    float* sZp = sB;                    // [R][ps+1]
    float* sSp = sB + R * (ps + 1);     // [ps][RK]
    stage_page(sZp, sSp, Zp + zbase, Sp + sbase, R, RK, ps);
    __syncthreads();
    if (tid < RR) a.summ[((size_t)phys * H + g) * RR + tid] = page_channel_sum(sZp, sSp, R, RK, ps, tid, slot + 1);
    __threadfence_block();
    __syncthreads();
  }

  // the query seen through the latent predictor P and the residual decoder R_dec
  for (int o = tid; o < G * 128; o += RT) {
    const int h = o / 128, x = o % 128;
    float acc = 0.f;
    if (x < RR) {
      const float4* row = reinterpret_cast<const float4*>(x < R ? sP + x * LDP : sRd + (x - R) * LDP);
      const float4* qv = reinterpret_cast<const float4*>(s_q[h]);
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
  const int n = a.seq_lens[b];
  const int npg = n > 0 ? min((n + ps - 1) / ps, a.s.max_pages) : 0;
  for (int j = tid; j < npg; j += RT) {
    const int phys = pt[j];
    const int cnt = min(ps, n - j * ps);
    const float* sm = a.summ + ((size_t)phys * H + g) * RR;
    float d[MAX_GROUP];
#pragma unroll
    for (int h = 0; h < MAX_GROUP; ++h) d[h] = 0.f;
    for (int x0 = 0; x0 < RR; x0 += 64) {
      float v[64];
#pragma unroll
      for (int u = 0; u < 16; ++u) {  // every load of the chunk issued before the first use
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
          const float* qc = &s_qc[h][x0];
#pragma unroll
          for (int x = 0; x < 64; ++x) d[h] = fmaf(qc[x], v[x], d[h]);
        }
    }
    float best = -__builtin_huge_valf();
#pragma unroll
    for (int h = 0; h < MAX_GROUP; ++h)
      if (h < G) best = fmaxf(best, d[h]);
    const float sc = best / (float)cnt;
    a.scores[(size_t)pair * a.s.max_pages + j] = sc;
    s_keys[j] = float_key(sc);
  }
  __syncthreads();

  // ---- top-k selection, by wave 0 alone ----
  if (tid >= 64) return;
  const int lane = tid;
  const int k = min(a.s.top_k, npg);
  int32_t* sel = a.sel + (size_t)pair * a.s.top_k;
  int32_t* selp = a.sel_phys ? a.sel_phys + (size_t)pair * a.s.top_k : nullptr;
  for (int p = k + lane; p < a.s.top_k; p += 64) {
    sel[p] = -1;
    if (selp) selp[p] = -1;
  }
  if (lane == 0) a.n_sel[pair] = k;
  if (k == 0) return;

  uint32_t thr = 0;
  int take_eq = 0;
  const bool all = k == npg;
  if (!all) {
    uint32_t prefix = 0, mask = 0;
    int krem = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) s_hist[lane + 64 * u] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < npg; j += 64) {
        const uint32_t key = s_keys[j];
        if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
      }
      __builtin_amdgcn_wave_barrier();
      // lane owns digits 255-4*lane .. 252-4*lane (descending)
      int c[4], own = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        c[u] = s_hist[255 - 4 * lane - u];
        own += c[u];
      }
      int run = wave_incl_scan(own) - own;  // keys with a larger digit than this lane's
      int digit = -1, nk = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (digit < 0 && run < krem && run + c[u] >= krem) {
          digit = 255 - 4 * lane - u;
          nk = krem - run;
        }
        run += c[u];
      }
      const unsigned long long hit = __ballot(digit >= 0);
      const int src = __ffsll((long long)hit) - 1;
      digit = __shfl(digit, src);
      krem = __shfl(nk, src);
      prefix |= (uint32_t)digit << shift;
      mask |= 0xffu << shift;
      __builtin_amdgcn_wave_barrier();
    }
    thr = prefix;
    take_eq = krem;
  }

  // compaction in page order with ballots
  const unsigned long long below = (1ull << lane) - 1ull;
  int eq_seen = 0, taken = 0;
  for (int base = 0; base < npg; base += 64) {
    const int j = base + lane;
    const uint32_t key = j < npg ? s_keys[j] : 0u;
    const bool eq = !all && j < npg && key == thr;
    const unsigned long long eqm = __ballot(eq);
    const bool take = j < npg && (all || key > thr || (eq && eq_seen + __popcll(eqm & below) < take_eq));
    const unsigned long long tm = __ballot(take);
    if (take) {
      const int p = taken + __popcll(tm & below);
      if (p < k) {
        sel[p] = j;
        if (selp) selp[p] = pt[j];
      }
    }
    eq_seen += __popcll(eqm);
    taken += __popcll(tm);
  }
}

size_t route_lds_bytes(const Shape& s, bool append) {
  const size_t D = s.head_dim, R = s.rank_v, RK = s.rank_k, ps = s.page_size;
  size_t f = (R + RK) * lds_row(s.head_dim);
  if (append) {
    const size_t factors = D * R + D * RK, page = R * (ps + 1) + ps * RK;
    f += factors > page ? factors : page;
  }
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
