// Router: page scores predicted from the Value latents plus the Key residual,
// then top-k page selection per (sequence, KV head).
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
//
// One launch: workgroups score chunks of pages (4 lanes per page, fp32); the
// last workgroup of a pair to finish selects with an MSB-first 8-bit radix
// select over order-preserving keys in LDS, then compacts in page order with
// two block scans.
#include "common.hpp"
#include "internal.hpp"

namespace bkv {

namespace {

constexpr int THREADS = 256;
constexpr int XPL = (MAX_RANK + MAX_RESID) / 4;  // summary values per lane, upper bound

__device__ int block_incl_scan(int x, int* s_wave) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int incl = wave_incl_scan(x);
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wave; ++w) off += s_wave[w];
  __syncthreads();
  return off + incl;
}

__global__ __launch_bounds__(THREADS) void route_kernel(RouteArgs a) {
  extern __shared__ uint32_t s_keys[];  // [max_pages]
  __shared__ float s_q[MAX_GROUP][128];
  __shared__ float s_qc[MAX_GROUP][MAX_RANK + MAX_RESID];
  __shared__ int s_hist[256];
  __shared__ int s_wave[4];
  __shared__ int s_digit, s_krem, s_last;

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = wg / a.n_chunks, chunk = wg % a.n_chunks;
  const int H = a.s.n_kv_heads, G = a.s.group, D = a.s.head_dim;
  const int R = a.s.rank_v, RR = a.s.rank_v + a.s.rank_k, ps = a.s.page_size;
  const int b = pair / H, g = pair % H;
  const int tid = threadIdx.x;
  const int n = a.seq_lens[b];
  const int npg = n > 0 ? min((n + ps - 1) / ps, a.s.max_pages) : 0;

  // ---- scores of this workgroup's pages ----
  const int j0 = chunk * a.pages_per_wg;
  const int j1 = min(j0 + a.pages_per_wg, npg);
  if (j0 < j1) {
    for (int o = tid; o < G * D; o += THREADS) {
      const size_t qi = ((size_t)b * a.s.n_q_heads + g * G + o / D) * D + o % D;
      s_q[o / D][o % D] = a.s.dtype == 0 ? static_cast<const float*>(a.q)[qi]
                                         : bf16_to_f32(static_cast<const uint16_t*>(a.q)[qi]);
    }
    __syncthreads();
    // the query seen through the latent predictor P and the residual decoder R_dec
    for (int o = tid; o < G * RR; o += THREADS) {
      const int h = o / RR, x = o % RR;
      const float* row = x < R ? a.P + ((size_t)g * R + x) * D : a.R_dec + ((size_t)g * a.s.rank_k + (x - R)) * D;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc += row[i] * s_q[h][i];
      s_qc[h][x] = acc * a.s.scale;
    }
    __syncthreads();
    const int xpl = RR / 4, sub = tid & 3;
    for (int j = j0 + tid / 4; j < j1; j += THREADS / 4) {
      const int phys = a.page_table[(size_t)b * a.s.max_pages + j];
      const int cnt = min(ps, n - j * ps);
      const float* sm = a.summ + ((size_t)phys * H + g) * RR + sub * xpl;
      float v[XPL];
#pragma unroll
      for (int u = 0; u < XPL; ++u) v[u] = u < xpl ? sm[u] : 0.f;
      float best = -__builtin_huge_valf();
      for (int h = 0; h < G; ++h) {
        const float* qc = &s_qc[h][sub * xpl];
        float d = 0.f;
#pragma unroll
        for (int u = 0; u < XPL; ++u)
          if (u < xpl) d += qc[u] * v[u];
        d += __shfl_xor(d, 1);
        d += __shfl_xor(d, 2);
        best = fmaxf(best, d);
      }
      if (sub == 0) a.scores[(size_t)pair * a.s.max_pages + j] = best / (float)cnt;
    }
  }

  // ---- the last workgroup of this pair selects ----
  __threadfence();
  __syncthreads();
  if (a.n_chunks > 1) {
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(&a.counters[pair], 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = prev == (unsigned)(a.n_chunks - 1);
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
  }

  const int k = min(a.s.top_k, npg);
  int32_t* sel = a.sel + (size_t)pair * a.s.top_k;
  for (int p = k + tid; p < a.s.top_k; p += THREADS) sel[p] = -1;
  if (tid == 0) a.n_sel[pair] = k;
  if (k > 0) {
    const float* sc = a.scores + (size_t)pair * a.s.max_pages;
    for (int j = tid; j < npg; j += THREADS) s_keys[j] = float_key(sc[j]);
    __syncthreads();

    uint32_t T = 0;
    int take_eq = 0;
    const bool all = k == npg;
    if (!all) {
      uint32_t prefix = 0, mask = 0;
      int krem = k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        s_hist[tid] = 0;
        __syncthreads();
        for (int j = tid; j < npg; j += THREADS) {
          const uint32_t key = s_keys[j];
          if ((key & mask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        const int c = s_hist[255 - tid];  // digits in descending order
        const int incl = block_incl_scan(c, s_wave);
        if (incl >= krem && incl - c < krem) {
          s_digit = 255 - tid;
          s_krem = krem - (incl - c);
        }
        __syncthreads();
        prefix |= (uint32_t)s_digit << shift;
        mask |= 0xffu << shift;
        krem = s_krem;
        __syncthreads();
      }
      T = prefix;
      take_eq = krem;
    }

    // ordered compaction: thread t owns pages [t*E, (t+1)*E)
    const int E = (npg + THREADS - 1) / THREADS;
    const int lo = min(tid * E, npg), hi = min(lo + E, npg);
    int n_eq = 0;
    if (!all)
      for (int j = lo; j < hi; ++j) n_eq += s_keys[j] == T;
    const int eq_before = block_incl_scan(n_eq, s_wave) - n_eq;
    int n_take = 0;
    {
      int seen = eq_before;
      for (int j = lo; j < hi; ++j) {
        const uint32_t key = s_keys[j];
        bool take = all || key > T;
        if (!all && key == T) take = seen++ < take_eq;
        n_take += take;
      }
    }
    int pos = block_incl_scan(n_take, s_wave) - n_take;
    {
      int seen = eq_before;
      for (int j = lo; j < hi; ++j) {
        const uint32_t key = s_keys[j];
        bool take = all || key > T;
        if (!all && key == T) take = seen++ < take_eq;
        if (take && pos < k) sel[pos++] = j;
      }
    }
  }
  if (a.n_chunks > 1 && tid == 0)
    __hip_atomic_store(&a.counters[pair], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

int route_pages_per_wg(const Shape& s) {
  // Enough workgroups to spread the page-sum reads over the chip: about 512
  // in total, at least 64 pages each.
  const long pairs = (long)s.batch * s.n_kv_heads;
  long per = (pairs * s.max_pages + 511) / 512;
  per = ((per + 63) / 64) * 64;
  if (per < 64) per = 64;
  const char* env = getenv("BASISKV_ROUTE_PAGES_PER_WG");
  if (env && atoi(env) > 0) per = atoi(env);
  return (int)per;
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  const int pairs = a.s.batch * a.s.n_kv_heads;
  const size_t lds = (size_t)a.s.max_pages * sizeof(uint32_t);
  hipLaunchKernelGGL(route_kernel, dim3(pairs * a.n_chunks), dim3(THREADS), lds, st, a);
  return hipGetLastError();
}

}  // namespace bkv
