// Gathered exact-QK split-K decode attention over the routed pages.
//
// The router keeps only the top-k pages per (sequence, KV head); their exact
// Keys are read back to score q.k exactly, and the softmax weights sum the
// stored Value latents (weekinpapers "BasisKV: Value Latents for
// Communication and Key Routing", Abstract; kongchang article, coarse routing
// then exact scoring; softmax(q.k / sqrt(d_h)) from machinelearning.ru
// "KV-кэширование", "Математическая формализация").
//
// Work split: a (sequence, KV head) pair's selected pages are cut into
// n_wsplit workgroup splits of `waves` waves (4 or 8); each wave owns
// pages_per_wave consecutive selected pages and keeps an online softmax
// (running max m, denominator l, latent accumulator) for every query head of
// the group.  The waves of a workgroup merge through LDS and the workgroup
// writes one partial (acc, m, l) per query head; the splits are combined by
// the kernel that consumes them (the merge, or the merge fused with the
// output projection), so no workgroup waits for another.  With a single
// split the workgroup writes the normalised latent itself.
//
// bf16 storage, d_h in {64,128}, page 32/64, r in {16,32,48,64}: matrix-core
// kernel.  Per 32-token chunk of a page, S = K.q^T runs as two 16x16x32 bf16
// MFMAs per 32 dims with the page's tokens as rows and the group's query
// heads as columns (q is the B operand, loaded once).  Row m of the two
// tiles a=0,1 is token 32c + 8*(m/4) + 4a + m%4, so each lane ends up holding
// 8 consecutive tokens (32c + 8*qd + 0..7) of one head: exactly the k-slice
// it must supply for the transposed latent product Acc^T[r][h] +=
// Z^T[r][t] . P^T[t][h], whose A operand is the channel-major latent page
// loaded straight from HBM.  Every softmax statistic of head h then lives in
// the lanes of column h, so rescaling needs no cross-lane traffic.  A page's
// 20 16-byte fragments per lane are all issued before its first MFMA, and the
// next page's while the current one is multiplied.
// Everything else (fp32 storage, other shapes): a plain VALU kernel with the
// same split and merge.
#include <cstdlib>

#include "attend_core.hpp"
#include "split_merge.hpp"

namespace bkv {

namespace {

// Selection in the prologue (the decode step): every workgroup of a pair
// ranks the pair's pages from the router's scores itself (select.hpp) and
// keeps the positions [split * waves * ppw, +waves * ppw) of the selection
// in page order, with their physical ids; split 0 also writes the selection
// (sel, n_sel) for the caller.  Returns the selection count.  after_issue()
// runs once the first scores and page-table entries are requested: loads it
// issues complete after them (in issue order), so the selection does not
// wait for them.
template <typename AfterIssue>
__device__ int select_prologue(const AttendArgs& a, int pair, int split, const SelLds& L, AfterIssue&& after_issue) {
  const int b = pair / a.s.n_kv_heads, ps = a.s.page_size, maxp = a.s.max_pages;
  const int tid = threadIdx.x, nt = blockDim.x;
  const float* sc = a.scores + (size_t)pair * maxp;
  const int32_t* pt = a.page_table + (size_t)b * maxp;
  // the first SEL_PRE strides of scores and page-table entries are requested
  // before the sequence length is known (clamped and unconditional, so that
  // they are in flight together with it, and so that the compiler's waits
  // for each stride count exactly the loads issued after it; entries past
  // the sequence or the table are read but not used)
  constexpr int SEL_PRE = SEL_SB;
  float s_pre[SEL_PRE];
  int32_t p_pre[SEL_PRE];
#pragma unroll
  for (int i = 0; i < SEL_PRE; ++i) {
    const int j = min(tid + i * nt, maxp - 1);
    s_pre[i] = sc[j];
    p_pre[i] = pt[j];
  }
  after_issue();
  const int n = a.seq_lens[b];
  const int npg = n > 0 ? min((n + ps - 1) / ps, maxp) : 0;
  uint32_t kmax = 0u, kmin = 0xffffffffu;  // the range of the keys of pages that are not forced
  auto take = [&](int j, float score, int32_t phys) {
    const uint32_t k = select_key(score, j < a.sink_pages || j >= npg - a.local_pages);
    L.pg.keys[j] = k;
    L.pt[j] = phys;
    if (k != 0xFFFFFFFFu) {
      kmax = max(kmax, k);
      kmin = min(kmin, k);
    }
  };
#pragma unroll
  for (int i = 0; i < SEL_PRE; ++i)
    if (tid + i * nt < npg) take(tid + i * nt, s_pre[i], p_pre[i]);
  for (int j = tid + SEL_PRE * nt; j < npg; j += nt) take(j, sc[j], pt[j]);
  return select_tail(a, pair, split, L, npg, kmax, kmin);
}

template <int D, int PS, int R, bool PIPE, bool SEL>
__global__ __launch_bounds__(64 * ATTEND_WAVES_MAX) void attend_mfma_kernel(AttendArgs a) {
  constexpr int KS = D / 32, MT = R / 16;
  __shared__ WaveState st;
  extern __shared__ __attribute__((aligned(16))) float s_acc[];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = wg / a.n_wsplit, split = wg % a.n_wsplit;
  const int H = a.s.n_kv_heads, G = a.s.group;
  const int b = pair / H, g = pair % H;
  const int CH = a.s.cache_heads, cg = g / a.s.unit_div;  // the pair's head in the cache pools
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;

  const int first = (split * a.waves + wave) * a.pages_per_wave;
  const int seq_len = a.seq_lens[b];
  bf16x8 qb[KS];
  // lanes of tile columns n >= G load head 0's query (unconditional loads:
  // exact waits); the products keep every column apart and those columns
  // are never stored
  auto load_q = [&] {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         ((size_t)b * a.s.n_q_heads + g * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = load_bf16x8(qp + 8 * qd + 32 * s);
  };
  int my_j = 0, my_phys = 0, nsel;
  if constexpr (SEL) {
    // the queries are requested after the first scores and stay in flight
    // while the workgroup selects
    const SelLds L = sel_lds(s_acc, a.waves, G, R, a.s.max_pages, a.pages_per_wave);
    nsel = select_prologue(a, pair, split, L, load_q);
    const int u = wave * a.pages_per_wave + lane;
    if (lane < a.pages_per_wave && first + lane < nsel) {
      my_j = L.mine_j[u];
      my_phys = L.mine_p[u];
    }
  } else {
    load_q();
    // this wave's slice of the selection is read in the same round trip as
    // the sequence length and the selection count (every slot < top_k is in
    // bounds; slots past the count are masked below)
    const bool in_list = lane < a.pages_per_wave && first + lane < a.s.top_k;
    if (in_list) {
      const size_t at = (size_t)pair * a.s.top_k + first + lane;
      my_j = a.sel[at];
      if (a.sel_phys) my_phys = a.sel_phys[at];
    }
    nsel = seq_len > 0 ? a.n_sel[pair] : 0;
  }
  const int np = max(0, min(first + a.pages_per_wave, nsel) - first);  // pages of this wave
  // page ids and valid-token counts of this wave's pages, lane u holds page u
  int my_cnt = 0;
  if (lane < np) {
    if (!SEL && !a.sel_phys) my_phys = a.page_table[(size_t)b * a.s.max_pages + my_j];
    my_cnt = min(PS, seq_len - my_j * PS);
  } else {
    my_phys = 0;
  }
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K);
  const uint16_t* Zp = static_cast<const uint16_t*>(a.Z);
  auto kpage = [&](int u) {
    const int phys = __builtin_amdgcn_readlane(my_phys, u);
    return Kp + ((size_t)phys * CH + cg) * PS * D;
  };
  auto zpage = [&](int u) {
    const int phys = __builtin_amdgcn_readlane(my_phys, u);
    return Zp + ((size_t)phys * CH + cg) * R * PS;
  };

  OnlineSoftmax<D, PS, R> os;
  if (PIPE && np == 2) {
    // two pages (the usual case of the plans with two pages a wave): both
    // requested at once, in straight-line code, so that the first page's
    // math waits only for its own loads (a conditional second request would
    // make the compiler's waits count the second page's loads in)
    PageFrags<D, PS, R> fa, fb;
    fa.load(kpage(0), zpage(0), n, qd);
    fb.load(kpage(1), zpage(1), n, qd);
    __builtin_amdgcn_sched_barrier(0);
    os.page(fa, qb, __builtin_amdgcn_readlane(my_cnt, 0), qd, a.scale_log2);
    __builtin_amdgcn_sched_barrier(0);
    os.page(fb, qb, __builtin_amdgcn_readlane(my_cnt, 1), qd, a.scale_log2);
  } else if (PIPE) {  // several pages per wave: the next page's loads overlap this page's math
    PageFrags<D, PS, R> fa, fb;
    if (np > 0) fa.load(kpage(0), zpage(0), n, qd);
    for (int u = 0; u < np; u += 2) {
      if (u + 1 < np) fb.load(kpage(u + 1), zpage(u + 1), n, qd);
      __builtin_amdgcn_sched_barrier(0);
      os.page(fa, qb, __builtin_amdgcn_readlane(my_cnt, u), qd, a.scale_log2);
      if (u + 1 < np) {
        if (u + 2 < np) fa.load(kpage(u + 2), zpage(u + 2), n, qd);
        __builtin_amdgcn_sched_barrier(0);
        os.page(fb, qb, __builtin_amdgcn_readlane(my_cnt, u + 1), qd, a.scale_log2);
      }
    }
  } else {
    for (int u = 0; u < np; ++u) {
      PageFrags<D, PS, R> fa;
      fa.load(kpage(u), zpage(u), n, qd);
      __builtin_amdgcn_sched_barrier(0);
      os.page(fa, qb, __builtin_amdgcn_readlane(my_cnt, u), qd, a.scale_log2);
    }
  }

  // this wave's state into LDS: head n lives in lanes n, n+16, n+32, n+48
  float l = os.l;
  l = pair_sum<32>(pair_sum<16>(l));
  if (n < G) {
    if (qd == 0) {
      st.m[wave][n] = os.m;
      st.l[wave][n] = l;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc_at(s_acc, wave, n, 16 * t + 4 * qd + e, G, R) = os.acc[t][e];
  }
  finish_split(a, st, s_acc, pair, split);
}

// Plain VALU kernel: one lane per token for q.k, one lane per latent channel
// for the weighted sum.  Any storage dtype and any supported shape.
template <typename T, bool SEL>
__global__ __launch_bounds__(64 * ATTEND_WAVES_MAX) void attend_valu_kernel(AttendArgs a) {
  __shared__ WaveState st;
  extern __shared__ __attribute__((aligned(16))) float s_acc[];
  __shared__ __attribute__((aligned(16))) float s_q[MAX_GROUP][128];
  __shared__ __attribute__((aligned(16))) float s_p[ATTEND_WAVES_MAX][64];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = wg / a.n_wsplit, split = wg % a.n_wsplit;
  const int H = a.s.n_kv_heads, G = a.s.group, D = a.s.head_dim, R = a.s.rank_v;
  const int PS = a.s.page_size;
  const int b = pair / H, g = pair % H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const T* Kp = static_cast<const T*>(a.K);
  const T* Zp = static_cast<const T*>(a.Z);
  const T* qp = static_cast<const T*>(a.q);

  for (int o = threadIdx.x; o < G * D; o += blockDim.x)
    s_q[o / D][o % D] = ld_elem(qp, ((size_t)b * a.s.n_q_heads + g * G + o / D) * D + o % D);
  __syncthreads();

  const int seq_len = a.seq_lens[b];
  SelLds L{};
  int nsel;
  if constexpr (SEL) {
    L = sel_lds(s_acc, a.waves, G, R, a.s.max_pages, a.pages_per_wave);
    nsel = select_prologue(a, pair, split, L, [] {});
  } else {
    nsel = seq_len > 0 ? a.n_sel[pair] : 0;
  }
  const int base = split * a.waves * a.pages_per_wave;
  const int first = (split * a.waves + wave) * a.pages_per_wave;
  const int last = min(first + a.pages_per_wave, nsel);

  float m_run[MAX_GROUP], l_run[MAX_GROUP], acc[MAX_GROUP];
  for (int h = 0; h < MAX_GROUP; ++h) {
    m_run[h] = NEG_INF;
    l_run[h] = 0.f;
    acc[h] = 0.f;
  }
  for (int i = first; i < last; ++i) {
    const int j = SEL ? L.mine_j[i - base] : a.sel[(size_t)pair * a.s.top_k + i];
    const int phys = SEL ? L.mine_p[i - base] : a.page_table[(size_t)b * a.s.max_pages + j];
    const int cnt = min(PS, seq_len - j * PS);
    const size_t kbase = ((size_t)phys * a.s.cache_heads + g / a.s.unit_div) * PS * D;
    const size_t zbase = ((size_t)phys * a.s.cache_heads + g / a.s.unit_div) * R * PS;
    for (int h = 0; h < G; ++h) {
      float s = NEG_INF;
      if (lane < cnt) {
        float d = 0.f;
        for (int x = 0; x < D; ++x) d += s_q[h][x] * ld_elem(Kp, kbase + (size_t)lane * D + x);
        s = d * a.scale_log2;
      }
      const float mx = wave_max(s);
      if (mx == NEG_INF) continue;
      const float m_new = fmaxf(m_run[h], mx);
      const float alpha = exp2f(m_run[h] - m_new);
      const float p = lane < cnt ? exp2f(s - m_new) : 0.f;
      l_run[h] = l_run[h] * alpha + wave_sum(p);
      m_run[h] = m_new;
      s_p[wave][lane] = p;
      __builtin_amdgcn_wave_barrier();
      float z = 0.f;
      if (lane < R)
        for (int t = 0; t < cnt; ++t) z += s_p[wave][t] * ld_elem(Zp, zbase + (size_t)lane * PS + t);
      acc[h] = acc[h] * alpha + z;
      __builtin_amdgcn_wave_barrier();
    }
  }
  for (int h = 0; h < G; ++h) {
    if (lane == 0) {
      st.m[wave][h] = m_run[h];
      st.l[wave][h] = l_run[h];
    }
    if (lane < R) acc_at(s_acc, wave, h, lane, G, R) = acc[h];
  }
  finish_split(a, st, s_acc, pair, split);
}

// One workgroup per pair: every split of the pair combined, four latent
// channels per thread.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int pair = blockIdx.x;
  const int G = a.s.group, R = a.s.rank_v;
  const int b = pair / a.s.n_kv_heads, g = pair % a.s.n_kv_heads;
  const float* acc = a.part_acc + (size_t)pair * a.n_wsplit * G * R;
  const float* ml = a.part_ml + (size_t)pair * a.n_wsplit * G * 2;
  for (int t = threadIdx.x; t < G * R / 4; t += blockDim.x) {
    const int h = t / (R / 4), r0 = 4 * (t % (R / 4));
    const f32x4 z = merge_splits4(acc, ml, a.n_wsplit, G, R, h, r0);
    *reinterpret_cast<f32x4*>(a.z_out + ((size_t)b * a.s.n_q_heads + g * G + h) * R + r0) = z;
  }
}

}  // namespace

bool attend_mfma_supported(const Shape& s) {
  return s.dtype == 1 && (s.head_dim == 64 || s.head_dim == 128) &&
         (s.page_size == 32 || s.page_size == 64) && s.rank_v % 16 == 0 && s.rank_v <= 64 &&
         s.group <= MAX_GROUP;
}

AttendPlan plan_attend(const Shape& s) {
  // Resident waves: the plain kernel (one page a wave, 132 VGPRs) runs three
  // waves per SIMD, 3072 over the chip; the pipelined one (about 230 VGPRs)
  // two, 2048.  One page a wave while the grid fits the plain kernel's slots;
  // beyond, enough pages a wave for the pipelined kernel's (measured at 4096
  // page units, the 70B 128K share and the ragged mix: two pages a wave 54.3
  // and 43.3 us per step against 58.0 and 47.4 with one, 54.2 and 45.1 with
  // four).
  const long units = (long)s.batch * s.n_kv_heads * s.top_k;
  int ppw = units <= 3072 ? 1 : (int)((units + 2047) / 2048);
  if (ppw > 8) ppw = 8;
  const char* env = getenv("BASISKV_PAGES_PER_WAVE");
  if (env && atoi(env) > 0) ppw = atoi(env) < 32 ? atoi(env) : 32;
  // Four waves per workgroup; eight when four would leave more splits than
  // the merge requests in one round (their merge then costs a second round
  // trip: at top_k 128, 16 splits of 8 waves measured faster than 32 of 4,
  // while at top_k 64 the 16 splits of 4 waves are faster).
  // With several pages a wave (long contexts) eight waves as well: each
  // thread's share of the selection halves (70B 128K share: 44.9 against
  // 46.2 us per step; the ragged mix unchanged).
  int waves = ppw > 1 || (s.top_k + 4 * ppw - 1) / (4 * ppw) > MERGE_CHUNK ? 8 : 4;
  const char* wenv = getenv("BASISKV_ATTEND_WAVES");
  if (wenv && (atoi(wenv) == 4 || atoi(wenv) == 8)) waves = atoi(wenv);
  AttendPlan p;
  p.pages_per_wave = ppw;
  p.waves = waves;
  p.n_wsplit = (s.top_k + waves * ppw - 1) / (waves * ppw);
  return p;
}

template <bool SEL>
hipError_t launch_attend_t(const AttendArgs& a, hipStream_t st) {
  const int pairs = a.s.batch * a.s.n_kv_heads;
  const dim3 grid(pairs * a.n_wsplit), block(64 * a.waves);
  size_t lds = attend_acc_bytes(a.waves, a.s.group, a.s.rank_v);
  if (SEL) lds += attend_sel_bytes(a.s.max_pages, a.waves, a.pages_per_wave);
  const void* kern = nullptr;
  if (attend_mfma_supported(a.s)) {
    const bool pipe = a.pages_per_wave > 1;
    const int key = a.s.head_dim * 10000 + a.s.page_size * 100 + a.s.rank_v;
    switch (key) {
#define BKV_CASE(D, PS, R) \
  case D * 10000 + PS * 100 + R:                                                                          \
    kern = pipe ? (const void*)attend_mfma_kernel<D, PS, R, true, SEL> : (const void*)attend_mfma_kernel<D, PS, R, false, SEL>; \
    break;
      BKV_CASE(128, 64, 16) BKV_CASE(128, 64, 32) BKV_CASE(128, 64, 48) BKV_CASE(128, 64, 64)
      BKV_CASE(128, 32, 16) BKV_CASE(128, 32, 32) BKV_CASE(128, 32, 48) BKV_CASE(128, 32, 64)
      BKV_CASE(64, 64, 16) BKV_CASE(64, 64, 32) BKV_CASE(64, 64, 48) BKV_CASE(64, 64, 64)
      BKV_CASE(64, 32, 16) BKV_CASE(64, 32, 32) BKV_CASE(64, 32, 48) BKV_CASE(64, 32, 64)
#undef BKV_CASE
      default: return hipErrorInvalidValue;
    }
  } else if (a.s.dtype == 0) {
    kern = (const void*)attend_valu_kernel<float, SEL>;
  } else {
    kern = (const void*)attend_valu_kernel<uint16_t, SEL>;
  }
  hipError_t e = allow_lds(kern, lds);
  if (e != hipSuccess) return e;
  void* args[] = {const_cast<AttendArgs*>(&a)};
  return hipLaunchKernel(kern, grid, block, args, lds, st);
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  return a.scores ? launch_attend_t<true>(a, st) : launch_attend_t<false>(a, st);
}

size_t attend_lds_bytes(const Shape& s, bool select) {
  const AttendPlan p = plan_attend(s);
  size_t lds = attend_acc_bytes(p.waves, s.group, s.rank_v);
  if (select) lds += attend_sel_bytes(s.max_pages, p.waves, p.pages_per_wave);
  return lds;
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.s.batch * a.s.n_kv_heads), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bkv
