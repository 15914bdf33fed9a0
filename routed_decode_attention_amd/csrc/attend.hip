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

#include "common.hpp"
#include "internal.hpp"
#include "split_merge.hpp"

namespace bkv {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

struct WaveState {  // LDS image of every wave's online-softmax state
  float m[ATTEND_WAVES_MAX][MAX_GROUP];
  float l[ATTEND_WAVES_MAX][MAX_GROUP];
};
// ... and of their latent accumulators: dynamic LDS [waves][group][rank_v]
__device__ __forceinline__ float& acc_at(float* acc, int w, int h, int r, int G, int R) {
  return acc[(w * G + h) * R + r];
}

// Merge the workgroup's waves into one partial per query head: plain stores
// of (acc, m, l), or the normalised latent when the pair has one split.
__device__ void finish_split(const AttendArgs& a, WaveState& ws, float* wacc, int pair, int split) {
  const int G = a.s.group, R = a.s.rank_v;
  const int tid = threadIdx.x;
  __syncthreads();
  const bool single = a.n_wsplit == 1 && a.z_out != nullptr;
  const int b = pair / a.s.n_kv_heads, g = pair % a.s.n_kv_heads;
  const size_t ps = (size_t)pair * a.n_wsplit + split;
  for (int o = tid; o < G * R; o += blockDim.x) {
    const int h = o / R, r = o % R;
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < ATTEND_WAVES_MAX; ++w)
      if (w < a.waves) M = fmaxf(M, ws.m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != NEG_INF) {
#pragma unroll
      for (int w = 0; w < ATTEND_WAVES_MAX; ++w)
        if (w < a.waves) {
          const float e = exp2f(ws.m[w][h] - M);
          L += e * ws.l[w][h];
          A += e * acc_at(wacc, w, h, r, G, R);
        }
    }
    if (single) {
      a.z_out[((size_t)b * a.s.n_q_heads + g * G + h) * R + r] = L > 0.f ? A / L : 0.f;
    } else {
      a.part_acc[(ps * G + h) * R + r] = A;
      if (r == 0) *reinterpret_cast<float2*>(a.part_ml + (ps * G + h) * 2) = make_float2(M, L);
    }
  }
}

// Zero the bf16 elements j of v whose index is >= valid (0 <= valid <= 8).
__device__ __forceinline__ bf16x8 keep_first(bf16x8 v, int valid) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = (2 * e < valid) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * e + 1 < valid) ? 0xffff0000u : 0u;
    u[e] &= (lo | hi);
  }
  return __builtin_bit_cast(bf16x8, u);
}

// One page's MFMA operands for this lane.
template <int D, int PS, int R>
struct PageFrags {
  static constexpr int KS = D / 32, NC = PS / 32, MT = R / 16;
  bf16x8 k[NC][2][KS];
  bf16x8 z[NC][MT];
  __device__ __forceinline__ void load(const uint16_t* kp, const uint16_t* zp, int n, int qd) {
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int tok = 32 * c + 8 * (n >> 2) + 4 * t2 + (n & 3);
#pragma unroll
        for (int s = 0; s < KS; ++s) k[c][t2][s] = load_bf16x8(kp + tok * D + 8 * qd + 32 * s);
      }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) z[c][t] = load_bf16x8(zp + (16 * t + n) * PS + 32 * c + 8 * qd);
  }
};

template <int D, int PS, int R>
struct OnlineSoftmax {
  static constexpr int KS = D / 32, NC = PS / 32, MT = R / 16;
  float m = NEG_INF, l = 0.f;
  f32x4 acc[MT];
  __device__ __forceinline__ OnlineSoftmax() {
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Fold one page (cnt valid tokens) into the state.
  __device__ __forceinline__ void page(PageFrags<D, PS, R>& f, const bf16x8 (&qb)[KS], int cnt, int qd,
                                       float scale_log2) {
    float sv[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.k[c][t2][s], qb[s], s4, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[c][4 * t2 + e] = s4[e] * scale_log2;
      }
    if (cnt < PS) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int valid = min(max(cnt - (32 * c + 8 * qd), 0), 8);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= valid) sv[c][e] = NEG_INF;
#pragma unroll
        for (int t = 0; t < MT; ++t) f.z[c][t] = keep_first(f.z[c][t], valid);
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[c][e]);
    mx = pair_max<32>(pair_max<16>(mx));
    const float m_new = fmaxf(m, mx);
    if (m_new == NEG_INF) return;  // wave-uniform: no valid token so far
    const float alpha = exp2f(m - m_new);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = exp2f(sv[c][e] - m_new);
      // the weights enter the product rounded to bf16; the denominator sums
      // the same rounded values
      const bf16x8 pb = pack_bf16x8(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) l += bf16x8_elem(pb, e);
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.z[c][t], pb, acc[t], 0, 0, 0);
    }
  }
};

template <int D, int PS, int R, bool PIPE>
__global__ __launch_bounds__(64 * ATTEND_WAVES_MAX) void attend_mfma_kernel(AttendArgs a) {
  constexpr int KS = D / 32, MT = R / 16;
  __shared__ WaveState st;
  extern __shared__ __attribute__((aligned(16))) float s_acc[];

  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int pair = wg / a.n_wsplit, split = wg % a.n_wsplit;
  const int H = a.s.n_kv_heads, G = a.s.group;
  const int b = pair / H, g = pair % H;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;

  const int first = (split * a.waves + wave) * a.pages_per_wave;
  // this wave's slice of the selection is read in the same round trip as the
  // sequence length and the selection count (every slot < top_k is in bounds;
  // slots past the count are masked below)
  int my_j = 0, my_phys = 0;
  const bool in_list = lane < a.pages_per_wave && first + lane < a.s.top_k;
  if (in_list) {
    const size_t at = (size_t)pair * a.s.top_k + first + lane;
    my_j = a.sel[at];
    if (a.sel_phys) my_phys = a.sel_phys[at];
  }
  const int seq_len = a.seq_lens[b];
  const int nsel = seq_len > 0 ? a.n_sel[pair] : 0;
  const int np = max(0, min(first + a.pages_per_wave, nsel) - first);  // pages of this wave
  // page ids and valid-token counts of this wave's pages, lane u holds page u
  int my_cnt = 0;
  if (lane < np) {
    if (!a.sel_phys) my_phys = a.page_table[(size_t)b * a.s.max_pages + my_j];
    my_cnt = min(PS, seq_len - my_j * PS);
  } else {
    my_phys = 0;
  }
  bf16x8 qb[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         ((size_t)b * a.s.n_q_heads + g * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = n < G ? load_bf16x8(qp + 8 * qd + 32 * s) : zero_bf16x8();
  }
  const uint16_t* Kp = static_cast<const uint16_t*>(a.K);
  const uint16_t* Zp = static_cast<const uint16_t*>(a.Z);
  auto kpage = [&](int u) {
    const int phys = __builtin_amdgcn_readlane(my_phys, u);
    return Kp + ((size_t)phys * H + g) * PS * D;
  };
  auto zpage = [&](int u) {
    const int phys = __builtin_amdgcn_readlane(my_phys, u);
    return Zp + ((size_t)phys * H + g) * R * PS;
  };

  OnlineSoftmax<D, PS, R> os;
  if (PIPE) {  // several pages per wave: the next page's loads overlap this page's math
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
template <typename T>
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
  const int nsel = seq_len > 0 ? a.n_sel[pair] : 0;
  const int first = (split * a.waves + wave) * a.pages_per_wave;
  const int last = min(first + a.pages_per_wave, nsel);

  float m_run[MAX_GROUP], l_run[MAX_GROUP], acc[MAX_GROUP];
  for (int h = 0; h < MAX_GROUP; ++h) {
    m_run[h] = NEG_INF;
    l_run[h] = 0.f;
    acc[h] = 0.f;
  }
  for (int i = first; i < last; ++i) {
    const int j = a.sel[(size_t)pair * a.s.top_k + i];
    const int phys = a.page_table[(size_t)b * a.s.max_pages + j];
    const int cnt = min(PS, seq_len - j * PS);
    const size_t kbase = ((size_t)phys * H + g) * PS * D;
    const size_t zbase = ((size_t)phys * H + g) * R * PS;
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
  // About 16 waves per CU over 256 CUs once every page unit is counted.
  const long units = (long)s.batch * s.n_kv_heads * s.top_k;
  int ppw = (int)((units + 4095) / 4096);
  if (ppw < 1) ppw = 1;
  if (ppw > 8) ppw = 8;
  const char* env = getenv("BASISKV_PAGES_PER_WAVE");
  if (env && atoi(env) > 0) ppw = atoi(env) < 32 ? atoi(env) : 32;
  // Four waves per workgroup; eight when four would leave more splits than
  // the merge requests in one round (their merge then costs a second round
  // trip: at top_k 128, 16 splits of 8 waves measured faster than 32 of 4,
  // while at top_k 64 the 16 splits of 4 waves are faster).
  int waves = (s.top_k + 4 * ppw - 1) / (4 * ppw) > MERGE_CHUNK ? 8 : 4;
  const char* wenv = getenv("BASISKV_ATTEND_WAVES");
  if (wenv && (atoi(wenv) == 4 || atoi(wenv) == 8)) waves = atoi(wenv);
  AttendPlan p;
  p.pages_per_wave = ppw;
  p.waves = waves;
  p.n_wsplit = (s.top_k + waves * ppw - 1) / (waves * ppw);
  return p;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t st) {
  const int pairs = a.s.batch * a.s.n_kv_heads;
  const dim3 grid(pairs * a.n_wsplit), block(64 * a.waves);
  const size_t lds = (size_t)a.waves * a.s.group * a.s.rank_v * sizeof(float);
  if (attend_mfma_supported(a.s)) {
    const bool pipe = a.pages_per_wave > 1;
    const int key = a.s.head_dim * 10000 + a.s.page_size * 100 + a.s.rank_v;
    switch (key) {
#define BKV_CASE(D, PS, R) \
  case D * 10000 + PS * 100 + R:                                                                 \
    if (pipe) hipLaunchKernelGGL((attend_mfma_kernel<D, PS, R, true>), grid, block, lds, st, a);   \
    else hipLaunchKernelGGL((attend_mfma_kernel<D, PS, R, false>), grid, block, lds, st, a);       \
    break;
      BKV_CASE(128, 64, 16) BKV_CASE(128, 64, 32) BKV_CASE(128, 64, 48) BKV_CASE(128, 64, 64)
      BKV_CASE(128, 32, 16) BKV_CASE(128, 32, 32) BKV_CASE(128, 32, 48) BKV_CASE(128, 32, 64)
      BKV_CASE(64, 64, 16) BKV_CASE(64, 64, 32) BKV_CASE(64, 64, 48) BKV_CASE(64, 64, 64)
      BKV_CASE(64, 32, 16) BKV_CASE(64, 32, 32) BKV_CASE(64, 32, 48) BKV_CASE(64, 32, 64)
#undef BKV_CASE
      default: return hipErrorInvalidValue;
    }
  } else if (a.s.dtype == 0) {
    hipLaunchKernelGGL((attend_valu_kernel<float>), grid, block, lds, st, a);
  } else {
    hipLaunchKernelGGL((attend_valu_kernel<uint16_t>), grid, block, lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.s.batch * a.s.n_kv_heads), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bkv
