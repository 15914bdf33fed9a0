// Causal prefill attention over the paged cache: exact Keys for q.k, stored
// Value latents for the weighted sum (weekinpapers "BasisKV: Value Latents
// for Communication and Key Routing", Abstract; machinelearning.ru
// "KV-кэширование", "Фаза Prefill" and "Математическая формализация").  Every
// page up to the query is attended (no routing); a query at position p sees
// keys 0..p.
//
// Rows of the product are (query, query head of the group) pairs, head
// fastest, so the group's heads share each Key fragment.  A wave owns 16
// rows.  Per 32-key chunk S^T = K.Q^T runs on v_mfma_f32_16x16x32_bf16 with
// keys as rows (two tiles, row m <-> key 32c + 8*(m/4) + 4a + m%4) and the 16
// query rows as columns; each lane then holds 8 consecutive keys of one
// query row, which is the k-slice it supplies to O^T[r][row] += Z^T[r][key] .
// P^T[key][row] with the channel-major latent page as the A operand.  The
// next page's fragments are loaded while the current one is multiplied.
#include "common.hpp"
#include "internal.hpp"

namespace bkv {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();

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

template <int D, int PS, int R>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  using F = PageFrags<D, PS, R>;
  constexpr int KS = F::KS, NC = F::NC, MT = F::MT;
  const int G = a.s.group, H = a.s.n_kv_heads;
  const int g = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int rows = a.n_tok * G;
  const int wgi = gridDim.x - 1 - blockIdx.x;  // longest (latest) queries first
  const int r0 = wgi * 64 + wave * 16;
  if (r0 >= rows) return;
  const int rr = r0 + n;
  const int qi = rr / G, hh = rr % G;
  const bool row_ok = rr < rows;
  const int qpos = a.start + qi;  // this lane's query position
  const int last_row = min(r0 + 15, rows - 1);
  const int maxpos = a.start + last_row / G;
  const int minpos = a.start + r0 / G;
  const int end = a.start + a.n_tok;  // tokens written in the cache

  bf16x8 qb[KS];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         ((size_t)(row_ok ? qi : 0) * a.s.n_q_heads + g * G + hh) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = row_ok ? load_bf16x8(qp + 8 * qd + 32 * s) : zero_bf16x8();
  }

  const uint16_t* Kp = static_cast<const uint16_t*>(a.K);
  const uint16_t* Zp = static_cast<const uint16_t*>(a.Z);
  const int32_t* pt = a.page_table + (size_t)a.seq * a.s.max_pages;
  const int n_pages = maxpos / PS + 1;

  float m_run = NEG_INF, l_run = 0.f;
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  F cur, nxt;
  {
    const int phys = pt[0];
    cur.load(Kp + ((size_t)phys * H + g) * PS * D, Zp + ((size_t)phys * H + g) * R * PS, n, qd);
  }
  for (int pg = 0; pg < n_pages; ++pg) {
    if (pg + 1 < n_pages) {
      const int phys = pt[pg + 1];
      nxt.load(Kp + ((size_t)phys * H + g) * PS * D, Zp + ((size_t)phys * H + g) * R * PS, n, qd);
    }
    const int kbase = pg * PS;
    const int written = min(PS, end - kbase);  // slots holding data

    float sv[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
          s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[c][t2][s], qb[s], s4, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[c][4 * t2 + e] = s4[e] * a.scale_log2;
      }
    if (kbase + PS - 1 > minpos) {  // the diagonal: per-row causal limit
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (!row_ok || kbase + 32 * c + 8 * qd + e > qpos) sv[c][e] = NEG_INF;
    }
    if (written < PS) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int valid = min(max(written - (32 * c + 8 * qd), 0), 8);
#pragma unroll
        for (int t = 0; t < MT; ++t) cur.z[c][t] = keep_first(cur.z[c][t], valid);
      }
    }
    float mx = NEG_INF;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[c][e]);
    mx = pair_max<32>(pair_max<16>(mx));
    const float m_new = fmaxf(m_run, mx);
    // rows with nothing valid yet keep a zero state (their p below is 0)
    const float alpha = m_new == NEG_INF ? 1.f : exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] *= alpha;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = m_new == NEG_INF ? 0.f : exp2f(sv[c][e] - m_new);
      // the weights enter the product rounded to bf16; the denominator sums
      // the same rounded values
      const bf16x8 pb = pack_bf16x8(p);
#pragma unroll
      for (int e = 0; e < 8; ++e) l_run += bf16x8_elem(pb, e);
#pragma unroll
      for (int t = 0; t < MT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.z[c][t], pb, acc[t], 0, 0, 0);
    }
    if (pg + 1 < n_pages) cur = nxt;
  }

  l_run = pair_sum<32>(pair_sum<16>(l_run));
  if (row_ok) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* zo = a.z_out + ((size_t)qi * a.s.n_q_heads + g * G + hh) * R;
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) zo[16 * t + 4 * qd + e] = acc[t][e] * inv;
  }
}

// Plain VALU causal attention: one workgroup per (query, query head); lanes
// over keys for q.k, lanes over latent channels for the weighted sum.
template <typename T>
__global__ __launch_bounds__(256) void prefill_valu_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) float s_q[128];
  __shared__ __attribute__((aligned(16))) float s_red[256];
  __shared__ __attribute__((aligned(16))) float s_p[256];
  const int qi = blockIdx.x, h = blockIdx.y;
  const int G = a.s.group, H = a.s.n_kv_heads, D = a.s.head_dim, R = a.s.rank_v;
  const int PS = a.s.page_size;
  const int g = h / G;
  const int tid = threadIdx.x;
  const T* q = static_cast<const T*>(a.q);
  const T* Kp = static_cast<const T*>(a.K);
  const T* Zp = static_cast<const T*>(a.Z);
  for (int i = tid; i < D; i += 256) s_q[i] = ld_elem(q, ((size_t)qi * a.s.n_q_heads + h) * D + i);
  __syncthreads();
  const int len = a.start + qi + 1;
  const int32_t* pt = a.page_table + (size_t)a.seq * a.s.max_pages;
  float m_run = NEG_INF, l_run = 0.f, acc = 0.f;  // acc: channel tid (tid < R)
  for (int t0 = 0; t0 < len; t0 += 256) {
    const int t = t0 + tid;
    float s = NEG_INF;
    if (t < len) {
      const int phys = pt[t / PS];
      const size_t kb = (((size_t)phys * H + g) * PS + t % PS) * D;
      float d = 0.f;
      for (int i = 0; i < D; ++i) d += s_q[i] * ld_elem(Kp, kb + i);
      s = d * a.scale_log2;
    }
    s_red[tid] = s;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) s_red[tid] = fmaxf(s_red[tid], s_red[tid + o]);
      __syncthreads();
    }
    const float m_new = fmaxf(m_run, s_red[0]);
    __syncthreads();
    const float alpha = exp2f(m_run - m_new);
    const float p = t < len ? exp2f(s - m_new) : 0.f;
    s_p[tid] = p;
    s_red[tid] = p;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
      if (tid < o) s_red[tid] += s_red[tid + o];
      __syncthreads();
    }
    l_run = l_run * alpha + s_red[0];
    m_run = m_new;
    if (tid < R) {
      float z = 0.f;
      const int nt = min(256, len - t0);
      for (int u = 0; u < nt; ++u) {
        const int tt = t0 + u;
        const int phys = pt[tt / PS];
        z += s_p[u] * ld_elem(Zp, (((size_t)phys * H + g) * R + tid) * PS + tt % PS);
      }
      acc = acc * alpha + z;
    }
    __syncthreads();
  }
  if (tid < R) a.z_out[((size_t)qi * a.s.n_q_heads + h) * R + tid] = acc / l_run;
}

}  // namespace

bool prefill_mfma_supported(const Shape& s) {
  return s.dtype == 1 && (s.head_dim == 64 || s.head_dim == 128) &&
         (s.page_size == 32 || s.page_size == 64) && s.rank_v % 16 == 0 && s.rank_v <= 64;
}

hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  if (prefill_mfma_supported(a.s)) {
    const int rows = a.n_tok * a.s.group;
    const dim3 grid((rows + 63) / 64, a.s.n_kv_heads), block(256);
    const int key = a.s.head_dim * 10000 + a.s.page_size * 100 + a.s.rank_v;
    switch (key) {
#define BKV_CASE(D, PS, R) \
  case D * 10000 + PS * 100 + R: hipLaunchKernelGGL((prefill_mfma_kernel<D, PS, R>), grid, block, 0, st, a); break;
      BKV_CASE(128, 64, 16) BKV_CASE(128, 64, 32) BKV_CASE(128, 64, 48) BKV_CASE(128, 64, 64)
      BKV_CASE(128, 32, 16) BKV_CASE(128, 32, 32) BKV_CASE(128, 32, 48) BKV_CASE(128, 32, 64)
      BKV_CASE(64, 64, 16) BKV_CASE(64, 64, 32) BKV_CASE(64, 64, 48) BKV_CASE(64, 64, 64)
      BKV_CASE(64, 32, 16) BKV_CASE(64, 32, 32) BKV_CASE(64, 32, 48) BKV_CASE(64, 32, 64)
#undef BKV_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    const dim3 grid(a.n_tok, a.s.n_q_heads), block(256);
    if (a.s.dtype == 0) hipLaunchKernelGGL((prefill_valu_kernel<float>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((prefill_valu_kernel<uint16_t>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace bkv
