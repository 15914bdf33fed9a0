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
// P^T[key][row] with the channel-major latent page as the A operand.
//
// Long chunks split the key pages into ranges (blockIdx.z), so that the
// late queries' long walks run as several workgroups; each range leaves a
// partial (unnormalised latent sum, max, denominator) per row and a second
// launch merges them (split_merge.hpp), as the decode splits are merged.
//
// The four waves of a workgroup (64 rows: consecutive queries) walk the same
// pages of its range: each page's Keys and latents are copied once per workgroup straight
// into LDS (gfx950's direct global -> LDS loads, 16-byte granules permuted
// within each row so that the fragment reads spread over the banks), double-buffered: a
// wave reads page p's fragments into registers, then the copy of page p + 1
// is issued and runs while page p is multiplied.
#include <cstdlib>

#include "common.hpp"
#include "internal.hpp"
#include "split_merge.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr float NEG_INF = -__builtin_huge_valf();
// 16-row tiles per wave.  Two tiles share each fragment read but halve the
// workgroups: a 2048-query chunk of the 8K prompt then runs 128 workgroups
// on 256 CUs and measured 1208 against 1003 us per prompt.
constexpr int PREFILL_RT = 1;

// One page staged in LDS: the Keys [PS][D], then the latents [R][PS], each
// row's 16-byte granules permuted within the row by an XOR with a function
// of the row (its own inverse, so the copy uses the same map).  A 16-byte LDS
// read serves 16 lanes per pass from a 256-byte bank row; the fragment reads
// below put 16 different rows in a pass (Key rows 8a + b (+4), a, b < 4;
// latent rows 16t + n), and the maps send them to 16 different positions.
template <int D, int PS, int R>
struct PageLds {
  static constexpr int KG = D / 8, ZG = PS / 8;    // granules per Key row / latent row
  static constexpr int NK = PS * KG, NZ = R * ZG;  // granules of each part
  static constexpr int BYTES = 16 * (NK + NZ);
  static_assert(KG == 16 || KG == 8, "head_dim 128 or 64");
  static_assert(ZG == 8 || ZG == 4, "pages of 64 or 32");
  // position within Key row `tok` of its granule g (and the reverse)
  static __device__ __forceinline__ int kpos(int tok, int g) {
    if constexpr (KG == 16) return g ^ ((tok & 3) | (((tok >> 3) & 3) << 2));
    else return g ^ (((tok >> 1) & 1) | (((tok >> 3) & 3) << 1));  // two rows per bank row
  }
  // position within latent row `row` of its granule g (and the reverse)
  static __device__ __forceinline__ int zpos(int row, int g) {
    if constexpr (ZG == 8) return g ^ ((row >> 1) & 7);  // two rows per bank row
    else return g ^ ((row >> 2) & 3);                    // four rows per bank row
  }
  // copy one page (its Key block kp, latent block zp) into buf; every wave
  // of the workgroup takes its share of 64-granule blocks
  static __device__ __forceinline__ void stage(char* buf, const uint16_t* kp, const uint16_t* zp, int wave,
                                               int lane) {
    const char* K = reinterpret_cast<const char*>(kp);
    const char* Z = reinterpret_cast<const char*>(zp);
    const int first = dma_stage(
        buf, NK, [&](int G) { const int x = G / KG, j = G % KG; return K + 16 * (x * KG + kpos(x, j)); }, 0, 4,
        wave, lane);
    dma_stage(
        buf + 16 * NK, NZ, [&](int G) { const int x = G / ZG, j = G % ZG; return Z + 16 * (x * ZG + zpos(x, j)); },
        first, 4, wave, lane);
  }
};

template <int D, int PS, int R>
struct PageFrags {
  static constexpr int KS = D / 32, NC = PS / 32, MT = R / 16;
  bf16x8 k[NC][2][KS];
  bf16x8 z[NC][MT];
  // this lane's fragments of a page staged by PageLds
  __device__ __forceinline__ void load(const char* buf, int n, int qd) {
    using L = PageLds<D, PS, R>;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const int tok = 32 * c + 8 * (n >> 2) + 4 * t2 + (n & 3);
#pragma unroll
        for (int s = 0; s < KS; ++s)
          k[c][t2][s] = *reinterpret_cast<const bf16x8*>(buf + 16 * (tok * L::KG + L::kpos(tok, qd + 4 * s)));
      }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int row = 16 * t + n;
        z[c][t] = *reinterpret_cast<const bf16x8*>(buf + 16 * (L::NK + row * L::ZG + L::zpos(row, 4 * c + qd)));
      }
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

// RT row tiles of 16 per wave (a workgroup: 64 RT rows), every tile
// multiplied with the same page fragments, which are read from LDS once.
template <int D, int PS, int R, int RT>
__global__ __launch_bounds__(256) void prefill_mfma_kernel(PrefillArgs a) {
  using F = PageFrags<D, PS, R>;
  using L = PageLds<D, PS, R>;
  constexpr int KS = F::KS, NC = F::NC, MT = F::MT;
  constexpr int WROWS = 16 * RT, BROWS = 4 * WROWS;  // rows per wave, per workgroup
  extern __shared__ __attribute__((aligned(16))) char s_pages[];  // two staged pages
  const int G = a.s.group, H = a.s.n_kv_heads;
  const int g = blockIdx.y;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int rows = a.n_tok * G;
  const int wgi = gridDim.x - 1 - blockIdx.x;  // longest (latest) queries first
  const int w0 = wgi * BROWS + wave * WROWS;    // this wave's first row
  // a wave past the chunk's rows still copies and meets the barriers
  const bool wave_ok = w0 < rows;
  const int end = a.start + a.n_tok;  // tokens written in the cache
  // pages the workgroup walks (its last row's) and the pages this wave needs
  const int n_pages = (a.start + min(wgi * BROWS + BROWS - 1, rows - 1) / G) / PS + 1;
  const int my_pages = wave_ok ? (a.start + min(w0 + WROWS - 1, rows - 1) / G) / PS + 1 : 0;
  // this workgroup's key range: pages [p0, p1) (empty past its last page)
  const int split = blockIdx.z;
  const int p0 = split * a.split_pages, p1 = min(n_pages, p0 + a.split_pages);

  // tile i: rows w0 + 16 i + (0..15); this lane's row w0 + 16 i + n
  int qpos[RT], minpos[RT], maxpos[RT];
  bool row_ok[RT];
  bf16x8 qb[RT][KS];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const int r0 = w0 + 16 * i, rr = r0 + n;
    const int qi = rr / G, hh = rr % G;
    row_ok[i] = rr < rows;
    qpos[i] = a.start + qi;
    minpos[i] = a.start + r0 / G;
    maxpos[i] = r0 < rows ? a.start + min(r0 + 15, rows - 1) / G : -1;  // -1: the tile has no row
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         ((size_t)(row_ok[i] ? qi : 0) * a.s.n_q_heads + g * G + (row_ok[i] ? hh : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[i][s] = row_ok[i] ? load_bf16x8(qp + 8 * qd + 32 * s) : zero_bf16x8();
  }

  const uint16_t* Kp = static_cast<const uint16_t*>(a.K);
  const uint16_t* Zp = static_cast<const uint16_t*>(a.Z);
  const int32_t* pt = a.page_table + (size_t)a.seq * a.s.max_pages;

  float m_run[RT], l_run[RT];
  f32x4 acc[RT][MT];
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    m_run[i] = NEG_INF;
    l_run[i] = 0.f;
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto stage = [&](int pg, int phys) {
    L::stage(s_pages + (pg & 1) * L::BYTES, Kp + ((size_t)phys * H + g) * PS * D, Zp + ((size_t)phys * H + g) * R * PS,
             wave, lane);
  };
  if (p0 < p1) stage(p0, load_uniform(pt, p0));
  int phys_next = p0 + 1 < p1 ? load_uniform(pt, p0 + 1) : 0;
  for (int pg = p0; pg < p1; ++pg) {
    wait_vmem();    // this wave's copies of page pg are in
    lds_barrier();  // every wave's are, and page pg - 1's buffer is no longer read
    F cur;
    if (pg < my_pages) cur.load(s_pages + (pg & 1) * L::BYTES, n, qd);
    // the fragment reads are issued before the next copy into the other buffer
    __builtin_amdgcn_sched_barrier(0);
    if (pg + 1 < p1) {
      stage(pg + 1, phys_next);
      if (pg + 2 < p1) phys_next = load_uniform(pt, pg + 2);  // (scalar: no wait on the copies)
    }
    if (pg >= my_pages) continue;  // (wave-uniform)
    const int kbase = pg * PS;
    const int written = min(PS, end - kbase);  // slots holding data
    if (written < PS) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int valid = min(max(written - (32 * c + 8 * qd), 0), 8);
#pragma unroll
        for (int t = 0; t < MT; ++t) cur.z[c][t] = keep_first(cur.z[c][t], valid);
      }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
      if (kbase > maxpos[i]) continue;  // (wave-uniform) every key of the page is after the tile's queries
      float sv[NC][8];
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s)
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[c][t2][s], qb[i][s], s4, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[c][4 * t2 + e] = s4[e] * a.scale_log2;
        }
      if (kbase + PS - 1 > minpos[i]) {  // the diagonal: per-row causal limit
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!row_ok[i] || kbase + 32 * c + 8 * qd + e > qpos[i]) sv[c][e] = NEG_INF;
      }
      float mx = NEG_INF;
#pragma unroll
      for (int c = 0; c < NC; ++c)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, sv[c][e]);
      mx = pair_max<32>(pair_max<16>(mx));
      const float m_new = fmaxf(m_run[i], mx);
      // rows with nothing valid yet keep a zero state (their p below is 0)
      const float alpha = m_new == NEG_INF ? 1.f : exp2f(m_run[i] - m_new);
      m_run[i] = m_new;
      l_run[i] *= alpha;
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[i][t] *= alpha;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = m_new == NEG_INF ? 0.f : exp2f(sv[c][e] - m_new);
        // the weights enter the product rounded to bf16; the denominator sums
        // the same rounded values
        const bf16x8 pb = pack_bf16x8(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) l_run[i] += bf16x8_elem(pb, e);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.z[c][t], pb, acc[i][t], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < RT; ++i) {
    const float l = pair_sum<32>(pair_sum<16>(l_run[i]));
    if (wave_ok && row_ok[i]) {
      const int rr = w0 + 16 * i + n, qi = rr / G, hh = rr % G;
      const size_t prow = (size_t)qi * a.s.n_q_heads + g * G + hh;
      if (a.n_ksplit == 1) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        float* zo = a.z_out + prow * R;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) zo[16 * t + 4 * qd + e] = acc[i][t][e] * inv;
      } else {  // this range's partial (an empty range: max -inf, zero sums)
        const size_t ps_ = prow * a.n_ksplit + split;
        float* po = a.part_acc + ps_ * R;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) po[16 * t + 4 * qd + e] = acc[i][t][e];
        if (qd == 0) *reinterpret_cast<float2*>(a.part_ml + ps_ * 2) = make_float2(m_run[i], l);
      }
    }
  }
}

// The key ranges' partials of every (query, query head) row merged into z,
// four latent channels per thread.
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a) {
  const int R = a.s.rank_v, quads = R / 4;
  const size_t tasks = (size_t)a.n_tok * a.s.n_q_heads * quads;
  for (size_t t = (size_t)blockIdx.x * 256 + threadIdx.x; t < tasks; t += (size_t)gridDim.x * 256) {
    const size_t prow = t / quads;
    const int r0 = 4 * (int)(t % quads);
    const f32x4 z = merge_splits4(a.part_acc + prow * a.n_ksplit * R, a.part_ml + prow * a.n_ksplit * 2, a.n_ksplit,
                                  1, R, 0, r0);
    *reinterpret_cast<f32x4*>(a.z_out + prow * R + r0) = z;
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

void plan_prefill(const Shape& s, int start, int n_tok, int* n_ksplit, int* split_pages) {
  const int pages = (start + n_tok - 1) / s.page_size + 1;  // the chunk's last query's pages
  // 16 pages a range (8K prompt in chunks of 2048: 559 us per prompt, against
  // 570 with 32, 586 with 64 and 665 unsplit)
  int per = 16;
  if (const char* e = getenv("BASISKV_PREFILL_SPLIT_PAGES")) per = atoi(e) > 0 ? atoi(e) : per;
  int ns = prefill_mfma_supported(s) && n_tok > 0 ? (pages + per - 1) / per : 1;
  ns = ns < 1 ? 1 : (ns > PREFILL_KSPLIT_MAX ? PREFILL_KSPLIT_MAX : ns);
  *n_ksplit = ns;
  *split_pages = (pages + ns - 1) / ns;
}

bool prefill_mfma_supported(const Shape& s) {
  return s.dtype == 1 && (s.head_dim == 64 || s.head_dim == 128) &&
         (s.page_size == 32 || s.page_size == 64) && s.rank_v % 16 == 0 && s.rank_v <= 64;
}

hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t st) {
  if (a.n_tok <= 0) return hipSuccess;
  if (prefill_mfma_supported(a.s)) {
    const int rows = a.n_tok * a.s.group;
    const dim3 grid((rows + 64 * PREFILL_RT - 1) / (64 * PREFILL_RT), a.s.n_kv_heads, a.n_ksplit), block(256);
    const int key = a.s.head_dim * 10000 + a.s.page_size * 100 + a.s.rank_v;
    switch (key) {
#define BKV_CASE(D, PS, R)                                                                              \
  case D * 10000 + PS * 100 + R: {                                                                       \
    const size_t lds = 2 * (size_t)PageLds<D, PS, R>::BYTES;                                             \
    const hipError_t e = allow_lds((const void*)prefill_mfma_kernel<D, PS, R, PREFILL_RT>, lds);         \
    if (e != hipSuccess) return e;                                                                       \
    hipLaunchKernelGGL((prefill_mfma_kernel<D, PS, R, PREFILL_RT>), grid, block, lds, st, a);            \
  } break;
      BKV_CASE(128, 64, 16) BKV_CASE(128, 64, 32) BKV_CASE(128, 64, 48) BKV_CASE(128, 64, 64)
      BKV_CASE(128, 32, 16) BKV_CASE(128, 32, 32) BKV_CASE(128, 32, 48) BKV_CASE(128, 32, 64)
      BKV_CASE(64, 64, 16) BKV_CASE(64, 64, 32) BKV_CASE(64, 64, 48) BKV_CASE(64, 64, 64)
      BKV_CASE(64, 32, 16) BKV_CASE(64, 32, 32) BKV_CASE(64, 32, 48) BKV_CASE(64, 32, 64)
#undef BKV_CASE
      default: return hipErrorInvalidValue;
    }
    if (a.n_ksplit > 1) {
      const size_t tasks = (size_t)a.n_tok * a.s.n_q_heads * (a.s.rank_v / 4);
      const unsigned blocks = (unsigned)((tasks + 255) / 256 < 4096 ? (tasks + 255) / 256 : 4096);
      hipLaunchKernelGGL(prefill_merge_kernel, dim3(blocks), dim3(256), 0, st, a);
    }
  } else {
    const dim3 grid(a.n_tok, a.s.n_q_heads), block(256);
    if (a.s.dtype == 0) hipLaunchKernelGGL((prefill_valu_kernel<float>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((prefill_valu_kernel<uint16_t>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace bkv
