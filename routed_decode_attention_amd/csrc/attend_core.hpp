// Device pieces of the gathered exact-QK decode attention shared by its
// kernels: the workgroup's LDS state and split partials, the second half of
// the prologue selection, one page's matrix-core operands and the online
// softmax over them (see attend.hip for the scheme).
#pragma once

#include "common.hpp"
#include "internal.hpp"
#include "select.hpp"

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

// Dynamic LDS of a workgroup that selects its pages itself: after the
// waves' latent accumulators, the pair's keys and page-table row, this
// workgroup's share of the selection (logical and physical ids) and the
// selection's scratch.
struct SelLds {
  SelectPages pg;
  int32_t *pt, *mine_j, *mine_p;
  SelectShared* sh;
};
__host__ __device__ inline size_t attend_acc_bytes(int waves, int G, int R) {
  return ((size_t)waves * G * R * sizeof(float) + 15) & ~(size_t)15;
}
__host__ __device__ inline size_t sel_a16(size_t x) { return (x + 15) & ~(size_t)15; }
// keys and page-table row (4 bytes a page each), bins and picks (a byte each)
__host__ __device__ inline size_t sel_page_bytes(int maxp) { return 2 * sel_a16((size_t)maxp * 4) + sel_a16((size_t)maxp * 2); }
__host__ __device__ inline size_t attend_sel_bytes(int maxp, int waves, int ppw) {
  return sel_page_bytes(maxp) + sel_a16((size_t)waves * ppw * 8) + sizeof(SelectShared);
}
__device__ inline SelLds sel_lds(float* dyn, int waves, int G, int R, int maxp, int ppw) {
  char* p = reinterpret_cast<char*>(dyn) + attend_acc_bytes(waves, G, R);
  const size_t kb = sel_a16((size_t)maxp * 4);
  SelLds L;
  L.pg.keys = reinterpret_cast<uint32_t*>(p);
  L.pt = reinterpret_cast<int32_t*>(p + kb);
  L.pg.bin = reinterpret_cast<uint8_t*>(p + 2 * kb);
  L.pg.pick = L.pg.bin + maxp;
  L.mine_j = reinterpret_cast<int32_t*>(p + sel_page_bytes(maxp));
  L.mine_p = L.mine_j + waves * ppw;
  L.sh = reinterpret_cast<SelectShared*>(p + sel_page_bytes(maxp) + sel_a16((size_t)waves * ppw * 8));
  return L;
}

// The selection's second half, shared by the prologue selections: with the
// pair's keys and page-table row in LDS (pages [0, npg)) and this thread's
// (max, min) over the keys of the pages that are not forced, rank the pages
// (select.hpp) and keep the positions [split * waves * ppw, +waves * ppw) of
// the selection in page order with their physical ids; split 0 also writes
// the selection (sel_out, n_sel_out).  Returns the selection count.
__device__ inline int select_tail(const AttendArgs& a, int pair, int split, const SelLds& L, int npg, uint32_t kmax,
                                  uint32_t kmin) {
  const int top_k = a.s.top_k;
  const int ks = min(top_k, npg);
  int32_t* sel = a.sel_out + (size_t)pair * top_k;
  if (split == 0) {
    for (int p = ks + threadIdx.x; p < top_k; p += blockDim.x) sel[p] = -1;
    if (threadIdx.x == 0) a.n_sel_out[pair] = ks;
  }
  if (ks == 0) return 0;
  key_range_publish(kmax, kmin, *L.sh);
  topk_clear(*L.sh);
  lds_barrier();
  const TopK t = topk_find(L.pg, npg, ks, *L.sh);
  const int base = split * a.waves * a.pages_per_wave, cnt = a.waves * a.pages_per_wave;
  auto put = [&](int p, int j) {
    if (p >= ks) return;  // (never: the selection keeps exactly ks pages)
    if (split == 0) sel[p] = j;
    if (p >= base && p < base + cnt) {
      L.mine_j[p - base] = j;
      L.mine_p[p - base] = L.pt[j];
    }
  };
  if (t.mode == 2) topk_emit(L.pg, npg, t, *L.sh, put);
  else topk_emit_masked(L.pg, npg, t, *L.sh, put);
  lds_barrier();
  return ks;
}

// Merge the workgroup's waves into one partial per query head: plain stores
// of (acc, m, l), or the normalised latent when the pair has one split.
__device__ inline void finish_split(const AttendArgs& a, WaveState& ws, float* wacc, int pair, int split) {
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
}  // namespace

}  // namespace bkv
