// Top-k page selection of one (sequence, KV head) by one workgroup.
//
// weekinpapers "BasisKV: Value Latents for Communication and Key Routing",
// Abstract: the router identifies which Key pages are read; the exact Keys
// are then retrieved only for those.  The min(top_k, n_pg) pages with the
// highest group scores are kept; equal scores go to the smaller logical page;
// the selection is listed in ascending page order.  Pages forced by
// sink_pages / local_pages rank above every score.
//
// The pages arrive as order-preserving 32-bit keys in LDS (larger score,
// larger key; -0 folded onto +0; 0xFFFFFFFF marks a forced page).  The
// selection is exact, in three steps:
//   1. bins: 255 equal-width bins between the smallest and the largest score
//      (bin 255 for forced pages).  Binning is monotone in the score (fp
//      subtraction and multiplication by a positive constant round
//      monotonically), so every page of a higher bin outranks every page of a
//      lower one; per-wave histograms (one barrier) and a scan from the top
//      find the boundary bin holding the k-th page.
//   2. the boundary bin's pages (a handful for spread-out scores) are ranked
//      among themselves by (key, page); the first ones still needed are kept.
//      Scores crowded into one bin (more pages than SEL_CAND) fall back to an
//      MSB-first radix cut over the keys (8-bit digits, per-wave histograms).
//   3. every thread counts the kept pages of a run of consecutive pages; a
//      workgroup prefix sum gives each run its first position, and each kept
//      page is emitted with its position in page order (for the bins' cut:
//      per-wave ballot masks and popcount prefixes instead).
// Every barrier orders LDS only, so global loads issued before the selection
// stay in flight.
#pragma once

#include "common.hpp"

namespace bkv {

constexpr int SEL_MAXW = 8;    // waves per selecting workgroup (4 or 8)
constexpr int SEL_CAND = 512;  // boundary-bin pages ranked directly
constexpr int SEL_SB = 8;      // strides of scores a thread requests together

// LDS the selection needs beside the per-page arrays (16-byte aligned: the
// histograms are cleared and read 16 bytes at a time).  The radix fallback's
// two histogram buffers reuse the bins' histograms and the candidate list.
struct __attribute__((aligned(16))) SelectShared {
  int area[2][SEL_MAXW][256];  // [0]: bin histograms; [1]: candidate keys and pages
  uint32_t red[SEL_MAXW][2];
  uint32_t scan[SEL_MAXW];
  uint32_t ncand;
};

// Per-page LDS arrays of the selection.
struct SelectPages {
  uint32_t* keys;  // [nk] order-preserving keys
  uint8_t* bin;    // [nk] bin of each page
  uint8_t* pick;   // [nk] kept among the boundary bin's pages
};

// Order-preserving map of a score (forced: above every score).
__device__ __forceinline__ uint32_t select_key(float score, bool forced) {
  return forced ? 0xFFFFFFFFu : float_key(score);
}
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Wave-wide max / min (every lane gets the result): DPP within rows of 16,
// gfx950's lane-half swaps across them.
#define BKV_DPPU(x, ctrl) (uint32_t) __builtin_amdgcn_mov_dpp((int)(x), ctrl, 0xF, 0xF, false)
template <bool MAX>
__device__ __forceinline__ uint32_t sel_wave_ext(uint32_t x) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  x = op(x, BKV_DPPU(x, 0xB1));   // quad_perm [1,0,3,2]
  x = op(x, BKV_DPPU(x, 0x4E));   // quad_perm [2,3,0,1]
  x = op(x, BKV_DPPU(x, 0x124));  // row_ror:4
  x = op(x, BKV_DPPU(x, 0x128));  // row_ror:8
  auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return op(r[0], r[1]);
}
#undef BKV_DPPU

// The key range, in two halves around a barrier the caller provides: each
// wave reduces its threads' (max, min) and publishes it; after the barrier
// every thread reads the workgroup's.
__device__ inline void key_range_publish(uint32_t kmax, uint32_t kmin, SelectShared& sh) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  kmax = sel_wave_ext<true>(kmax);
  kmin = sel_wave_ext<false>(kmin);
  if (lane == 0) {
    sh.red[wave][0] = kmax;
    sh.red[wave][1] = kmin;
  }
}
__device__ inline void key_range_read(const SelectShared& sh, uint32_t& kmax, uint32_t& kmin) {
  const int nw = blockDim.x >> 6;
  kmax = 0u;
  kmin = 0xffffffffu;
  for (int w = 0; w < nw; ++w) {
    kmax = max(kmax, sh.red[w][0]);
    kmin = min(kmin, sh.red[w][1]);
  }
}
// Largest and smallest key (forced pages aside when skip_forced), whole workgroup.
__device__ inline void key_range(const uint32_t* keys, int nk, bool skip_forced, SelectShared& sh, uint32_t& kmax,
                                 uint32_t& kmin) {
  const int tid = threadIdx.x, nt = blockDim.x;
  uint32_t hi = 0u, lo = 0xffffffffu;
  for (int j = tid; j < nk; j += nt) {
    const uint32_t k = keys[j];
    if (skip_forced && k == 0xFFFFFFFFu) continue;
    hi = max(hi, k);
    lo = min(lo, k);
  }
  key_range_publish(hi, lo, sh);
  lds_barrier();
  key_range_read(sh, kmax, kmin);
}

struct TopKCut {  // radix fallback: kept = (key & mask) > prefix, or == prefix among the first take_eq
  uint32_t prefix, mask;
  int take_eq;
};

struct TopK {
  int mode;     // 0: every page kept; 1: bins; 2: radix cut
  int bstar;    // boundary bin
  int all_b;    // every page of the boundary bin kept
  TopKCut cut;
};

// The radix cut of the ks best keys among keys[0, nk) (0 < ks < nk).
__device__ inline TopKCut radix_cut(const uint32_t* keys, int nk, int ks, SelectShared& sh) {
  const int tid = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  uint32_t kmax, kmin;
  lds_barrier();  // sh.red may still be read by the bins' range
  key_range(keys, nk, false, sh, kmax, kmin);
  const uint32_t diff = kmax ^ kmin;
  int hi = diff ? 31 - __builtin_clz(diff) : -1;
  uint32_t mask = hi >= 0 ? ~((2u << hi) - 1u) : ~0u;
  uint32_t prefix = kmax & mask;
  int krem = ks;
  for (int pass = 0; hi >= 0; ++pass) {
    int* hb = &sh.area[pass & 1][0][0];
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (2u << (hi - shift)) - 1u;  // digit bits [shift, hi]
    *reinterpret_cast<int4*>(hb + wave * 256 + 4 * lane) = int4{0, 0, 0, 0};
    __builtin_amdgcn_wave_barrier();
    for (int j = tid; j < nk; j += nt) {
      const uint32_t key = keys[j];
      if ((key & mask) == prefix) atomicAdd(hb + wave * 256 + ((key >> shift) & dmask), 1);
    }
    lds_barrier();
    // lane owns digits 255-4*lane .. 252-4*lane (descending)
    int cd[4] = {0, 0, 0, 0};
    for (int w = 0; w < nw; ++w) {
      const int4 h4 = *reinterpret_cast<const int4*>(hb + w * 256 + 252 - 4 * lane);
      cd[0] += h4.w;
      cd[1] += h4.z;
      cd[2] += h4.y;
      cd[3] += h4.x;
    }
    const int owns = cd[0] + cd[1] + cd[2] + cd[3];
    int run = wave_incl_scan(owns) - owns;  // keys with a larger digit than this lane's
    int digit = 0, nrem = 0, done = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (run < krem && run + cd[u] >= krem) {
        digit = 255 - 4 * lane - u;
        nrem = krem - run;
        done = cd[u] == krem - run;
      }
      run += cd[u];
    }
    const unsigned long long hit = __ballot(nrem > 0);
    const int src = __ffsll((long long)hit) - 1;
    digit = __builtin_amdgcn_readlane(digit, src);
    krem = __builtin_amdgcn_readlane(nrem, src);
    done = __builtin_amdgcn_readlane(done, src);
    prefix |= (uint32_t)digit << shift;
    mask |= dmask << shift;
    if (done || shift == 0) break;
    hi = shift - 1;
  }
  return TopKCut{prefix, mask, krem};
}

// Every wave clears its row of the bins' histograms (and thread 0 the
// candidate count); call before the barrier that precedes topk_find.
__device__ inline void topk_clear(SelectShared& sh) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  *reinterpret_cast<int4*>(&sh.area[0][wave][4 * lane]) = int4{0, 0, 0, 0};
  if (tid == 0) sh.ncand = 0u;
}

// Find which of pages [0, nk) the ks best are (0 < ks), whole workgroup.
// Before the call the caller has written the keys, cleared the histograms
// (topk_clear), published the range of the keys of pages that are not forced
// (key_range_publish), and passed an LDS barrier.
__device__ inline TopK topk_find(const SelectPages& pg, int nk, int ks, SelectShared& sh) {
  const int tid = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  TopK t{0, 0, 0, TopKCut{0u, 0u, 0}};
  if (ks >= nk) return t;
  int* hist = &sh.area[0][0][0];
  // 1. the scores' range, forced pages aside (keys order like scores)
  uint32_t kmax, kmin;
  key_range_read(sh, kmax, kmin);
  float lo = 0.f, scale = 0.f;
  if (kmin <= kmax) {
    lo = key_score(kmin);
    const float hi = key_score(kmax);
    scale = hi > lo ? 254.f / (hi - lo) : 0.f;
  }
  // 2. bins (monotone in the score) and per-wave histograms
  for (int j = tid; j < nk; j += nt) {
    const uint32_t k = pg.keys[j];
    int b = 255;
    if (k != 0xFFFFFFFFu) b = (int)fminf(fmaxf((key_score(k) - lo) * scale, 0.f), 254.f);
    pg.bin[j] = (uint8_t)b;
    atomicAdd(hist + wave * 256 + b, 1);
  }
  lds_barrier();
  // 3. the boundary bin, scanning from the top: lane owns bins 255-4*lane .. 252-4*lane
  int cd[4] = {0, 0, 0, 0};
  for (int w = 0; w < nw; ++w) {
    const int4 h4 = *reinterpret_cast<const int4*>(hist + w * 256 + 252 - 4 * lane);
    cd[0] += h4.w;
    cd[1] += h4.z;
    cd[2] += h4.y;
    cd[3] += h4.x;
  }
  const int owns = cd[0] + cd[1] + cd[2] + cd[3];
  int run = wave_incl_scan(owns) - owns;  // pages in higher bins than this lane's
  int bst = 0, nrem = 0, nin = 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    if (run < ks && run + cd[u] >= ks) {
      bst = 255 - 4 * lane - u;
      nrem = ks - run;
      nin = cd[u];
    }
    run += cd[u];
  }
  const unsigned long long hit = __ballot(nrem > 0);
  const int src = __ffsll((long long)hit) - 1;
  t.bstar = __builtin_amdgcn_readlane(bst, src);
  const int krem = __builtin_amdgcn_readlane(nrem, src);
  const int nb = __builtin_amdgcn_readlane(nin, src);
  t.mode = 1;
  t.all_b = krem == nb;
  if (t.all_b) return t;
  if (nb > SEL_CAND) {  // crowded scores: the radix cut over all keys
    t.mode = 2;
    t.cut = radix_cut(pg.keys, nk, ks, sh);
    return t;
  }
  // 4. the boundary bin's pages, ranked among themselves by (key, page): as
  // 64-bit values key << 32 | ~page, of which a larger one ranks higher
  // (the count was cleared by topk_clear)
  uint64_t* cand = reinterpret_cast<uint64_t*>(&sh.area[1][0][0]);
  for (int j = tid; j < nk; j += nt)
    if (pg.bin[j] == t.bstar) {
      const uint32_t c = atomicAdd(&sh.ncand, 1u);
      cand[c] = (uint64_t)pg.keys[j] << 32 | (uint32_t)~j;
    }
  if (tid < 2) cand[nb + tid] = 0u;  // pads the list to pairs (the area holds 1024); 0 ranks below every page
  lds_barrier();
  for (int c = tid; c < nb; c += nt) {
    const uint64_t kc = cand[c];
    int rank = 0;
    // two candidates per 16-byte read, several reads in flight
#pragma unroll 4
    for (int d = 0; d < nb; d += 2) {
      const ulonglong2 two = *reinterpret_cast<const ulonglong2*>(cand + d);
      rank += (two.x > kc) + (two.y > kc);
    }
    pg.pick[(int)~(uint32_t)kc] = rank < krem;
  }
  lds_barrier();
  return t;
}

// Emit (position, page) for every kept page of [0, nk), positions in page
// order; whole workgroup.  emit may be called from any thread.
template <typename Emit>
__device__ inline void topk_emit(const SelectPages& pg, int nk, const TopK& t, SelectShared& sh, Emit&& emit) {
  const int tid = threadIdx.x, nt = blockDim.x, nw = nt >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int run = (nk + nt - 1) / nt;  // consecutive pages per thread
  const int j0 = min(nk, tid * run), j1 = min(nk, j0 + run);
  // kept pages (g) and, for the radix cut, pages equal to its prefix (e)
  auto classify = [&](int j, bool& g, bool& e) {
    if (t.mode == 0) {
      g = true;
      e = false;
    } else if (t.mode == 1) {
      const int b = pg.bin[j];
      g = b > t.bstar || (b == t.bstar && (t.all_b || pg.pick[j]));
      e = false;
    } else {
      const uint32_t mk = pg.keys[j] & t.cut.mask;
      g = mk > t.cut.prefix;
      e = mk == t.cut.prefix;
    }
  };
  uint32_t gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    bool g, e;
    classify(j, g, e);
    gt += g;
    eq += e;
  }
  // workgroup exclusive prefix sum of (gt, eq) packed in 16-bit halves (nk <= 8192)
  const uint32_t packed = gt | eq << 16;
  const uint32_t incl = (uint32_t)wave_incl_scan((int)packed);
  if (lane == 63) sh.scan[wave] = incl;
  lds_barrier();
  uint32_t before = incl - packed;
  for (int w = 0; w < nw; ++w)
    if (w < wave) before += sh.scan[w];
  int gt_before = (int)(before & 0xffffu), eq_before = (int)(before >> 16);
  const int take_eq = t.mode == 2 ? t.cut.take_eq : 0;
  for (int j = j0; j < j1; ++j) {
    bool g, e;
    classify(j, g, e);
    if (g || (e && eq_before < take_eq)) emit(gt_before + min(eq_before, take_eq), j);
    gt_before += g;
    eq_before += e;
  }
}

// Emit as topk_emit does, for the bins' cut (modes 0 and 1), through
// per-wave ballot masks: page j is classified by thread j mod the workgroup
// size, each wave's kept bits for one stride of pages form a 64-bit word in
// LDS, and after one barrier a kept page's position is the kept count of the
// words before its own (a scan over at most 128 words that every wave does
// for itself) plus the kept lanes below it in its word.
template <typename Emit>
__device__ inline void topk_emit_masked(const SelectPages& pg, int nk, const TopK& t, SelectShared& sh, Emit&& emit) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  // the candidate list's area is free once the cut is found: 8 KiB, 1024 words
  uint64_t* words = reinterpret_cast<uint64_t*>(&sh.area[1][0][0]);
  const int nwords = (nk + 63) / 64;
  for (int j0 = 0; j0 < nk; j0 += nt) {
    const int j = j0 + tid;
    bool g = false;
    if (j < nk) {
      if (t.mode == 0) {
        g = true;
      } else {
        const int b = pg.bin[j];
        g = b > t.bstar || (b == t.bstar && (t.all_b || pg.pick[j]));
      }
    }
    const uint64_t m = __ballot(g);
    if (lane == 0 && j0 + 64 * wave < nk) words[(j0 >> 6) + wave] = m;
  }
  lds_barrier();
  const int c0 = lane < nwords ? __popcll(words[lane]) : 0;
  const int c1 = lane + 64 < nwords ? __popcll(words[lane + 64]) : 0;
  const int i0 = wave_incl_scan(c0), i1 = wave_incl_scan(c1);
  const int ex0 = i0 - c0, ex1 = __builtin_amdgcn_readlane(i0, 63) + i1 - c1;  // kept pages before each word
  for (int j0 = 0; j0 < nk; j0 += nt) {
    const int w = (j0 >> 6) + wave;  // this wave's word of the stride (wave-uniform)
    if (j0 + 64 * wave >= nk) break;
    const uint64_t m = words[w];
    const int before = w < 64 ? __builtin_amdgcn_readlane(ex0, w) : __builtin_amdgcn_readlane(ex1, w - 64);
    if ((m >> lane) & 1u) emit(before + __popcll(m & ((1ull << lane) - 1ull)), j0 + tid);
  }
}

}  // namespace bkv
