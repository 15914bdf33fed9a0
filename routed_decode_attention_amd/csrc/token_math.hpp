// Per-token writer arithmetic shared by the chunk writer and the fused
// append+route kernel, so both produce bit-identical latents, residuals and
// page sums (weekinpapers "BasisKV: Value Latents for Communication and Key
// Routing", Abstract: Value latent z = v.B; Key residual s = (k - z~.P).R_enc;
// the router reads per-page sums of the stored z~ and s~).
//
// Everything here is executed by one whole wave (64 lanes) per token.  A
// matrix-vector product spreads its outputs over lanes in groups of four
// (one 16-byte LDS read per row) and its rows over lane slices; each slice
// accumulates its rows in order and the slices are combined by an xor tree,
// so the summation order is fixed by the shapes alone.
#pragma once

#include "common.hpp"

namespace bkv {

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// Direct 16-byte global -> LDS copy: lane l writes LDS bytes
// [dst + 16 l, dst + 16 l + 16) with the 16 bytes at its own src (dst must be
// the same for every lane of the wave).  Completion is counted by vmcnt.
__device__ __forceinline__ void dma16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)dst, 16, 0, 0);
}

// Intra-wave LDS hand-off: the wave's LDS writes are complete and visible to
// its other lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS only: the wave's LDS accesses complete
// before it, while its global loads stay in flight across it (a plain
// __syncthreads also waits for every outstanding global load).  Not for
// handing off LDS written by direct global -> LDS copies.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// LDS layout of the factor P (and R_dec): row x holds D floats whose 16-byte
// granules are rotated by x, so lanes reading the same column of different
// rows (or different columns of one row) spread over the banks.
__host__ __device__ constexpr int rot_granule(int x, int c, int D) { return (c + x) & (D / 4 - 1); }

// Stage n16 16-byte granules into LDS (granule G lands at dst + 16 G) from
// the global granule src(G); the waves of a workgroup take 64-granule blocks
// in turn, block 0 going to wave `first`.  Returns the wave for the next
// item's block 0.  The caller waits (vmcnt) and barriers before reading.
template <typename F>
__device__ __forceinline__ int dma_stage(void* dst, int n16, F src, int first, int nwaves, int wave, int lane) {
  const int nblk = (n16 + 63) / 64;
  for (int blk = (wave - first + nwaves) % nwaves; blk < nblk; blk += nwaves) {
    const int G = blk * 64 + lane;
    if (G < n16) dma16(src(G), static_cast<char*>(dst) + (size_t)blk * 1024);
  }
  return (first + nblk) % nwaves;
}

// Granule G of the rotated LDS image of a row-major [rows][D] fp32 matrix
// comes from this source granule.
__device__ __forceinline__ int rot_source(int G, int D) {
  const int x = G / (D / 4), c = G % (D / 4);
  return x * (D / 4) + ((c - x) & (D / 4 - 1));
}

// One page's stored latents and residuals as a raw LDS image (Z granules,
// then S granules), carried in registers: up to 8 granules per lane are
// requested by load() and written by store(); larger pages copy the rest
// directly.
struct PageImage {
  u32x4 v[8];
  const u32x4 *z, *s;
  int nz16, n16;
  __device__ __forceinline__ void load(const void* Zpage, const void* Spage, int nz, int ns, int lane) {
    z = static_cast<const u32x4*>(Zpage);
    s = static_cast<const u32x4*>(Spage);
    nz16 = nz;
    n16 = nz + ns;
    // unconditional loads (granules past the image re-read its last one and
    // are not stored), so all are in flight together
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = min(lane + 64 * u, n16 - 1);
      v[u] = *(c < nz16 ? z + c : s + (c - nz16));
    }
  }
  __device__ __forceinline__ void store(void* img, int lane) const {
    u32x4* d = static_cast<u32x4*>(img);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = lane + 64 * u;
      if (c < n16) d[c] = v[u];
    }
    for (int c = lane + 512; c < n16; c += 64) d[c] = c < nz16 ? z[c] : s[c - nz16];
  }
};

// x[l] + x[l ^ M] for M in {1, 2, 4, 8, 16, 32}, on the vector ALU only (DPP
// and the gfx950 lane-half swaps).  Both lanes of a pair get the same bits.
#define BKV_DPP(x, ctrl) __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false))
template <int M>
__device__ __forceinline__ float xor_add(float x, int lane) {
  if constexpr (M == 1) {
    return x + BKV_DPP(x, 0xB1);  // quad_perm [1,0,3,2]
  } else if constexpr (M == 2) {
    return x + BKV_DPP(x, 0x4E);  // quad_perm [2,3,0,1]
  } else if constexpr (M == 4) {
    const float up = BKV_DPP(x, 0x104), down = BKV_DPP(x, 0x114);  // row_shl:4, row_shr:4
    return x + ((lane & 4) ? down : up);
  } else if constexpr (M == 8) {
    return x + BKV_DPP(x, 0x128);  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}
#undef BKV_DPP

// Add the values of lanes l ^ m for m = FROM, 2 FROM, ..., 32 (every lane of
// a group ends with the same bits).
template <int FROM>
__device__ __forceinline__ void xor_tree(f32x4& a, int lane) {
  if constexpr (FROM < 64) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = xor_add<FROM>(a[k], lane);
    xor_tree<FROM * 2>(a, lane);
  }
}

// Element i of an LDS operand as fp32 (storage dtype or fp32).
__device__ __forceinline__ float lds_elem(const float* p, int i) { return p[i]; }
__device__ __forceinline__ float lds_elem(const uint16_t* p, int i) { return bf16_to_f32(p[i]); }

// acc[k] += x[i] * M[i][k] for i < ROWS in order (M rows nc floats apart).
template <int ROWS, typename X>
__device__ __forceinline__ void rows_fma(const X* x, const float* M, int nc, f32x4& acc) {
  if constexpr (ROWS > 16) {  // at most 16 rows of operands in flight
    rows_fma<16>(x, M, nc, acc);
    rows_fma<ROWS - 16>(x + 16, M + (size_t)16 * nc, nc, acc);
    return;
  }
  float xv[ROWS];
  f32x4 mv[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    xv[i] = lds_elem(x, i);
    mv[i] = *reinterpret_cast<const f32x4*>(M + (size_t)i * nc);
  }
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = fmaf(xv[i], mv[i][k], acc[k]);
}

// A token's three products are split over CW "virtual waves" of 64 lanes,
// each taking a fixed 1/CW of the contraction; their partials are combined
// in virtual-wave order starting from 0.  The router runs the CW virtual
// waves as its CW real waves at once (partials through LDS); the chunk
// writer runs them in turn on one wave.  The same additions happen in the
// same order, so both produce the same bits.
constexpr int CW = 8;

// Partial of virtual wave w for out[c] = sum_i x[i] M[i][c] (nc % 4 == 0,
// nc <= 64; x [D], M row-major [D][nc], both in LDS): rows
// [w D/CW, (w+1) D/CW).  Lane layout: output group g = lane % GP (GP = nc/4
// rounded up to a power of two), slice s = lane / GP of RS consecutive rows
// (S slices; lanes of later slices contribute 0), slices combined by the xor
// tree.  Returns whether this lane holds outputs 4g..4g+3 in acc.
template <int D, int GP, typename X>
__device__ __forceinline__ bool part_matvec_gp(const X* x, const float* M, int nc, int w, int lane, f32x4& acc,
                                               int& g) {
  constexpr int RW = D / CW, S = (64 / GP) < RW ? 64 / GP : RW, RS = RW / S;
  const int G4 = nc >> 2;
  g = lane & (GP - 1);
  const int s = lane / GP;
  const int r0 = w * RW + (s < S ? s : 0) * RS;
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // lanes past the last output group read group 0 and are discarded
  rows_fma<RS>(x + r0, M + (size_t)r0 * nc + 4 * (g < G4 ? g : 0), nc, acc);
  if (s >= S) acc = f32x4{0.f, 0.f, 0.f, 0.f};
  xor_tree<GP>(acc, lane);
  return s == 0 && g < G4;
}

template <int D, typename X>
__device__ __forceinline__ bool part_matvec(const X* x, const float* M, int nc, int w, int lane, f32x4& acc,
                                            int& g) {
  const int G4 = nc >> 2;
  switch (G4 <= 1 ? 1 : 1 << (32 - __builtin_clz(G4 - 1))) {
    case 1: return part_matvec_gp<D, 1>(x, M, nc, w, lane, acc, g);
    case 2: return part_matvec_gp<D, 2>(x, M, nc, w, lane, acc, g);
    case 4: return part_matvec_gp<D, 4>(x, M, nc, w, lane, acc, g);
    case 8: return part_matvec_gp<D, 8>(x, M, nc, w, lane, acc, g);
    default: return part_matvec_gp<D, 16>(x, M, nc, w, lane, acc, g);
  }
}

// acc[q] += zt[r] * P[r][4 gi + q] over ROWS rows from r0, P rotated.
template <int D, int ROWS>
__device__ __forceinline__ void remainder_rows(const float* zt, const float* P, int r0, int gi, f32x4& acc) {
  float zv[ROWS];
  f32x4 pv[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    zv[i] = zt[r0 + i];
    pv[i] = *reinterpret_cast<const f32x4*>(P + (r0 + i) * D + rot_granule(r0 + i, gi, D) * 4);
  }
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(zv[i], pv[i][q], acc[q]);
}

// Partial of virtual wave w for kh[i] = sum_r zt[r] P[r][i], i < D (P in the
// rotated layout, R a multiple of 16): latent rows [w R/CW, (w+1) R/CW).
// Lane layout: column group gi = lane % (D/4), slice lane / (D/4) of RS rows
// (S slices: the largest power of two <= 256/D dividing R/CW; lanes of later
// slices contribute 0), slices combined by the xor tree.  Lanes of slice 0
// hold kh[4gi .. 4gi+3].
template <int D>
__device__ __forceinline__ f32x4 part_remainder(const float* zt, const float* P, int R, int w, int lane) {
  constexpr int GD = D / 4, SL = 64 / GD;
  const int RW = R / CW;
  int S = SL;
  while (RW % S) S >>= 1;
  const int RS = RW / S;
  const int gi = lane % GD, sr = lane / GD;
  const int r0 = w * RW + (sr < S ? sr : 0) * RS;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  switch (RS) {
    case 1: remainder_rows<D, 1>(zt, P, r0, gi, acc); break;
    case 2: remainder_rows<D, 2>(zt, P, r0, gi, acc); break;
    case 3: remainder_rows<D, 3>(zt, P, r0, gi, acc); break;
    default: remainder_rows<D, 4>(zt, P, r0, gi, acc); break;
  }
  if (sr >= S) acc = f32x4{0.f, 0.f, 0.f, 0.f};
  xor_tree<GD>(acc, lane);
  return acc;
}

// LDS operands of one token's write.
template <typename T>
struct TokenLds {
  const T *v, *k;            // [D] the token, storage dtype
  const float *B, *P, *Re;   // B [D][R], P rotated [R][D], R_enc [D][RK]
  float* e;                  // [D] scratch: the Key remainder
  float* st;                 // [R + RK] out: stored latent, then residual (fp32 values)
};

// One token's stored values on one wave (the chunk writer), LDS only: the
// rounded latent z~ = round(v.B) and residual s~ = round((k - z~.P).R_enc)
// as fp32 into L.st, the CW virtual waves of each product taken in turn.
template <typename T, int D>
__device__ __forceinline__ void wave_token_values(const TokenLds<T>& L, int R, int RK, int lane) {
  f32x4 acc, sum = {0.f, 0.f, 0.f, 0.f};
  int g = 0;
  bool own = false;
  for (int w = 0; w < CW; ++w) {
    own = part_matvec<D>(L.v, L.B, R, w, lane, acc, g);
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] += acc[q];
  }
  if (own) {
#pragma unroll
    for (int q = 0; q < 4; ++q) L.st[4 * g + q] = round_only(sum[q], static_cast<const T*>(nullptr));
  }
  wave_sync();
  f32x4 kh = {0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < CW; ++w) {
    const f32x4 p = part_remainder<D>(L.st, L.P, R, w, lane);
#pragma unroll
    for (int q = 0; q < 4; ++q) kh[q] += p[q];
  }
  if (lane < D / 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) L.e[4 * lane + q] = lds_elem(L.k, 4 * lane + q) - kh[q];
  }
  wave_sync();
  sum = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < CW; ++w) {
    own = part_matvec<D>(L.e, L.Re, RK, w, lane, acc, g);
#pragma unroll
    for (int q = 0; q < 4; ++q) sum[q] += acc[q];
  }
  if (own) {
#pragma unroll
    for (int q = 0; q < 4; ++q) L.st[R + 4 * g + q] = round_only(sum[q], static_cast<const T*>(nullptr));
  }
  wave_sync();
}

// Store one token (whole wave): the exact Key into Krow[0..D), z~ into
// Zpage[r * ps + slot] and s~ into Spage[slot * RK + j] (values exactly
// representable in T).
template <typename T, int D>
__device__ __forceinline__ void wave_token_store(const TokenLds<T>& L, int R, int RK, int ps, int slot, T* Krow,
                                                 T* Zpage, T* Spage, int lane) {
#pragma unroll
  for (int i = lane; i < D; i += 64) Krow[i] = L.k[i];
  for (int x = lane; x < R + RK; x += 64) {
    if (x < R) store_elem(Zpage, (size_t)x * ps + slot, L.st[x]);
    else store_elem(Spage, (size_t)slot * RK + (x - R), L.st[x]);
  }
}

// Page sums over slots [0, valid) of a page image in LDS (storage dtype,
// latents channel-major [R][ps], residuals [ps][RK]) into out[R + RK]
// (whole wave).  bf16: matrix-core products with a ones operand, the page's
// slots >= valid zeroed; latents as the A operand (16 channels x 32 slots,
// 16 contiguous bytes per lane), residuals as the B operand (32 slots x 16
// channels).  fp32: one lane per channel, in slot order.
__device__ __forceinline__ bf16x8 keep_first_n(bf16x8 v, int valid) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = (2 * e < valid) ? 0x0000ffffu : 0u;
    const uint32_t hi = (2 * e + 1 < valid) ? 0xffff0000u : 0u;
    u[e] &= (lo | hi);
  }
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void wave_page_sums(const uint16_t* Zimg, const uint16_t* Simg, int R, int RK, int ps,
                                               int valid, float* out, int lane) {
  const int n = lane & 15, qd = lane >> 4;
  const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);
  // latents: every fragment of up to 4 channel tiles x 2 slot halves is read
  // first (addresses clamped into the page, out-of-range parts zeroed)
  bf16x8 a[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int t0 = 32 * kc + 8 * qd;
      const int row = min(16 * mt + n, R - 1), tt = min(t0, ps - 8);
      const int keep = (16 * mt < R && t0 < ps) ? valid - t0 : 0;
      a[mt][kc] = keep_first_n(*reinterpret_cast<const bf16x8*>(Zimg + row * ps + tt), keep);
    }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    if (16 * mt < R) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][0], ones, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mt][1], ones, acc, 0, 0, 0);
      // lane (n, qd) holds rows 4 qd + i of column n; column 0 is taken
      if (n == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) out[16 * mt + 4 * qd + i] = acc[i];
      }
    }
  // residuals: 16-channel tiles as the B operand (32 slots x 16 channels)
  for (int nt = 0; 16 * nt < RK; ++nt) {
    const int ch = 16 * nt + n, cc = min(ch, RK - 1);
    u32x4 u[2];
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      // every element is read (addresses clamped into the page) and then
      // masked, so the sixteen reads issue together
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = Simg[min(32 * kc + 8 * qd + e, ps - 1) * RK + cc];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = 32 * kc + 8 * qd + e;
        const uint32_t kept = h[e] & (0u - (uint32_t)(ch < RK && t < valid));
        if (e & 1) u[kc][e >> 1] |= kept << 16;
        else u[kc][e >> 1] = kept;
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[1]), acc, 0, 0, 0);
    // every row of the product is the column sum; row 4 qd of column n
    if (qd == 0 && ch < RK) out[R + ch] = acc[0];
  }
}

__device__ __forceinline__ void wave_page_sums(const float* Zimg, const float* Simg, int R, int RK, int ps,
                                               int valid, float* out, int lane) {
  for (int x = lane; x < R + RK; x += 64) {
    float acc = 0.f;
    if (x < R) {
      for (int t = 0; t < valid; ++t) acc += Zimg[x * ps + t];
    } else {
      for (int t = 0; t < valid; ++t) acc += Simg[t * RK + (x - R)];
    }
    out[x] = acc;
  }
}

}  // namespace bkv
