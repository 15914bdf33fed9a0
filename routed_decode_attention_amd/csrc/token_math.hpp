// Per-token writer arithmetic shared by the chunk writer and the fused
// append+route kernel, so both produce bit-identical latents, residuals and
// page sums (weekinpapers "BasisKV: Value Latents for Communication and Key
// Routing", Abstract: Value latent z = v.B; Key residual s = (k - z~.P).R_enc;
// the router reads per-page sums of the stored z~ and s~).
//
// Everything here is executed by one whole wave (64 lanes) per token.  A
// matrix-vector product puts its outputs on lanes and its rows on lane
// slices; each slice accumulates its rows in order and the slices are
// combined by an xor tree, so the summation order is fixed by the shapes
// alone.
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

// Four consecutive LDS elements (storage dtype or fp32) as fp32; p 8-byte
// (bf16) or 16-byte (fp32) aligned.
__device__ __forceinline__ f32x4 lds_f4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 lds_f4(const uint16_t* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
               __uint_as_float(w.y & 0xffff0000u)};
}

// A token's three products are each split into TP fixed parts of their
// contraction, combined in part order (part 0, then + part 1, + part 2,
// + part 3).  The decode-step append computes the parts on TP waves at once;
// the chunk writer computes them in turn on one wave.  The same additions
// happen in the same order, so both store the same bits.
constexpr int TP = 4;

// Part p of out[c] = sum_i x[i] M[i][c], c < nc (x [D], M row-major [D][nc],
// in LDS; nc a multiple of 4): rows [p D/TP, (p+1) D/TP) on one wave.  Lane
// = g + GP s: outputs 4g..4g+3 (GP the power of two >= nc/4) over the s-th of
// S runs of consecutive rows (accumulated in row order), the runs added by
// the xor tree over the lane bits >= log2(GP); lanes of runs >= S add zeros.
// Lanes g < nc/4 of run 0 return the part's outputs 4g..4g+3.
template <int D, int GP, typename X>
__device__ __forceinline__ f32x4 part_dot(const X* x, const float* M, int nc, int p, int lane) {
  constexpr int ROWS = D / TP;
  constexpr int S = (64 / GP) < (ROWS / 4) ? (64 / GP) : (ROWS / 4);
  constexpr int TS = ROWS / S;
  static_assert(TS % 4 == 0, "rows per run in fours");
  const int g = lane & (GP - 1), s = lane / GP;
  const int gg = 4 * g < nc ? g : 0;  // lanes past the outputs repeat group 0, unused
  const int r0 = p * ROWS + (s < S ? s : 0) * TS;
  const X* xs = x + r0;
  const float* Ms = M + (size_t)r0 * nc + 4 * gg;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i0 = 0; i0 < TS; i0 += 4) {
    const f32x4 x4 = lds_f4(xs + i0);
    f32x4 m[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) m[e] = *reinterpret_cast<const f32x4*>(Ms + (size_t)(i0 + e) * nc);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(x4[e], m[e][k], acc[k]);
  }
  if (s >= S) acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if constexpr (GP < 64) xor_tree<GP>(acc, lane);
  return acc;
}

// part_dot for nc <= 64; `own`: this lane holds outputs 4 lane .. 4 lane + 3.
template <int D, typename X>
__device__ __forceinline__ f32x4 part_dot_any(const X* x, const float* M, int nc, int p, int lane, bool& own) {
  f32x4 r;
  int gp;
  if (nc <= 8) {
    gp = 2;
    r = part_dot<D, 2>(x, M, nc, p, lane);
  } else if (nc <= 16) {
    gp = 4;
    r = part_dot<D, 4>(x, M, nc, p, lane);
  } else if (nc <= 32) {
    gp = 8;
    r = part_dot<D, 8>(x, M, nc, p, lane);
  } else {
    gp = 16;
    r = part_dot<D, 16>(x, M, nc, p, lane);
  }
  own = lane < gp && 4 * lane < nc;
  return r;
}

// Part p of k^[i] = sum_r z~[r] P[r][i], i < D (rows [p R/TP, (p+1) R/TP)):
// lane gi < D/4 takes outputs 4gi..4gi+3 over the part's rows in order (P
// rotated: granule gi of row r at rot_granule(r, gi)); other lanes return 0.
template <int D>
__device__ __forceinline__ f32x4 part_keyest(const float* zt, const float* P, int R, int p, int lane) {
  const int RP = R / TP, gi = lane & (D / 4 - 1);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = p * RP; r0 < (p + 1) * RP; r0 += 4) {
    const f32x4 z4 = *reinterpret_cast<const f32x4*>(zt + r0);
    f32x4 pv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = *reinterpret_cast<const f32x4*>(P + (r0 + e) * D + rot_granule(r0 + e, gi, D) * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(z4[e], pv[e][k], acc[k]);
  }
  return lane < D / 4 ? acc : f32x4{0.f, 0.f, 0.f, 0.f};
}

// x0 + x1 + x2 + x3 in part order, four at a time from part buffers
// [TP][stride] at column c.
__device__ __forceinline__ f32x4 parts_sum4(const float* parts, int stride, int c) {
  f32x4 v = *reinterpret_cast<const f32x4*>(parts + c);
#pragma unroll
  for (int q = 1; q < TP; ++q) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(parts + q * stride + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] += w[k];
  }
  return v;
}

// LDS operands of one token's write.
template <typename T>
struct TokenLds {
  const T *v, *k;            // [D] the token, storage dtype
  const float *B, *P, *Re;   // B [D][R], P rotated [R][D], R_enc [D][RK]
  float* e;                  // [D] scratch: the Key remainder
  float* st;                 // [R + RK] out: stored latent, then residual (fp32 values)
  float *zp, *kp, *sp;       // part buffers [TP][64], [TP][128], [TP][64]
};

// Steps of one token's stored values, each taking part p of its product
// (LDS only; all buffers 16-byte aligned):
//   latent:    zp[p] = part p of v.B;              z~ = round(sum of the parts)
//   remainder: kp[p] = part p of z~.P;             e = k - sum of the parts
//   residual:  sp[p] = part p of e.R_enc;          s~ = round(sum of the parts)
template <typename T, int D>
__device__ __forceinline__ void token_latent_part(const TokenLds<T>& L, int R, int p, int lane) {
  bool own;
  const f32x4 z = part_dot_any<D>(L.v, L.B, R, p, lane, own);
  if (own) *reinterpret_cast<f32x4*>(L.zp + p * 64 + 4 * lane) = z;
}
// z~ rows [r0, r0 + n) from the latent parts (n <= 64, r0 + n <= R), lanes < n
template <typename T>
__device__ __forceinline__ void token_latent_finish(const TokenLds<T>& L, int r0, int n, int lane) {
  if (lane < n) {
    float v = L.zp[r0 + lane];
#pragma unroll
    for (int q = 1; q < TP; ++q) v += L.zp[q * 64 + r0 + lane];
    L.st[r0 + lane] = round_only(v, static_cast<const T*>(nullptr));
  }
}
template <typename T, int D>
__device__ __forceinline__ void token_keyest_part(const TokenLds<T>& L, int R, int p, int lane) {
  const f32x4 kh = part_keyest<D>(L.st, L.P, R, p, lane);
  if (lane < D / 4) *reinterpret_cast<f32x4*>(L.kp + p * 128 + 4 * lane) = kh;
}
// e[i] for i in [i0, i0 + 4 n4) from the key-estimate parts, lanes < n4
template <typename T>
__device__ __forceinline__ void token_remainder_finish(const TokenLds<T>& L, int i0, int n4, int lane) {
  if (lane < n4) {
    const int c = i0 + 4 * lane;
    const f32x4 kh = parts_sum4(L.kp, 128, c);
    const f32x4 k4 = lds_f4(L.k + c);
    *reinterpret_cast<f32x4*>(L.e + c) = f32x4{k4[0] - kh[0], k4[1] - kh[1], k4[2] - kh[2], k4[3] - kh[3]};
  }
}
template <typename T, int D>
__device__ __forceinline__ void token_residual_part(const TokenLds<T>& L, int RK, int p, int lane) {
  bool own;
  const f32x4 s = part_dot_any<D>(static_cast<const float*>(L.e), L.Re, RK, p, lane, own);
  if (own) *reinterpret_cast<f32x4*>(L.sp + p * 64 + 4 * lane) = s;
}
template <typename T>
__device__ __forceinline__ void token_residual_finish(const TokenLds<T>& L, int R, int RK, int lane) {
  if (lane < RK) {
    float v = L.sp[lane];
#pragma unroll
    for (int q = 1; q < TP; ++q) v += L.sp[q * 64 + lane];
    L.st[R + lane] = round_only(v, static_cast<const T*>(nullptr));
  }
}

// One token's stored values on one wave (the chunk writer): the parts in
// turn, then their sums, for each product; values into L.st.
template <typename T, int D>
__device__ __forceinline__ void wave_token_values(const TokenLds<T>& L, int R, int RK, int lane) {
  for (int p = 0; p < TP; ++p) token_latent_part<T, D>(L, R, p, lane);
  wave_sync();
  token_latent_finish(L, 0, R, lane);
  wave_sync();
  for (int p = 0; p < TP; ++p) token_keyest_part<T, D>(L, R, p, lane);
  wave_sync();
  token_remainder_finish(L, 0, D / 4, lane);
  wave_sync();
  for (int p = 0; p < TP; ++p) token_residual_part<T, D>(L, RK, p, lane);
  wave_sync();
  token_residual_finish(L, R, RK, lane);
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

// Page sums over slots [0, valid) of a page image (storage dtype, latents
// channel-major [R][ps], residuals [ps][RK]) into out[R + RK] (whole wave).
// bf16: the sums of slots [0, valid - 1) as matrix-core products with a ones
// operand (the page's slots >= valid - 1 zeroed; latents as the A operand,
// 16 channels x 32 slots, 16 contiguous bytes per lane; residuals as the B
// operand, 32 slots x 16 channels), then slot valid - 1 added in fp32.  So a
// decode-step append at slot s gets the same bits from the sums of the
// slots before it, which it can take before its own token exists, plus the
// token.  fp32: one lane per channel, in slot order.
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
  const int last = max(valid - 1, 0);  // slot added after the products
  // latents: every fragment of up to 4 channel tiles x 2 slot halves is read
  // first (addresses clamped into the page, out-of-range parts zeroed)
  bf16x8 a[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int t0 = 32 * kc + 8 * qd;
      const int row = min(16 * mt + n, R - 1), tt = min(t0, ps - 8);
      const int keep = (16 * mt < R && t0 < ps) ? last - t0 : 0;
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
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * mt + 4 * qd + i;
          out[ch] = valid > 0 ? acc[i] + bf16_to_f32(Zimg[ch * ps + last]) : acc[i];
        }
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
        const uint32_t kept = h[e] & (0u - (uint32_t)(ch < RK && t < last));
        if (e & 1) u[kc][e >> 1] |= kept << 16;
        else u[kc][e >> 1] = kept;
      }
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[0]), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[1]), acc, 0, 0, 0);
    // every row of the product is the column sum; row 4 qd of column n
    if (qd == 0 && ch < RK) out[R + ch] = valid > 0 ? acc[0] + bf16_to_f32(Simg[last * RK + ch]) : acc[0];
  }
}

// wave_page_sums' operands for a bf16 page read straight from memory into
// registers (latents [R][ps], residuals [ps][RK]; r, r_k <= 64), so that the
// sums of the slots before a new token's slot need no LDS copy of the page.
// prefix() applies wave_page_sums' masks and products to the same operand
// values, so both give the same bits.
struct PageSumRegs {
  bf16x8 a[4][2];       // latents: channel 16 mt + n, slots 32 kc + 8 qd + 0..7
  u32x4 h[4][2][2];     // residuals: channel 16 nt + n, slot 32 kc + 8 qd + e in h[nt][kc][e / 4][e % 4] (16-bit values)
  __device__ __forceinline__ void load(const uint16_t* Z, const uint16_t* S, int R, int RK, int ps, int lane) {
    const int n = lane & 15, qd = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      if (16 * mt < R)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) a[mt][kc] = load_bf16x8(Z + (16 * mt + n) * ps + min(32 * kc + 8 * qd, ps - 8));
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (16 * nt < RK) {
        const int cc = min(16 * nt + n, RK - 1);
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int e = 0; e < 8; ++e) h[nt][kc][e >> 2][e & 3] = S[min(32 * kc + 8 * qd + e, ps - 1) * RK + cc];
      }
  }
  // The matrix-core part of wave_page_sums for a page whose slot `slot` is
  // its last: the sums over slots [0, slot) into out[R + RK] (whole wave);
  // the slot's own values are added to them afterwards.
  __device__ __forceinline__ void prefix(int R, int RK, int ps, int slot, float* out, int lane) const {
    const int n = lane & 15, qd = lane >> 4;
    const u32x4 ones_u = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      if (16 * mt < R) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int t0 = 32 * kc + 8 * qd;
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(keep_first_n(a[mt][kc], t0 < ps ? slot - t0 : 0), ones, acc,
                                                        0, 0, 0);
        }
        if (n == 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) out[16 * mt + 4 * qd + i] = acc[i];
        }
      }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
      if (16 * nt < RK) {
        const int ch = 16 * nt + n;
        u32x4 u[2];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 32 * kc + 8 * qd + e;
            const uint32_t kept = h[nt][kc][e >> 2][e & 3] & (0u - (uint32_t)(ch < RK && t < slot));
            if (e & 1) u[kc][e >> 1] |= kept << 16;
            else u[kc][e >> 1] = kept;
          }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[0]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u[1]), acc, 0, 0, 0);
        if (qd == 0 && ch < RK) out[R + ch] = acc[0];
      }
  }
};

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
