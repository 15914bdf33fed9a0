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
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int c = lane + 64 * u;
      if (c < n16) v[u] = c < nz16 ? z[c] : s[c - nz16];
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

// Add the values of lanes l ^ m for m = from, 2 from, ..., 32 (every lane of
// a group ends with the same bits).
__device__ __forceinline__ void xor_tree(f32x4& a, int from) {
  for (int m = from; m < 64; m <<= 1) {
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] += __shfl_xor(a[k], m);
  }
}

// out[c] = sum_i x[i] * M[i][c] for c < nc (nc % 4 == 0, nc <= 64); x [D]
// fp32 and M row-major [D][nc] fp32, both in LDS.  Lane layout: output group
// g = lane % GP (GP = nc/4 rounded up to a power of two), row slice
// s = lane / GP of D / (64 / GP) consecutive rows.  Returns whether this lane
// holds outputs 4g..4g+3 (slice 0, g < nc/4) in acc.
template <int D>
__device__ __forceinline__ bool wave_matvec(const float* x, const float* M, int nc, int lane, f32x4& acc,
                                            int& g) {
  const int G4 = nc >> 2;
  const int GP = G4 <= 1 ? 1 : 1 << (32 - __builtin_clz(G4 - 1));
  const int S = 64 / GP, rows = D / S;
  g = lane & (GP - 1);
  const int s = lane / GP;
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  if (g < G4) {
    const float* xr = x + s * rows;
    const float* mr = M + (size_t)s * rows * nc + 4 * g;
#pragma unroll 4
    for (int i = 0; i < rows; ++i) {
      const float xi = xr[i];
      const f32x4 m4 = *reinterpret_cast<const f32x4*>(mr + (size_t)i * nc);
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = fmaf(xi, m4[k], acc[k]);
    }
  }
  xor_tree(acc, GP);
  return s == 0 && g < G4;
}

// e[i] = k[i] - sum_r zt[r] * P[r][i] for i < D, P in the rotated layout.
// Lane layout: column group gi = lane % (D/4), latent slice lane / (D/4) of
// R / (256/D) consecutive rows (R a multiple of 16).
template <int D>
__device__ __forceinline__ void wave_key_remainder(const float* k, const float* zt, const float* P, int R,
                                                   int lane, float* e) {
  constexpr int GD = D / 4, SR = 64 / GD;
  const int gi = lane % GD, sr = lane / GD, rows = R / SR;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = sr * rows; r < (sr + 1) * rows; ++r) {
    const float z = zt[r];
    const f32x4 p = *reinterpret_cast<const f32x4*>(P + r * D + rot_granule(r, gi, D) * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(z, p[q], acc[q]);
  }
  xor_tree(acc, GD);
  if (sr == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) e[4 * gi + q] = k[4 * gi + q] - acc[q];
  }
}

// LDS operands of one token's write.
struct TokenLds {
  const float *v, *k;        // [D] the token, fp32
  const float *B, *P, *Re;   // B [D][R], P rotated [R][D], R_enc [D][RK]
  float* e;                  // [D] scratch: the Key remainder
  float* st;                 // [R + RK] out: stored latent, then residual (fp32 values)
};

// Write one token (whole wave): the exact Key into Krow[0..D), the rounded
// latent z~ = round(v.B) into Zpage[r * ps + slot] and the rounded residual
// s~ = round((k - z~.P).R_enc) into Spage[slot * RK + j]; their fp32 values
// go to L.st.
template <typename T, int D>
__device__ __forceinline__ void wave_write_token(const TokenLds& L, int R, int RK, int ps, int slot, T* Krow,
                                                 T* Zpage, T* Spage, int lane) {
#pragma unroll
  for (int i = lane; i < D; i += 64) store_elem(Krow, i, L.k[i]);  // exact: k came from T
  f32x4 acc;
  int g;
  if (wave_matvec<D>(L.v, L.B, R, lane, acc, g)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) L.st[4 * g + q] = round_store(Zpage, (size_t)(4 * g + q) * ps + slot, acc[q]);
  }
  wave_sync();
  wave_key_remainder<D>(L.k, L.st, L.P, R, lane, L.e);
  wave_sync();
  if (wave_matvec<D>(L.e, L.Re, RK, lane, acc, g)) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      L.st[R + 4 * g + q] = round_store(Spage, (size_t)slot * RK + 4 * g + q, acc[q]);
  }
  wave_sync();
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
  const int kcs = (ps + 31) / 32;
  for (int mt = 0; mt < R / 16; ++mt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int kc = 0; kc < kcs; ++kc) {
      const int t0 = 32 * kc + 8 * qd;
      bf16x8 a = zero_bf16x8();
      if (t0 < ps) a = keep_first_n(*reinterpret_cast<const bf16x8*>(Zimg + (16 * mt + n) * ps + t0), valid - t0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ones, acc, 0, 0, 0);
    }
    // lane (n, qd) holds rows 4 qd + i of column n; column 0 is taken
    if (n == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) out[16 * mt + 4 * qd + i] = acc[i];
    }
  }
  for (int nt = 0; nt < (RK + 15) / 16; ++nt) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int ch = 16 * nt + n;
    for (int kc = 0; kc < kcs; ++kc) {
      const int t0 = 32 * kc + 8 * qd;
      u32x4 u = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = t0 + e;
        const uint32_t h = (ch < RK && t < valid) ? Simg[t * RK + ch] : 0u;
        u[e >> 1] |= (e & 1) ? (h << 16) : h;
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, __builtin_bit_cast(bf16x8, u), acc, 0, 0, 0);
    }
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
