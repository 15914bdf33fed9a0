// Per-token writer arithmetic shared by the chunk writer and the fused
// append+route kernel, so both produce bit-identical latents, residuals and
// page sums (weekinpapers "BasisKV: Value Latents for Communication and Key
// Routing", Abstract: Value latent z = v.B; Key residual s = (k - z~.P).R_enc).
// Every dot product is one fp32 fused multiply-add chain in index order.
#pragma once

#include "common.hpp"

namespace bkv {

// Every long dot product runs as four interleaved fused multiply-add chains
// (indices i = 4m + c for chain c) combined as (c0 + c1) + (c2 + c3).

// z_r = sum_i v_i * B[i][r]   (B row-major [D][R]; D % 4 == 0)
__device__ __forceinline__ float latent_dot(const float* v, const float* B, int D, int R, int r) {
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < D; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = fmaf(v[i + u], B[(i + u) * R + r], c[u]);
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

// e_i = k_i - sum_r z~_r * P[r][i]   (P rows [R] with row stride ldp >= D)
__device__ __forceinline__ float key_remainder(float k, const float* zt, const float* P, int ldp, int R, int i) {
  float kh = 0.f;
  for (int r = 0; r < R; ++r) kh = fmaf(zt[r], P[r * ldp + i], kh);
  return k - kh;
}

// s_j = sum_i e_i * R_enc[i][j]   (R_enc row-major [D][RK]; D % 4 == 0)
__device__ __forceinline__ float residual_dot(const float* e, const float* Re, int D, int RK, int j) {
  float c[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < D; i += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = fmaf(e[i + u], Re[(i + u) * RK + j], c[u]);
  }
  return (c[0] + c[1]) + (c[2] + c[3]);
}

}  // namespace bkv

namespace bkv {

// Up to four row-major fp32 matrices staged into LDS together: every thread
// issues all of its 16-byte loads (up to 8) before its first LDS store.
struct StageItem {
  float* dst;
  const float* src;
  int ld, rows, cols;
};
struct StageList {
  StageItem it[4];
  int n;
};
__device__ __forceinline__ void stage_matrices(const StageList& L, int t0 = 0, int nt = 0) {
  if (nt == 0) nt = blockDim.x;
  const int me = (int)threadIdx.x - t0;
  if (me < 0 || me >= nt) return;
  int start[5];
  start[0] = 0;
#pragma unroll
  for (int m = 0; m < 4; ++m) start[m + 1] = start[m] + (m < L.n ? L.it[m].rows * L.it[m].cols / 4 : 0);
  const int total = start[4];
  for (int base = me; base < total; base += nt * 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * nt;
      if (idx < total) {
        const float* src = L.it[0].src + (size_t)idx * 4;
#pragma unroll
        for (int m = 1; m < 4; ++m)
          if (idx >= start[m]) src = L.it[m].src + (size_t)(idx - start[m]) * 4;
        v[u] = *reinterpret_cast<const float4*>(src);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * nt;
      if (idx < total) {
        int e = idx * 4, cols = L.it[0].cols, ld = L.it[0].ld;
        float* dst = L.it[0].dst;
#pragma unroll
        for (int m = 1; m < 4; ++m)
          if (idx >= start[m]) {
            e = (idx - start[m]) * 4;
            cols = L.it[m].cols;
            ld = L.it[m].ld;
            dst = L.it[m].dst;
          }
        float* d = dst + (e / cols) * ld + e % cols;
        d[0] = v[u].x;
        d[1] = v[u].y;
        d[2] = v[u].z;
        d[3] = v[u].w;
      }
    }
  }
}

// Copy a row-major [rows][cols] fp32 matrix (cols % 4 == 0, 16-byte aligned)
// into LDS with row stride ld, every thread issuing up to 8 16-byte loads
// before its first store so the copy costs one memory round trip per batch.
__device__ __forceinline__ void stage_matrix(float* dst, int ld, const float* src, int rows, int cols) {
  const int n4 = rows * cols / 4, c4 = cols / 4;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  for (int base = threadIdx.x; base < n4; base += blockDim.x * 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * blockDim.x;
      if (idx < n4) v[u] = s4[idx];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = base + u * blockDim.x;
      if (idx < n4) {
        float* d = dst + (idx / c4) * ld + (idx % c4) * 4;
        d[0] = v[u].x;
        d[1] = v[u].y;
        d[2] = v[u].z;
        d[3] = v[u].w;
      }
    }
  }
}

}  // namespace bkv

namespace bkv {

// Row stride (floats) of P and R_dec rows staged in LDS: 16-byte aligned rows
// that spread consecutive rows over the banks.
__host__ __device__ constexpr int lds_row(int D) { return D + 4; }

// Stage one page's stored latents (channel-major [R][ps], into rows of ps+1
// floats) and residuals ([ps][RK]) into LDS as fp32, one 16-byte load per
// thread and chunk.
template <typename T>
__device__ __forceinline__ void stage_page(float* sZ, float* sS, const T* Zpage, const T* Spage, int R,
                                           int RK, int ps, int t0 = 0, int nt = 0) {
  constexpr int PER = 16 / sizeof(T);
  if (nt == 0) nt = blockDim.x;
  const int me = (int)threadIdx.x - t0;
  if (me < 0 || me >= nt) return;
  const int nz = R * ps / PER, ns = ps * RK / PER;
  for (int c = me; c < nz + ns; c += nt) {
    const bool isz = c < nz;
    const int cc = isz ? c : c - nz;
    const u32x4 v = reinterpret_cast<const u32x4*>(isz ? (const void*)Zpage : (const void*)Spage)[cc];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const uint32_t w = v[e * sizeof(T) / 4];
      const float f = sizeof(T) == 2 ? __uint_as_float(((e & 1) ? (w >> 16) : (w & 0xffffu)) << 16)
                                     : __uint_as_float(w);
      const int idx = cc * PER + e;
      if (isz) sZ[(idx / ps) * (ps + 1) + idx % ps] = f;
      else sS[idx] = f;
    }
  }
}

// Page sum of channel x (latent x < R, else residual x - R) over slots
// [0, valid), in slot order, from a staged page.
__device__ __forceinline__ float page_channel_sum(const float* sZ, const float* sS, int R, int RK, int ps, int x,
                                                  int valid) {
  float acc = 0.f;
  if (x < R) {
    for (int t = 0; t < valid; ++t) acc += sZ[x * (ps + 1) + t];
  } else {
    for (int t = 0; t < valid; ++t) acc += sS[t * RK + (x - R)];
  }
  return acc;
}

}  // namespace bkv
