// Output projection through the folded weights: out = z . W_of, with W_of =
// B^T.W_O (weekinpapers "BasisKV: Value Latents for Communication and Key
// Routing", Abstract, observation (ii): Value compression associated with the
// output projection; kongchang article, same section).  z is the attention
// output still in latent space, [rows][n_q_heads*r]; W_ofT is stored
// [d_model][n_q_heads*r], so both MFMA operands are contiguous along the
// contraction and load straight from memory as 16-byte fragments.
//
// bf16: v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  z is split on load
// into a bf16 high part and the bf16 rounding of its remainder, and both are
// multiplied (two MFMAs): z keeps about 16 significant bits instead of 8, so
// the only rounding left in the product is the stored weights'.  A wave
// computes WM x WN tiles of 16x16; a workgroup holds WAVES_M x WAVES_N waves.  Decode batches use one 16-row tile per wave (the
// rows are the batch), prefill chunks 64x64 per wave.
// fp32 (or shapes the matrix cores do not tile): a VALU dot per output.

#include <stdlib.h>

#include "common.hpp"
#include "internal.hpp"
#include "split_merge.hpp"

namespace bkv {

namespace {

template <int WM, int WN, int WAVES_M, int WAVES_N>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void project_mfma_kernel(ProjectArgs a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tiles_n = a.n / (16 * WN * WAVES_N);
  const int bid = blockIdx.x;
  const int row0 = (bid / tiles_n) * (16 * WM * WAVES_M) + wm * 16 * WM;
  const int col0 = (bid % tiles_n) * (16 * WN * WAVES_N) + wn * 16 * WN;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  f32x4 acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // KB slices of 32 along the contraction per batch: every fragment of a
  // batch is loaded before its first MFMA (one memory round trip per batch).
  constexpr int KB = (WM + WN) <= 2 ? 8 : 2;
  for (int k0 = 0; k0 < a.kdim; k0 += 32 * KB) {
    float4 zr[KB][WM][2];
    bf16x8 bfr[KB][WN];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int k = k0 + 32 * kb;
      if (k < a.kdim) {
#pragma unroll
        for (int i = 0; i < WM; ++i) {
          const int row = row0 + 16 * i + n;
          const float4* zp = reinterpret_cast<const float4*>(a.z + (size_t)row * a.kdim + k + 8 * qd);
          zr[kb][i][0] = row < a.rows ? zp[0] : float4{0.f, 0.f, 0.f, 0.f};
          zr[kb][i][1] = row < a.rows ? zp[1] : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < WN; ++j) bfr[kb][j] = load_bf16x8(W + (size_t)(col0 + 16 * j + n) * a.kdim + k + 8 * qd);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if (k0 + 32 * kb >= a.kdim) break;
#pragma unroll
      for (int i = 0; i < WM; ++i) {
        const float x[8] = {zr[kb][i][0].x, zr[kb][i][0].y, zr[kb][i][0].z, zr[kb][i][0].w,
                            zr[kb][i][1].x, zr[kb][i][1].y, zr[kb][i][1].z, zr[kb][i][1].w};
        bf16x8 af, al;
        split_bf16x8(x, af, al);
#pragma unroll
        for (int j = 0; j < WN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[kb][j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfr[kb][j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 16 * i + 4 * qd + e;
      if (row < a.rows) {
#pragma unroll
        for (int j = 0; j < WN; ++j) a.out[(size_t)row * a.n + col0 + 16 * j + n] = acc[i][j][e];
      }
    }
}

// Decode: the attention splits' merge and the projection in one launch.  A
// workgroup of MP_WAVES waves owns MP_ROWS batch rows and 16 * MP_WN *
// MP_WAVES output columns: it requests its weight fragments for the whole
// contraction first, then merges the splits of its rows into LDS (one
// 4-channel task per thread), then each wave multiplies its 16 x 16 tiles as
// project_mfma_kernel does, the A operand padded to 16 rows with zeros.  The
// partials are re-read by every column group and the weights by every row
// group (from L2); small tiles keep both per workgroup small.
constexpr int MP_WAVES = 8;
constexpr int MP_ROWS = 2;
constexpr int MP_WN = 1;  // 16-column tiles per wave
constexpr int MP_COLS = 16 * MP_WN * MP_WAVES;
constexpr int MP_KMAX = 512;  // contraction length held in registers and LDS

__global__ __launch_bounds__(64 * MP_WAVES) void merge_project_kernel(MergeProjectArgs a) {
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [16][kdim], rows past MP_ROWS zero
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int G = a.s.group, R = a.s.rank_v, H = a.s.n_kv_heads, kdim = a.kdim;
  const int row0 = blockIdx.y * MP_ROWS;
  const int col = blockIdx.x * MP_COLS + wave * 16 * MP_WN + n;  // and col + 16 j
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  bf16x8 bfr[MP_KMAX / 32][MP_WN];
#pragma unroll
  for (int kb = 0; kb < MP_KMAX / 32; ++kb)
    if (32 * kb < kdim) {
#pragma unroll
      for (int j = 0; j < MP_WN; ++j) bfr[kb][j] = load_bf16x8(W + (size_t)(col + 16 * j) * kdim + 32 * kb + 8 * qd);
    }

  // z rows: z[b][hq * R + r] is head h = hq % G of pair (b, hq / G)
  const int quads = kdim / 4;
  for (int t = threadIdx.x; t < 16 * quads; t += blockDim.x) {
    const int row = t / quads, k = 4 * (t % quads);
    const int b = row0 + row, hq = k / R, r0 = k % R;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    if (row < MP_ROWS && b < a.rows) {
      const size_t pair = (size_t)b * H + hq / G;
      z = merge_splits4(a.part_acc + pair * a.n_wsplit * G * R, a.part_ml + pair * a.n_wsplit * G * 2,
                        a.n_wsplit, G, R, hq % G, r0);
      if (a.z_out && blockIdx.x == 0) *reinterpret_cast<f32x4*>(a.z_out + (size_t)b * kdim + k) = z;
    }
    *reinterpret_cast<f32x4*>(zs + row * kdim + k) = z;
  }
  __syncthreads();

  f32x4 acc[MP_WN];
#pragma unroll
  for (int j = 0; j < MP_WN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < MP_KMAX / 32; ++kb) {
    if (32 * kb >= kdim) break;
    const float* zp = zs + n * kdim + 32 * kb + 8 * qd;
    const f32x4 lo4 = *reinterpret_cast<const f32x4*>(zp), hi4 = *reinterpret_cast<const f32x4*>(zp + 4);
    const float x[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    bf16x8 af, al;
    split_bf16x8(x, af, al);
#pragma unroll
    for (int j = 0; j < MP_WN; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[kb][j], acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfr[kb][j], acc[j], 0, 0, 0);
    }
  }
  // tile rows 4 qd + e; only the first MP_ROWS are real
  if (4 * qd < MP_ROWS) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 4 * qd + e;
      if (4 * qd + e < MP_ROWS && row < a.rows) {
#pragma unroll
        for (int j = 0; j < MP_WN; ++j) a.out[(size_t)row * a.n + col + 16 * j] = acc[j][e];
      }
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void project_valu_kernel(ProjectArgs a) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  const int row = blockIdx.y;
  if (c >= a.n) return;
  const T* W = static_cast<const T*>(a.W);
  const float* z = a.z + (size_t)row * a.kdim;
  float acc = 0.f;
  for (int x = 0; x < a.kdim; ++x) acc += z[x] * ld_elem(W, (size_t)c * a.kdim + x);
  a.out[(size_t)row * a.n + c] = acc;
}

}  // namespace

bool merge_project_supported(const Shape& s) {
  // BASISKV_MERGE_PROJECT=0: the split merge and the projection as two
  // launches instead (same results; a tuning override)
  static const bool off = [] {
    const char* e = getenv("BASISKV_MERGE_PROJECT");
    return e && e[0] == '0';
  }();
  const int kdim = s.n_q_heads * s.rank_v;
  return !off && s.dtype == 1 && kdim % 32 == 0 && kdim <= MP_KMAX && s.d_model % MP_COLS == 0;
}

hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(a.n / MP_COLS, (a.rows + MP_ROWS - 1) / MP_ROWS);
  hipLaunchKernelGGL(merge_project_kernel, grid, dim3(64 * MP_WAVES), (size_t)16 * a.kdim * sizeof(float), st, a);
  return hipGetLastError();
}

bool project_mfma_supported(int kdim, int n, int dtype) {
  return dtype == 1 && kdim % 32 == 0 && n % 16 == 0;
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (project_mfma_supported(a.kdim, a.n, a.dtype)) {
    if (a.rows > 64 && a.n % 128 == 0) {
      // 128x128 per workgroup (2x2 waves of 64x64)
      const int grid = ((a.rows + 127) / 128) * (a.n / 128);
      hipLaunchKernelGGL((project_mfma_kernel<4, 4, 2, 2>), dim3(grid), dim3(256), 0, st, a);
    } else {
      // 16 rows x 16 columns per single-wave workgroup: the weights spread
      // over as many CUs as there are column tiles (holding every row tile
      // in one wave, so that each weight tile is read once, measured slower:
      // 63.4 against 62.8 us per 70B 128K step, 49.4 against 48.0 ragged)
      const int grid = ((a.rows + 15) / 16) * (a.n / 16);
      hipLaunchKernelGGL((project_mfma_kernel<1, 1, 1, 1>), dim3(grid), dim3(64), 0, st, a);
    }
  } else {
    const dim3 grid((a.n + 255) / 256, a.rows);
    if (a.dtype == 0) hipLaunchKernelGGL((project_valu_kernel<float>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((project_valu_kernel<uint16_t>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace bkv
