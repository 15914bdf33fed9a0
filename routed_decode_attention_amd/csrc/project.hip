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
//
// Decode can fuse the combination of the attention splits into the
// projection: a workgroup merges the partials of its 16 rows into LDS (every
// column tile repeats this small merge) while its W fragments are already in
// flight, then multiplies them as above.
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

constexpr int MP_THREADS = 512;               // 8 waves
constexpr int MP_COLS = 256;                  // columns per workgroup: 32 per wave
constexpr int MP_KB = 8;                      // contraction steps of 32 loaded per batch

// Merge of 16 decode rows' attention splits, then out = z.W_of for 256
// columns.  Dynamic LDS: the merged rows, fp32 [16][kdim].
__global__ __launch_bounds__(MP_THREADS) void merge_project_kernel(MergeProjectArgs a) {
  extern __shared__ float zs[];
  const int R = a.s.rank_v, G = a.s.group, H = a.s.n_kv_heads, Hq = a.s.n_q_heads;
  const int kdim = Hq * R, ksteps = kdim / 32, nout = a.s.d_model;
  const int tiles_n = nout / MP_COLS;
  const int row0 = (blockIdx.x / tiles_n) * 16, colt = blockIdx.x % tiles_n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, qd = lane >> 4;
  const int col0 = colt * MP_COLS + wave * 32;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  // this wave's weight fragments (two 16-column tiles), first batch in flight
  bf16x8 wf[MP_KB][2];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int kk = 0; kk < MP_KB; ++kk)
      if (k0 + kk < ksteps) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          wf[kk][j] = load_bf16x8(W + (size_t)(col0 + 16 * j + n) * kdim + 32 * (k0 + kk) + 8 * qd);
      }
  };
  load_w(0);

  // merge: one task per (row, 4 latent channels of one query head)
  const int q4 = kdim / 4;
  for (int t = tid; t < 16 * q4; t += MP_THREADS) {
    const int bl = t / q4, k = 4 * (t % q4);
    const int b = row0 + bl, hq = k / R, r0 = k % R;
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    if (b < a.s.batch) {
      const int pair = b * H + hq / G;
      z = merge_splits4(a.part_acc + (size_t)pair * a.n_wsplit * G * R, a.part_ml + (size_t)pair * a.n_wsplit * G * 2,
                        a.n_wsplit, G, R, hq % G, r0);
      if (a.z_out && colt == 0) *reinterpret_cast<f32x4*>(a.z_out + ((size_t)b * Hq + hq) * R + r0) = z;
    }
    *reinterpret_cast<f32x4*>(zs + bl * kdim + k) = z;
  }
  __syncthreads();

  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int k0 = 0; k0 < ksteps; k0 += MP_KB) {
    if (k0 > 0) load_w(k0);
#pragma unroll
    for (int kk = 0; kk < MP_KB; ++kk) {
      if (k0 + kk >= ksteps) break;
      const float* zp = zs + n * kdim + 32 * (k0 + kk) + 8 * qd;
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(zp), x1 = *reinterpret_cast<const f32x4*>(zp + 4);
      const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      bf16x8 af, al;
      split_bf16x8(x, af, al);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf[kk][j], acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wf[kk][j], acc[j], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = row0 + 4 * qd + i;
    if (row < a.s.batch) {
#pragma unroll
      for (int j = 0; j < 2; ++j) a.out[(size_t)row * nout + col0 + 16 * j + n] = acc[j][i];
    }
  }
}

}  // namespace

bool project_mfma_supported(int kdim, int n, int dtype) {
  return dtype == 1 && kdim % 32 == 0 && n % 64 == 0;
}

bool merge_project_supported(const Shape& s, int n_wsplit) {
  const int kdim = s.n_q_heads * s.rank_v;
  // every workgroup re-reads its 16 rows' partials: keep that under 160 KiB
  const size_t part_bytes = (size_t)16 * s.n_kv_heads * n_wsplit * s.group * (s.rank_v + 2) * sizeof(float);
  return s.dtype == 1 && kdim % 32 == 0 && kdim <= 1024 && s.d_model % MP_COLS == 0 && n_wsplit > 1 &&
         part_bytes <= 160 * 1024;
}

hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t st) {
  const int kdim = a.s.n_q_heads * a.s.rank_v;
  const size_t lds = (size_t)16 * kdim * sizeof(float);
  const hipError_t e = allow_lds((const void*)merge_project_kernel, lds);
  if (e != hipSuccess) return e;
  const int grid = ((a.s.batch + 15) / 16) * (a.s.d_model / MP_COLS);
  hipLaunchKernelGGL(merge_project_kernel, dim3(grid), dim3(MP_THREADS), lds, st, a);
  return hipGetLastError();
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (project_mfma_supported(a.kdim, a.n, a.dtype)) {
    if (a.rows > 64 && a.n % 128 == 0) {
      // 128x128 per workgroup (2x2 waves of 64x64)
      const int grid = ((a.rows + 127) / 128) * (a.n / 128);
      hipLaunchKernelGGL((project_mfma_kernel<4, 4, 2, 2>), dim3(grid), dim3(256), 0, st, a);
    } else {
      // 16 rows x 64 columns per workgroup (4 waves of 16x16)
      const int grid = ((a.rows + 15) / 16) * (a.n / 64);
      hipLaunchKernelGGL((project_mfma_kernel<1, 1, 1, 4>), dim3(grid), dim3(256), 0, st, a);
    }
  } else {
    const dim3 grid((a.n + 255) / 256, a.rows);
    if (a.dtype == 0) hipLaunchKernelGGL((project_valu_kernel<float>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((project_valu_kernel<uint16_t>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace bkv
