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
#include "token_math.hpp"

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

// Many rows (prefill chunks): 128 x 256 outputs per workgroup of eight waves
// (2 x 4 waves of 64 x 64), the contraction in steps of 64 staged through
// LDS so that each z row and weight column is read once per workgroup: z is
// split into its bf16 high and low parts once, as it is written to LDS; the
// weights are copied straight into LDS.  Each row of a stage keeps its
// 16-byte granules at positions permuted by an XOR with a function of the row,
// so the sixteen rows of a fragment read land on sixteen different bank
// positions.  Two stages: the next step's loads are in flight while this step
// multiplies.  (8K prefill, 2048-row chunks, d_model 4096: 21.2 us per chunk
// with steps of 32, 21.6 with steps of 64, 41 with register-fed 128 x 128
// tiles; what remains is each step's load latency and the fp32 output.)
constexpr int PT_BM = 128, PT_BN = 256, PT_WAVES = 8;
// bytes of one stage (z high, z low, weights) for steps of BK
__host__ __device__ constexpr int pt_stage(int BK) { return (2 * PT_BM + PT_BN) * BK * 2; }

// granule g of a row of GR granules: its position in the row's LDS copy
template <int GR>
__device__ __forceinline__ int pt_pos(int row, int g) {
  if constexpr (GR == 8) return g ^ ((row >> 1) & 7);
  else return g ^ ((row >> 2) & 3);
}

template <int PT_BK>
__global__ __launch_bounds__(64 * PT_WAVES) void project_tiled_kernel(ProjectArgs a) {
  constexpr int PT_GR = PT_BK / 8, PT_STAGE = pt_stage(PT_BK);
  extern __shared__ __attribute__((aligned(16))) char pt_lds[];  // two stages
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_n = a.n / PT_BN;
  const int row0 = (blockIdx.x / tiles_n) * PT_BM, col0 = (blockIdx.x % tiles_n) * PT_BN;
  const int K = a.kdim, steps = (K + PT_BK - 1) / PT_BK;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);
  // this thread's z piece of a stage: row tid / 4, granules ZG (tid % 4) .. + ZG
  constexpr int ZG = PT_GR / 4;
  const int arow = tid >> 2, ag = ZG * (tid & 3);
  const bool arow_ok = row0 + arow < a.rows;
  const float* zrow = a.z + (size_t)(arow_ok ? row0 + arow : 0) * K;
  auto stage_hi = [&](int s) { return pt_lds + (s & 1) * PT_STAGE; };
  auto stage_lo = [&](int s) { return pt_lds + (s & 1) * PT_STAGE + PT_BM * PT_BK * 2; };
  auto stage_w = [&](int s) { return pt_lds + (s & 1) * PT_STAGE + 2 * PT_BM * PT_BK * 2; };
  // (a contraction shorter than the last step: the missing granules are zero)
  auto load_z = [&](int s, float4 (&z)[2 * ZG]) {
#pragma unroll
    for (int u = 0; u < 2 * ZG; ++u) {
      const int k = PT_BK * s + 8 * ag + 4 * u;
      z[u] = arow_ok && k < K ? *reinterpret_cast<const float4*>(zrow + k) : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto put_z = [&](int s, const float4 (&z)[2 * ZG]) {
#pragma unroll
    for (int h = 0; h < ZG; ++h) {
      const float x[8] = {z[2 * h].x, z[2 * h].y, z[2 * h].z, z[2 * h].w,
                          z[2 * h + 1].x, z[2 * h + 1].y, z[2 * h + 1].z, z[2 * h + 1].w};
      bf16x8 hi, lo;
      split_bf16x8(x, hi, lo);
      const int off = 16 * (arow * PT_GR + pt_pos<PT_GR>(arow, ag + h));
      *reinterpret_cast<bf16x8*>(stage_hi(s) + off) = hi;
      *reinterpret_cast<bf16x8*>(stage_lo(s) + off) = lo;
    }
  };
  // the weights of a stage: 256 columns x GR granules, GR / 2 64-granule
  // blocks a wave (granules past the contraction re-read its last one, unused)
  auto copy_w = [&](int s) {
    char* dst = stage_w(s);
    constexpr int NB = PT_GR / 2;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int G = (NB * wave + b) * 64 + lane, c = G / PT_GR, p = G % PT_GR;
      const int k = min(PT_BK * s + 8 * pt_pos<PT_GR>(c, p), K - 8);
      dma16(W + (size_t)(col0 + c) * K + k, dst + (NB * wave + b) * 1024);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  float4 z[2 * ZG];
  load_z(0, z);
  copy_w(0);
  put_z(0, z);
  for (int s = 0; s < steps; ++s) {
    wait_vmem();    // this wave's copies of step s are in
    lds_barrier();  // every wave's are, and every wave is done with step s - 1's buffers
    if (s + 1 < steps) {
      copy_w(s + 1);
      load_z(s + 1, z);
    }
#pragma unroll
    for (int kk = 0; kk < PT_BK / 32; ++kk) {
      if (PT_BK * s + 32 * kk >= K) break;  // (uniform) a contraction shorter than the step
      // this wave's fragments of the step's kk-th 32
      bf16x8 ah[4], al[4], bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 64 * wm + 16 * i + n;
        const int off = 16 * (r * PT_GR + pt_pos<PT_GR>(r, 4 * kk + qd));
        ah[i] = *reinterpret_cast<const bf16x8*>(stage_hi(s) + off);
        al[i] = *reinterpret_cast<const bf16x8*>(stage_lo(s) + off);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 64 * wn + 16 * j + n;
        bw[j] = *reinterpret_cast<const bf16x8*>(stage_w(s) + 16 * (c * PT_GR + pt_pos<PT_GR>(c, 4 * kk + qd)));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bw[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bw[j], acc[i][j], 0, 0, 0);
        }
    }
    if (s + 1 < steps) put_z(s + 1, z);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = row0 + 64 * wm + 16 * i + 4 * qd + e;
      if (row < a.rows) {
#pragma unroll
        for (int j = 0; j < 4; ++j) a.out[(size_t)row * a.n + col0 + 64 * wn + 16 * j + n] = acc[i][j][e];
      }
    }
}

// Decode: the attention splits' merge and the projection in one launch.  A
// workgroup of MP_WAVES waves owns MP_ROWS batch rows and 16 * MP_WN *
// MP_WAVES output columns.  The threads that merge (one 4-channel task of a
// row each) request their rows' partials first, then every thread requests
// its weight fragments for the whole contraction (KB steps of 32), so the
// merge waits only for the partials while the weights are in flight; the
// merged rows go to LDS (row stride kdim + 4 floats, so the lanes reading
// one column of different rows hit different banks), then each wave
// multiplies its 16 x 16 tiles as project_mfma_kernel does, the A operand
// padded to 16 rows with zeros (lanes past MP_ROWS read nothing).  The
// partials are re-read by every column group and the weights by every row
// group (from L2); small tiles keep both per workgroup small.
constexpr int MP_WAVES = 8;
constexpr int MP_ROWS = 2;
constexpr int MP_WN = 1;  // 16-column tiles per wave
constexpr int MP_COLS = 16 * MP_WN * MP_WAVES;
constexpr int MP_KMAX = 512;  // contraction length held in registers and LDS

template <int KB>
__global__ __launch_bounds__(64 * MP_WAVES) void merge_project_kernel(MergeProjectArgs a) {
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [MP_ROWS][kdim + 4]
  constexpr int KDIM = 32 * KB, ZST = KDIM + 4, QUADS = KDIM / 4;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int G = a.s.group, R = a.s.rank_v, H = a.s.n_kv_heads;
  const int row0 = blockIdx.y * MP_ROWS;
  const int col = blockIdx.x * MP_COLS + wave * 16 * MP_WN + n;  // and col + 16 j
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  // z rows: z[b][hq * R + r] is head h = hq % G of pair (b, hq / G); thread t
  // < MP_ROWS * QUADS merges row t / QUADS, channels 4 (t % QUADS) ..
  const int t = threadIdx.x, row = t / QUADS, k = 4 * (t % QUADS);
  const int b = row0 + row;
  const bool merger = t < MP_ROWS * QUADS && b < a.rows;
  SplitMerge m{nullptr, nullptr, a.n_wsplit, G, R, 0, 0};
  if (merger) {
    const int hq = k / R;
    const size_t pair = (size_t)b * H + hq / G;
    m.acc = a.part_acc + pair * a.n_wsplit * G * R;
    m.ml = a.part_ml + pair * a.n_wsplit * G * 2;
    m.h = hq % G;
    m.r0 = k % R;
    m.load(0);
  }
  bf16x8 bfr[KB][MP_WN];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int j = 0; j < MP_WN; ++j) bfr[kb][j] = load_bf16x8(W + (size_t)(col + 16 * j) * KDIM + 32 * kb + 8 * qd);
  if (merger) {
    __builtin_amdgcn_sched_barrier(0);
    m.fold(0);
    for (int s0 = MERGE_CHUNK; s0 < a.n_wsplit; s0 += MERGE_CHUNK) {
      m.load(s0);
      __builtin_amdgcn_sched_barrier(0);
      m.fold(s0);
    }
    const f32x4 z = m.finish();
    if (a.z_out && blockIdx.x == 0) *reinterpret_cast<f32x4*>(a.z_out + (size_t)b * KDIM + k) = z;
    *reinterpret_cast<f32x4*>(zs + row * ZST + k) = z;
  } else if (t < MP_ROWS * QUADS) {
    *reinterpret_cast<f32x4*>(zs + row * ZST + k) = f32x4{0.f, 0.f, 0.f, 0.f};  // rows past the batch
  }
  lds_barrier();

  f32x4 acc[MP_WN];
#pragma unroll
  for (int j = 0; j < MP_WN; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (n < MP_ROWS) {
      const float* zp = zs + n * ZST + 32 * kb + 8 * qd;
      const f32x4 lo4 = *reinterpret_cast<const f32x4*>(zp), hi4 = *reinterpret_cast<const f32x4*>(zp + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = lo4[e];
        x[4 + e] = hi4[e];
      }
    }
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
      const int r = row0 + 4 * qd + e;
      if (4 * qd + e < MP_ROWS && r < a.rows) {
#pragma unroll
        for (int j = 0; j < MP_WN; ++j) a.out[(size_t)r * a.n + col + 16 * j] = acc[j][e];
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

// Beyond 16 rows: the same with a whole 16-row tile of real rows per
// workgroup (16 rows x 128 columns), so the weights are read by every row
// tile and the partials re-merged by every column group; NW waves, each
// thread merging TPT 4-channel tasks with all their partials requested before
// the weights, the first MP_WAVES waves then multiplying.
constexpr int MR_ROWS = 16;
constexpr int MR_KMAX = 256;  // the merged rows' registers: two tasks a thread at most

namespace {

template <int KB, int NW>
__global__ __launch_bounds__(64 * NW) void merge_project_rows_kernel(MergeProjectArgs a) {
  extern __shared__ __attribute__((aligned(16))) float zs[];  // [MR_ROWS][kdim + 4]
  constexpr int KDIM = 32 * KB, ZST = KDIM + 4, QUADS = KDIM / 4;
  constexpr int TASKS = MR_ROWS * QUADS, TPT = (TASKS + 64 * NW - 1) / (64 * NW);
  static_assert(TPT <= 2, "contraction too long for the row-tile merge");
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, qd = lane >> 4;
  const int G = a.s.group, R = a.s.rank_v, H = a.s.n_kv_heads;
  const int row0 = blockIdx.y * MR_ROWS;
  const int col = blockIdx.x * MP_COLS + wave * 16 * MP_WN + n;
  const uint16_t* W = static_cast<const uint16_t*>(a.W);

  // task u = threadIdx.x + 512 i: row u / QUADS, channels 4 (u % QUADS) ..;
  // eight splits requested together (the long-context plans' split counts)
  using SM = SplitMergeT<8>;
  SM m[TPT];
  bool merger[TPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int u = threadIdx.x + 64 * NW * i, row = u / QUADS, k = 4 * (u % QUADS), b = row0 + row;
    merger[i] = u < TASKS && b < a.rows;
    m[i] = SM{nullptr, nullptr, a.n_wsplit, G, R, 0, 0};
    if (merger[i]) {
      const int hq = k / R;
      const size_t pair = (size_t)b * H + hq / G;
      m[i].acc = a.part_acc + pair * a.n_wsplit * G * R;
      m[i].ml = a.part_ml + pair * a.n_wsplit * G * 2;
      m[i].h = hq % G;
      m[i].r0 = k % R;
      m[i].load(0);
    }
  }
  // (waves past MP_WAVES only merge)
  bf16x8 bfr[KB];
  if (wave < MP_WAVES) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) bfr[kb] = load_bf16x8(W + (size_t)col * KDIM + 32 * kb + 8 * qd);
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int u = threadIdx.x + 64 * NW * i, row = u / QUADS, k = 4 * (u % QUADS), b = row0 + row;
    if (merger[i]) {
      __builtin_amdgcn_sched_barrier(0);
      m[i].fold(0);
      for (int s0 = SM::MERGE_CHUNK; s0 < a.n_wsplit; s0 += SM::MERGE_CHUNK) {
        m[i].load(s0);
        __builtin_amdgcn_sched_barrier(0);
        m[i].fold(s0);
      }
      const f32x4 z = m[i].finish();
      if (a.z_out && blockIdx.x == 0) *reinterpret_cast<f32x4*>(a.z_out + (size_t)b * KDIM + k) = z;
      *reinterpret_cast<f32x4*>(zs + row * ZST + k) = z;
    } else if (u < TASKS) {
      *reinterpret_cast<f32x4*>(zs + row * ZST + k) = f32x4{0.f, 0.f, 0.f, 0.f};  // rows past the batch
    }
  }
  lds_barrier();
  if (wave >= MP_WAVES) return;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const float* zp = zs + n * ZST + 32 * kb + 8 * qd;
    const f32x4 lo4 = *reinterpret_cast<const f32x4*>(zp), hi4 = *reinterpret_cast<const f32x4*>(zp + 4);
    const float x[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    bf16x8 af, al;
    split_bf16x8(x, af, al);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bfr[kb], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bfr[kb], acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int r = row0 + 4 * qd + e;
    if (r < a.rows) a.out[(size_t)r * a.n + col] = acc[e];
  }
}

}  // namespace

template <int KB>
void launch_mr(const MergeProjectArgs& a, hipStream_t st) {
  const dim3 grid(a.n / MP_COLS, (a.rows + MR_ROWS - 1) / MR_ROWS);
  // sixteen waves: one merge task a thread at contractions up to 256 (the
  // last eight waves only merge); measured 7.8-8.0 against 8.25 us at the
  // 70B 128K share, 5.3-5.5 against 5.6 at the ragged mix.
  // BASISKV_MR_WAVES=8 overrides (a tuning override)
  static const int nw = [] {
    const char* e = getenv("BASISKV_MR_WAVES");
    return e && atoi(e) == 8 ? 8 : 16;
  }();
  const size_t lds = (size_t)MR_ROWS * (32 * KB + 4) * sizeof(float);
  if (nw == 16) hipLaunchKernelGGL((merge_project_rows_kernel<KB, 16>), grid, dim3(64 * 16), lds, st, a);
  else hipLaunchKernelGGL((merge_project_rows_kernel<KB, 8>), grid, dim3(64 * 8), lds, st, a);
}

template <int KB>
void launch_mp(const MergeProjectArgs& a, dim3 grid, hipStream_t st) {
  hipLaunchKernelGGL(merge_project_kernel<KB>, grid, dim3(64 * MP_WAVES), (size_t)MP_ROWS * (32 * KB + 4) * sizeof(float),
                     st, a);
}

bool merge_project_rows_supported(const Shape& s) {
  // BASISKV_MERGE_PROJECT_ROWS=0: beyond 16 rows the separate merge and
  // projection instead (a tuning override)
  static const bool off = [] {
    const char* e = getenv("BASISKV_MERGE_PROJECT_ROWS");
    return e && e[0] == '0';
  }();
  return !off && merge_project_supported(s) && s.n_q_heads * s.rank_v <= MR_KMAX;
}

hipError_t launch_merge_project_rows(const MergeProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  switch (a.kdim / 32) {  // merge_project_rows_supported: kdim % 32 == 0, kdim <= MR_KMAX
    case 1: launch_mr<1>(a, st); break;
    case 2: launch_mr<2>(a, st); break;
    case 3: launch_mr<3>(a, st); break;
    case 4: launch_mr<4>(a, st); break;
    case 5: launch_mr<5>(a, st); break;
    case 6: launch_mr<6>(a, st); break;
    case 7: launch_mr<7>(a, st); break;
    case 8: launch_mr<8>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  const dim3 grid(a.n / MP_COLS, (a.rows + MP_ROWS - 1) / MP_ROWS);
  switch (a.kdim / 32) {  // merge_project_supported: kdim % 32 == 0, kdim <= MP_KMAX
    case 1: launch_mp<1>(a, grid, st); break;
    case 2: launch_mp<2>(a, grid, st); break;
    case 3: launch_mp<3>(a, grid, st); break;
    case 4: launch_mp<4>(a, grid, st); break;
    case 5: launch_mp<5>(a, grid, st); break;
    case 6: launch_mp<6>(a, grid, st); break;
    case 7: launch_mp<7>(a, grid, st); break;
    case 8: launch_mp<8>(a, grid, st); break;
    case 9: launch_mp<9>(a, grid, st); break;
    case 10: launch_mp<10>(a, grid, st); break;
    case 11: launch_mp<11>(a, grid, st); break;
    case 12: launch_mp<12>(a, grid, st); break;
    case 13: launch_mp<13>(a, grid, st); break;
    case 14: launch_mp<14>(a, grid, st); break;
    case 15: launch_mp<15>(a, grid, st); break;
    case 16: launch_mp<16>(a, grid, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool project_mfma_supported(int kdim, int n, int dtype) {
  return dtype == 1 && kdim % 32 == 0 && n % 16 == 0;
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (project_mfma_supported(a.kdim, a.n, a.dtype)) {
    if (a.rows > 64 && a.n % PT_BN == 0) {
      // LDS-staged 128x256 tiles
      // steps of 32 (or BASISKV_PROJECT_BK=64)
      static const int bk = [] {
        const char* e = getenv("BASISKV_PROJECT_BK");
        return e && atoi(e) == 64 ? 64 : 32;
      }();
      const int grid = ((a.rows + PT_BM - 1) / PT_BM) * (a.n / PT_BN);
      const void* k = bk == 32 ? (const void*)project_tiled_kernel<32> : (const void*)project_tiled_kernel<64>;
      const size_t lds = 2 * (size_t)pt_stage(bk);
      hipError_t e = allow_lds(k, lds);
      if (e != hipSuccess) return e;
      void* args[] = {const_cast<ProjectArgs*>(&a)};
      e = hipLaunchKernel(k, dim3(grid), dim3(64 * PT_WAVES), args, lds, st);
      if (e != hipSuccess) return e;
    } else if (a.rows > 64 && a.n % 128 == 0) {
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
