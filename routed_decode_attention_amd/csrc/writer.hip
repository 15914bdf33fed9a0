// Cache writer and the folded output projection.
//
// weekinpapers "BasisKV: Value Latents for Communication and Key Routing",
// Abstract: a Value is kept only as its low-rank latent; the latent predicts
// part of the Key and a Key-specific residual stores what it cannot; the
// exact Key is kept for the pages routing selects.  kongchang article,
// output-projection binding: the Value basis is associated with the output
// projection, so W_of = B^T.W_O replaces reconstructing Values.
//
// One workgroup writes the tokens that fall in one page for one KV head
// (decode append: a single token; prefill chunk: up to a page of tokens),
// 16 tokens at a time through LDS:
//   z~ = round(v.B);  e = k - z~.P;  s~ = round(e.R_enc);  store k, z~, s~.
// Then it sets the page's sums to the fp32 sum, in slot order, of the stored
// z~ and s~ over slots [0, last written].  Append and chunk writes therefore
// produce identical sums, and rewriting a position is idempotent.
#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int THREADS = 256;
constexpr int TB = 16;  // tokens per LDS batch

// LDS floats the writer needs: staged B, P (row stride D+1), R_enc, then a
// batch of v, k (reused for the Key remainder) and stored latents.
size_t writer_lds_floats(const Shape& s) {
  const int D = s.head_dim, R = s.rank_v, RK = s.rank_k, ps = s.page_size;
  return (size_t)D * R + (size_t)R * lds_row(D) + (size_t)D * RK + 2 * TB * D + TB * R +
         (size_t)R * (ps + 1) + (size_t)ps * RK;
}

template <typename T>
__global__ __launch_bounds__(THREADS) void write_kernel(WriteArgs a) {
  extern __shared__ float lds[];
  const int H = a.s.n_kv_heads, D = a.s.head_dim, R = a.s.rank_v, RK = a.s.rank_k;
  const int ps = a.s.page_size;
  const int g = blockIdx.y;
  int b, t0, t1, row0;
  if (a.pos) {
    b = blockIdx.x;
    t0 = a.pos[b];
    if (t0 < 0 || t0 >= a.s.max_pages * ps) return;
    t1 = t0 + 1;
    row0 = b;  // input row of token t0
  } else {
    b = a.seq;
    const int page = a.start / ps + blockIdx.x;
    t0 = max(a.start, page * ps);
    t1 = min(a.start + a.n_tok, (page + 1) * ps);
    if (t0 >= t1) return;
    row0 = t0 - a.start;
  }
  const int LDP = lds_row(D);
  float* sB = lds;
  float* sP = sB + D * R;
  float* sRe = sP + R * LDP;
  float* s_v = sRe + D * RK;  // [TB][D]: v, then the Key remainder
  float* s_k = s_v + TB * D;  // [TB][D]
  float* s_z = s_k + TB * D;  // [TB][R] stored latents
  float* sZp = s_z + TB * R;  // [R][ps+1] the page's stored latents, for its sums
  float* sSp = sZp + R * (ps + 1);  // [ps][RK] ... and residuals
  {
    StageList L;
    L.it[0] = StageItem{sB, a.B + (size_t)g * D * R, R, D, R};
    L.it[1] = StageItem{sP, a.P + (size_t)g * R * D, LDP, R, D};
    L.it[2] = StageItem{sRe, a.R_enc + (size_t)g * D * RK, RK, D, RK};
    L.it[3] = L.it[2];
    L.n = 3;
    stage_matrices(L);
  }

  const int page = t0 / ps;
  const int phys = a.page_table[(size_t)b * a.s.max_pages + page];
  const T* kin = static_cast<const T*>(a.k);
  const T* vin = static_cast<const T*>(a.v);
  T* Kp = static_cast<T*>(a.K);
  T* Zp = static_cast<T*>(a.Z);
  T* Sp = static_cast<T*>(a.S);
  const size_t kbase = ((size_t)phys * H + g) * ps * D;
  const size_t zbase = ((size_t)phys * H + g) * R * ps;
  const size_t sbase = ((size_t)phys * H + g) * ps * RK;
  const int tid = threadIdx.x;

  for (int tb = t0; tb < t1; tb += TB) {
    const int nb = min(TB, t1 - tb);
    const int slot0 = tb - page * ps;
    for (int o = tid; o < nb * D; o += THREADS) {
      const int t = o / D, i = o % D;
      const size_t src = ((size_t)(row0 + tb - t0 + t) * H + g) * D + i;
      s_v[t * D + i] = ld_elem(vin, src);
      s_k[t * D + i] = ld_elem(kin, src);
      Kp[kbase + (size_t)(slot0 + t) * D + i] = kin[src];  // the exact Key, bit for bit
    }
    __syncthreads();
    for (int o = tid; o < nb * R; o += THREADS) {
      const int t = o / R, r = o % R;
      s_z[t * R + r] = round_store(Zp, zbase + (size_t)r * ps + slot0 + t, latent_dot(s_v + t * D, sB, D, R, r));
    }
    __syncthreads();
    for (int o = tid; o < nb * D; o += THREADS) {
      const int t = o / D, i = o % D;
      s_v[t * D + i] = key_remainder(s_k[t * D + i], s_z + t * R, sP, LDP, R, i);
    }
    __syncthreads();
    for (int o = tid; o < nb * RK; o += THREADS) {
      const int t = o / RK, j = o % RK;
      round_store(Sp, sbase + (size_t)(slot0 + t) * RK + j, residual_dot(s_v + t * D, sRe, D, RK, j));
    }
    __syncthreads();
  }

  // page sums over slots [0, last written], in slot order
  __threadfence_block();
  __syncthreads();
  const int valid = t1 - page * ps;
  stage_page(sZp, sSp, Zp + zbase, Sp + sbase, R, RK, ps);
  __syncthreads();
  for (int x = tid; x < R + RK; x += THREADS)
    a.summ[((size_t)phys * H + g) * (R + RK) + x] = page_channel_sum(sZp, sSp, R, RK, ps, x, valid);
}

// W_ofT[c][h*R + j] = round(sum_i B[g(h)][i][j] * W_O[h*D + i][c]); one block
// per (column tile, h*R + j).
template <typename T>
__global__ __launch_bounds__(THREADS) void fold_kernel(Shape s, const float* B, const T* W_O, T* W_ofT) {
  const int c = blockIdx.x * THREADS + threadIdx.x;
  const int hj = blockIdx.y;
  const int R = s.rank_v, D = s.head_dim;
  const int h = hj / R, j = hj % R, g = h / s.group;
  if (c >= s.d_model) return;
  float acc = 0.f;
  for (int i = 0; i < D; ++i)
    acc += B[((size_t)g * D + i) * R + j] * ld_elem(W_O, ((size_t)h * D + i) * s.d_model + c);
  round_store(W_ofT, (size_t)c * s.n_q_heads * R + hj, acc);
}

__global__ void zero_u32_kernel(unsigned* p, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_write(const WriteArgs& a, hipStream_t st) {
  dim3 grid;
  if (a.pos) {
    grid = dim3(a.s.batch, a.s.n_kv_heads);
  } else {
    const int ps = a.s.page_size;
    const int pages = (a.start + a.n_tok - 1) / ps - a.start / ps + 1;
    grid = dim3(pages, a.s.n_kv_heads);
  }
  const size_t lds = writer_lds_floats(a.s) * sizeof(float);
  if (a.s.dtype == 0) {
    const hipError_t e = allow_lds((const void*)write_kernel<float>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((write_kernel<float>), grid, dim3(THREADS), lds, st, a);
  } else {
    const hipError_t e = allow_lds((const void*)write_kernel<uint16_t>, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((write_kernel<uint16_t>), grid, dim3(THREADS), lds, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_fold(const Shape& s, const float* B, const void* W_O, void* W_ofT, hipStream_t st) {
  const dim3 grid((s.d_model + THREADS - 1) / THREADS, s.n_q_heads * s.rank_v);
  if (s.dtype == 0)
    hipLaunchKernelGGL((fold_kernel<float>), grid, dim3(THREADS), 0, st, s, B,
                       static_cast<const float*>(W_O), static_cast<float*>(W_ofT));
  else
    hipLaunchKernelGGL((fold_kernel<uint16_t>), grid, dim3(THREADS), 0, st, s, B,
                       static_cast<const uint16_t*>(W_O), static_cast<uint16_t*>(W_ofT));
  return hipGetLastError();
}

hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace bkv
