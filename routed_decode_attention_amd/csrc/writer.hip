// Cache writer and the folded output projection.
//
// weekinpapers "BasisKV: Value Latents for Communication and Key Routing",
// Abstract: a Value is kept only as its low-rank latent; the latent predicts
// part of the Key and a Key-specific residual stores what it cannot; the
// exact Key is kept for the pages routing selects.  kongchang article,
// output-projection binding: the Value basis is associated with the output
// projection, so W_of = B^T.W_O replaces reconstructing Values.
//
// Per token, on one wave:
//   z~ = round(v.B);  e = k - z~.P;  s~ = round(e.R_enc);  store k, z~, s~.
// Then each touched page's sums over slots [0, last written] are set from
// scratch.  Each of a token's products is taken in four fixed parts of its
// contraction, added in part order; the fused decode-step append computes
// the parts on four waves at once and adds them in the same order, so append
// and chunk writes are bit-identical, and rewriting a position is idempotent.
// Appends (one token per row): a workgroup per (row, KV head) with the
// token's page image in LDS and its sums in the same workgroup.  Chunks: one
// wave per token, sixteen tokens a workgroup (every token of a 2048-token
// chunk at once), then a second launch with one wave per touched (page, KV
// head) that sums the page from memory.
#include "common.hpp"
#include "internal.hpp"
#include "token_math.hpp"

namespace bkv {

namespace {

constexpr int THREADS = 256;
constexpr int NWAVES = THREADS / 64;
// per wave: v, k, Key remainder [D], stored values [R + RK], part buffers
constexpr int TOKEN_SCRATCH = 3 * 128 + 128 + TP * (64 + 128 + 64);

// LDS bytes: B, rotated P, R_enc (fp32), the page image (storage dtype), and
// each wave's token scratch.
size_t writer_lds_bytes(const Shape& s) {
  const size_t D = s.head_dim, R = s.rank_v, RK = s.rank_k, ps = s.page_size;
  const size_t es = s.dtype == 0 ? 4 : 2;
  return (D * R + R * D + D * RK) * 4 + (R * ps + ps * RK) * es + NWAVES * TOKEN_SCRATCH * 4;
}

template <typename T, int D>
__global__ __launch_bounds__(THREADS) void write_kernel(WriteArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int H = a.s.n_kv_heads, R = a.s.rank_v, RK = a.s.rank_k, RR = R + RK;
  const int ps = a.s.page_size;
  const int g = blockIdx.y;
  // one token: position pos[b] of row b (a negative or out-of-range position skips the row)
  const int b = blockIdx.x, row0 = b;
  const int t0 = a.pos[b];
  if (t0 < 0 || t0 >= a.s.max_pages * ps) return;
  const int t1 = t0 + 1;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int page = t0 / ps;
  const int phys = a.page_table[(size_t)b * a.s.max_pages + page];
  const T* kin = static_cast<const T*>(a.k);
  const T* vin = static_cast<const T*>(a.v);
  T* Kp = static_cast<T*>(a.K) + ((size_t)phys * H + g) * ps * D;
  T* Zp = static_cast<T*>(a.Z) + ((size_t)phys * H + g) * R * ps;
  T* Sp = static_cast<T*>(a.S) + ((size_t)phys * H + g) * ps * RK;

  float* sB = lds;            // [D][R]
  float* sP = sB + D * R;     // [R][D] rotated
  float* sRe = sP + R * D;    // [D][RK]
  T* img = reinterpret_cast<T*>(sRe + D * RK);  // the page: Z [R][ps], then S [ps][RK]
  const int nz16 = (int)(R * ps * sizeof(T) / 16), ns16 = (int)(ps * RK * sizeof(T) / 16);
  float* my = reinterpret_cast<float*>(img + (size_t)R * ps + (size_t)ps * RK) + wave * TOKEN_SCRATCH;

  {
    const char* B = reinterpret_cast<const char*>(a.B + (size_t)g * D * R);
    const char* P = reinterpret_cast<const char*>(a.P + (size_t)g * R * D);
    const char* Re = reinterpret_cast<const char*>(a.R_enc + (size_t)g * D * RK);
    const char* Zs = reinterpret_cast<const char*>(Zp);
    const char* Ss = reinterpret_cast<const char*>(Sp);
    int first = dma_stage(sB, D * R / 4, [&](int G) { return B + 16 * G; }, 0, NWAVES, wave, lane);
    first = dma_stage(sP, R * D / 4, [&](int G) { return P + 16 * rot_source(G, D); }, first, NWAVES, wave, lane);
    first = dma_stage(sRe, D * RK / 4, [&](int G) { return Re + 16 * G; }, first, NWAVES, wave, lane);
    dma_stage(img, nz16 + ns16, [&](int G) { return G < nz16 ? Zs + 16 * G : Ss + 16 * (G - nz16); }, first,
              NWAVES, wave, lane);
  }
  __syncthreads();

  T* mv = reinterpret_cast<T*>(my);  // the token's v and k, storage dtype
  T* mk = mv + D;
  float* parts = my + 3 * D + 128;
  const TokenLds<T> L{mv, mk, sB, sP, sRe, my + 2 * D, my + 3 * D, parts, parts + TP * 64, parts + TP * 192};
  for (int t = t0 + wave; t < t1; t += NWAVES) {
    const int slot = t - page * ps;
    const size_t src = ((size_t)(row0 + t - t0) * H + g) * D;
#pragma unroll
    for (int i = lane; i < D; i += 64) {
      mv[i] = vin[src + i];
      mk[i] = kin[src + i];
    }
    wave_sync();
    wave_token_values<T, D>(L, R, RK, lane);
    wave_token_store<T, D>(L, R, RK, ps, slot, Kp + (size_t)slot * D, Zp, Sp, lane);
    for (int x = lane; x < RR; x += 64) {
      if (x < R) store_elem(img, (size_t)x * ps + slot, L.st[x]);
      else store_elem(img, (size_t)R * ps + (size_t)slot * RK + (x - R), L.st[x]);
    }
    wave_sync();
  }
  __syncthreads();
  if (wave == 0)
    wave_page_sums(img, img + (size_t)R * ps, R, RK, ps, t1 - page * ps,
                   a.summ + ((size_t)phys * H + g) * RR, lane);
}

// Chunk tokens [start, start + n_tok) of row seq: one wave per token (up to
// sixteen a workgroup, as many as the LDS holds beside the factors), the
// factors staged once per workgroup; the page sums follow in
// write_sums_kernel.
constexpr int CHUNK_WAVES_MAX = 16;
constexpr size_t CU_LDS = 160 * 1024;  // gfx950
size_t chunk_factor_bytes(const Shape& s) {
  const size_t D = s.head_dim, R = s.rank_v, RK = s.rank_k;
  return (D * R + R * D + D * RK) * 4;
}
int chunk_waves(const Shape& s) {
  const size_t room = (CU_LDS - chunk_factor_bytes(s)) / (TOKEN_SCRATCH * 4);
  return (int)(room < (size_t)CHUNK_WAVES_MAX ? room : CHUNK_WAVES_MAX);
}

template <typename T, int D>
__global__ __launch_bounds__(64 * CHUNK_WAVES_MAX) void write_tokens_kernel(WriteArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int H = a.s.n_kv_heads, R = a.s.rank_v, RK = a.s.rank_k, ps = a.s.page_size;
  const int g = blockIdx.y, b = a.seq;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
  float* sB = lds;            // [D][R]
  float* sP = sB + D * R;     // [R][D] rotated
  float* sRe = sP + R * D;    // [D][RK]
  float* my = sRe + D * RK + wave * TOKEN_SCRATCH;
  {
    const char* B = reinterpret_cast<const char*>(a.B + (size_t)g * D * R);
    const char* P = reinterpret_cast<const char*>(a.P + (size_t)g * R * D);
    const char* Re = reinterpret_cast<const char*>(a.R_enc + (size_t)g * D * RK);
    int first = dma_stage(sB, D * R / 4, [&](int G) { return B + 16 * G; }, 0, nw, wave, lane);
    first = dma_stage(sP, R * D / 4, [&](int G) { return P + 16 * rot_source(G, D); }, first, nw, wave, lane);
    dma_stage(sRe, D * RK / 4, [&](int G) { return Re + 16 * G; }, first, nw, wave, lane);
  }
  const int i = blockIdx.x * nw + wave;  // this wave's token in the chunk
  T* mv = reinterpret_cast<T*>(my);               // the token's v and k, storage dtype
  T* mk = mv + D;
  if (i < a.n_tok) {
    const size_t src = ((size_t)i * H + g) * D;
#pragma unroll
    for (int x = lane; x < D; x += 64) {
      mv[x] = static_cast<const T*>(a.v)[src + x];
      mk[x] = static_cast<const T*>(a.k)[src + x];
    }
  }
  wait_vmem();  // this wave's copies of the factors
  __syncthreads();
  if (i >= a.n_tok) return;
  const int t = a.start + i, page = t / ps, slot = t - page * ps;
  const int phys = a.page_table[(size_t)b * a.s.max_pages + page];
  T* Kp = static_cast<T*>(a.K) + ((size_t)phys * H + g) * ps * D;
  T* Zp = static_cast<T*>(a.Z) + ((size_t)phys * H + g) * R * ps;
  T* Sp = static_cast<T*>(a.S) + ((size_t)phys * H + g) * ps * RK;
  float* parts = my + 3 * D + 128;
  const TokenLds<T> L{mv, mk, sB, sP, sRe, my + 2 * D, my + 3 * D, parts, parts + TP * 64, parts + TP * 192};
  wave_token_values<T, D>(L, R, RK, lane);
  wave_token_store<T, D>(L, R, RK, ps, slot, Kp + (size_t)slot * D, Zp, Sp, lane);
}

// The sums of the pages a chunk wrote, one wave per (page, KV head), over
// slots [0, last written] of the page as it is in memory.
template <typename T>
__global__ __launch_bounds__(64) void write_sums_kernel(WriteArgs a) {
  const int H = a.s.n_kv_heads, R = a.s.rank_v, RK = a.s.rank_k, ps = a.s.page_size;
  const int g = blockIdx.y, b = a.seq, page = a.start / ps + blockIdx.x;
  const int last = min(a.start + a.n_tok, (page + 1) * ps);  // one past the last slot written
  const int phys = a.page_table[(size_t)b * a.s.max_pages + page];
  const T* Zp = static_cast<const T*>(a.Z) + ((size_t)phys * H + g) * R * ps;
  const T* Sp = static_cast<const T*>(a.S) + ((size_t)phys * H + g) * ps * RK;
  wave_page_sums(Zp, Sp, R, RK, ps, last - page * ps, a.summ + ((size_t)phys * H + g) * (R + RK),
                 (int)threadIdx.x);
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
  if (!a.pos) {  // a chunk: the tokens, then the sums of the pages they touched
    const int ps = a.s.page_size;
    const int pages = (a.start + a.n_tok - 1) / ps - a.start / ps + 1;
    const int nw = chunk_waves(a.s);
    const size_t lds = chunk_factor_bytes(a.s) + (size_t)nw * TOKEN_SCRATCH * 4;
    const void* k = nullptr;
    if (a.s.dtype == 0)
      k = a.s.head_dim == 64 ? (const void*)write_tokens_kernel<float, 64> : (const void*)write_tokens_kernel<float, 128>;
    else
      k = a.s.head_dim == 64 ? (const void*)write_tokens_kernel<uint16_t, 64>
                             : (const void*)write_tokens_kernel<uint16_t, 128>;
    hipError_t e = allow_lds(k, lds);
    if (e != hipSuccess) return e;
    const dim3 grid((a.n_tok + nw - 1) / nw, a.s.n_kv_heads);
    void* args[] = {const_cast<WriteArgs*>(&a)};
    e = hipLaunchKernel(k, grid, dim3(64 * nw), args, lds, st);
    if (e != hipSuccess) return e;
    const void* ks = a.s.dtype == 0 ? (const void*)write_sums_kernel<float> : (const void*)write_sums_kernel<uint16_t>;
    return hipLaunchKernel(ks, dim3(pages, a.s.n_kv_heads), dim3(64), args, 0, st);
  }
  const dim3 grid(a.s.batch, a.s.n_kv_heads);
  const size_t lds = writer_lds_bytes(a.s);
  const void* k = nullptr;
  if (a.s.dtype == 0) k = a.s.head_dim == 64 ? (const void*)write_kernel<float, 64> : (const void*)write_kernel<float, 128>;
  else k = a.s.head_dim == 64 ? (const void*)write_kernel<uint16_t, 64> : (const void*)write_kernel<uint16_t, 128>;
  const hipError_t e = allow_lds(k, lds);
  if (e != hipSuccess) return e;
#define BKV_W(T, D) hipLaunchKernelGGL((write_kernel<T, D>), grid, dim3(THREADS), lds, st, a)
  if (a.s.dtype == 0) {
    if (a.s.head_dim == 64) BKV_W(float, 64);
    else BKV_W(float, 128);
  } else {
    if (a.s.head_dim == 64) BKV_W(uint16_t, 64);
    else BKV_W(uint16_t, 128);
  }
#undef BKV_W
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
