// Achievable HBM read bandwidth: a measurement aid beside the method, the
// denominator the attention kernel's bytes per second are also compared
// with (spec-sheet peaks are rarely reached by streaming reads).
//
// A grid of n_sink workgroups of 256 threads walks the buffer with 16-byte
// loads, eight in flight per thread and step (consecutive threads on
// consecutive granules), and sums the words as fp32; each workgroup writes
// its sum, so nothing the loads bring in is dead.
#include "common.hpp"
#include "internal.hpp"

namespace bkv {

namespace {

constexpr int SR_THREADS = 256;

__global__ __launch_bounds__(SR_THREADS) void stream_read_kernel(const f32x4* src, size_t n16, const float* tail,
                                                                 int n_tail, float* sink) {
  const size_t tid = (size_t)blockIdx.x * SR_THREADS + threadIdx.x, nt = (size_t)gridDim.x * SR_THREADS;
  float acc = 0.f;
  size_t i = tid;
  for (; i + 7 * nt < n16; i += 8 * nt) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * nt);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (v[u][0] + v[u][1]) + (v[u][2] + v[u][3]);
  }
  for (; i < n16; i += nt) {
    const f32x4 v = __builtin_nontemporal_load(src + i);
    acc += (v[0] + v[1]) + (v[2] + v[3]);
  }
  if (tid < (size_t)n_tail) acc += tail[tid];  // the words past the last whole granule
  __shared__ float s_part[SR_THREADS / 64];
  for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < SR_THREADS / 64; ++w) t += s_part[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, int n_sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  const int n_tail = (int)((bytes % 16) / 4);
  hipLaunchKernelGGL(stream_read_kernel, dim3(n_sink), dim3(SR_THREADS), 0, st, static_cast<const f32x4*>(src),
                     n16, reinterpret_cast<const float*>(static_cast<const char*>(src) + n16 * 16), n_tail, sink);
  return hipGetLastError();
}

}  // namespace bkv
