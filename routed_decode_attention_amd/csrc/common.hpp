// Device helpers shared by the gfx950 kernels of the routed latent decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bkv {

// A value the same in every lane, moved to a scalar register so that the
// compiler treats branches on it as uniform.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (quiet NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}


// Storage element access: T is float (fp32 storage) or uint16_t (bf16 storage).
__device__ __forceinline__ float ld_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float ld_elem(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ float round_store(float* p, size_t i, float x) {
  p[i] = x;
  return x;
}
__device__ __forceinline__ float round_store(uint16_t* p, size_t i, float x) {
  uint16_t h = f32_to_bf16(x);
  p[i] = h;
  return bf16_to_f32(h);
}
__device__ __forceinline__ float round_only(float x, const float*) { return x; }
__device__ __forceinline__ float round_only(float x, const uint16_t*) {
  return bf16_to_f32(f32_to_bf16(x));
}

// Element k of a 16-byte chunk of storage-dtype values, as fp32.
template <typename T>
__device__ __forceinline__ float unpack_elem(const u32x4& w, int k) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t x = w[k >> 1];
    return __uint_as_float(((k & 1) ? (x >> 16) : (x & 0xffffu)) << 16);
  } else {
    return __uint_as_float(w[k]);
  }
}

// Store a value that is exactly representable in the storage dtype.
__device__ __forceinline__ void store_elem(float* p, size_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store_elem(uint16_t* p, size_t i, float x) {
  p[i] = static_cast<uint16_t>(__float_as_uint(x) >> 16);
}

// 16-byte global load as an MFMA bf16x8 operand.
__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// Eight fp32 -> an MFMA bf16x8 operand with the hardware's packed
// round-to-nearest-even conversion (one instruction per pair).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ bf16x8 pack_bf16x8(const float (&x)[8]) {
  u32x4 v;
  v[0] = cvt_pk_bf16(x[0], x[1]);
  v[1] = cvt_pk_bf16(x[2], x[3]);
  v[2] = cvt_pk_bf16(x[4], x[5]);
  v[3] = cvt_pk_bf16(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, v);
}
// Element e of a packed bf16x8 as fp32.
__device__ __forceinline__ float bf16x8_elem(const bf16x8& v, int e) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
  const uint32_t w = u[e >> 1];
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}
// x split into a bf16 high part and the bf16 rounding of the remainder.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  hi = pack_bf16x8(x);
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = x[e] - bf16x8_elem(hi, e);
  lo = pack_bf16x8(r);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 v = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, v);
}

// Max / sum of x over lanes l and l ^ 16 (16: rows of 16 lanes) or l ^ 32
// (32: wave halves), with gfx950's lane-half swaps instead of LDS permutes;
// both lanes of a pair get the same bits.
template <int M>
__device__ __forceinline__ float pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int M>
__device__ __forceinline__ float pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                         : __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Inclusive prefix sum across the 64 lanes of a wave: shifts within each
// 16-lane row on the DPP path, then the rows' totals added from scalar reads.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & (WAVE - 1);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47);
  return x + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key);
// -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint32_t float_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Intra-wave LDS hand-off: the wave's LDS writes are complete and visible to
// its other lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Workgroup barrier that orders LDS only: the wave's LDS accesses complete
// before it, while its global loads stay in flight across it (a plain
// __syncthreads also waits for every outstanding global load).  LDS filled
// by direct global -> LDS copies may be read after it only when every wave
// has waited for its copies (vmcnt) before arriving.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// A wave-uniform 32-bit load of data the kernel never writes, through the
// scalar cache (constant address space): it is counted by lgkmcnt, so waiting
// for it does not also wait for the wave's vector loads and direct copies,
// which vmcnt counts in issue order.
__device__ __forceinline__ int32_t load_uniform(const int32_t* p, int i) {
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  // (global memory has the same address in the constant address space)
  return reinterpret_cast<const_i32_ptr>(reinterpret_cast<uintptr_t>(p))[uniform(i)];
}

// Wait until every global load (and direct global -> LDS copy) this wave
// issued has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Map a linear workgroup id so that consecutive "logical" ids owned by one
// unit land on the same XCD: the hardware deals workgroups round-robin over
// the 8 XCDs, so logical id L is placed at a physical id with the same
// residue modulo 8 as its unit.  Only used when count % 8 == 0.
__device__ __forceinline__ int xcd_remap(int phys, int count) {
  if ((count & 7) != 0) return phys;
  const int per = count >> 3;
  return (phys & 7) * per + (phys >> 3);
}

}  // namespace bkv
