// Debug-mode check of the device data a call is about to read: sequence
// lengths, the page-table entries of every page those lengths (or an
// append position, or a chunk) reach, and a given selection.  Runs before
// the call's kernels, only when the host layer's debug switch is on; each
// kind of violation sets one bit of *flag.
#include "common.hpp"
#include "internal.hpp"

namespace bkv {

namespace {

__device__ __forceinline__ bool phys_ok(int p, int num_phys) { return p >= 0 && p < num_phys; }

// one workgroup per sequence row; the chunk is checked by workgroup 0
__global__ __launch_bounds__(256) void validate_kernel(ValidateArgs v) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int cap = v.max_pages * v.page_size;
  const int32_t* pt = v.page_table + (size_t)b * v.max_pages;
  unsigned bits = 0;
  int npg = 0;
  if (v.seq_lens) {
    const int n = v.seq_lens[b];
    if (n < 0 || n > cap) bits |= VALIDATE_SEQ_LEN;
    npg = n > 0 ? min((n + v.page_size - 1) / v.page_size, v.max_pages) : 0;
    for (int j = tid; j < npg; j += blockDim.x)
      if (!phys_ok(pt[j], v.num_phys)) bits |= VALIDATE_PAGE;
  }
  if (v.pos && tid == 0) {
    const int p = v.pos[b];
    if (p >= 0 && p < cap && !phys_ok(pt[p / v.page_size], v.num_phys)) bits |= VALIDATE_APPEND_PAGE;
  }
  if (v.sel) {
    for (int h = 0; h < v.n_kv_heads; ++h) {
      const size_t pair = (size_t)b * v.n_kv_heads + h;
      const int k = v.n_sel[pair];
      if (k < 0 || k > v.top_k) {
        bits |= VALIDATE_COUNT;
        continue;
      }
      for (int i = tid; i < k; i += blockDim.x) {
        const int j = v.sel[pair * v.top_k + i];
        if (j < 0 || j >= npg) bits |= VALIDATE_SELECTION;
        else if (!phys_ok(pt[j], v.num_phys)) bits |= VALIDATE_PAGE;
        if (v.sel_phys && !phys_ok(v.sel_phys[pair * v.top_k + i], v.num_phys)) bits |= VALIDATE_SELECTION;
      }
    }
  }
  if (b == 0 && v.chunk_pages > 0) {
    const int32_t* row = v.page_table + (size_t)v.chunk_seq * v.max_pages;
    for (int j = v.chunk_first + tid; j < v.chunk_first + v.chunk_pages; j += blockDim.x)
      if (!phys_ok(row[j], v.num_phys)) bits |= VALIDATE_PAGE;
  }
  if (bits) atomicOr(v.flag, bits);
}

}  // namespace

hipError_t launch_validate(const ValidateArgs& v, hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(v.rows), dim3(256), 0, st, v);
  return hipGetLastError();
}

}  // namespace bkv
