// Top-k page selection over the router's scores, one workgroup per
// (sequence, KV head): the standalone step behind basiskv_route and
// basiskv_append_route (the decode step selects inside the attention
// kernel instead).  See select.hpp for the rule and the method.
#include "internal.hpp"
#include "select.hpp"

namespace bkv {

namespace {

constexpr int SEL_T = 256;

__global__ __launch_bounds__(SEL_T) void select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_keys[];  // [max_pages] keys, then bins and picks
  __shared__ SelectShared sh;
  const SelectPages pg{s_keys, reinterpret_cast<uint8_t*>(s_keys + a.s.max_pages),
                       reinterpret_cast<uint8_t*>(s_keys + a.s.max_pages) + a.s.max_pages};
  const int pair = blockIdx.x;
  const int b = pair / a.s.n_kv_heads;
  const int ps = a.s.page_size, maxp = a.s.max_pages, top_k = a.s.top_k;
  const int n = a.seq_lens[b];
  const int npg = n > 0 ? min((n + ps - 1) / ps, maxp) : 0;
  const int ks = min(top_k, npg);
  const float* sc = a.scores + (size_t)pair * maxp;
  uint32_t kmax = 0u, kmin = 0xffffffffu;  // the range of the keys of pages that are not forced
  for (int s0 = 0; s0 < npg; s0 += SEL_SB * SEL_T) {
    const int ns = min(SEL_SB, (npg - s0 + SEL_T - 1) / SEL_T), j0 = s0 + threadIdx.x;  // (uniform)
    float v[SEL_SB];  // the batch's scores requested together (clamped)
#pragma unroll
    for (int u = 0; u < SEL_SB; ++u)
      if (u < ns) v[u] = sc[min(j0 + u * SEL_T, npg - 1)];
#pragma unroll
    for (int u = 0; u < SEL_SB; ++u) {
      const int j = j0 + u * SEL_T;
      if (u < ns && j < npg) {
        const uint32_t k = select_key(v[u], j < a.sink_pages || j >= npg - a.local_pages);
        s_keys[j] = k;
        if (k != 0xFFFFFFFFu) {
          kmax = max(kmax, k);
          kmin = min(kmin, k);
        }
      }
    }
  }
  int32_t* sel = a.sel + (size_t)pair * top_k;
  int32_t* selp = a.sel_phys ? a.sel_phys + (size_t)pair * top_k : nullptr;
  for (int p = ks + threadIdx.x; p < top_k; p += SEL_T) {
    sel[p] = -1;
    if (selp) selp[p] = -1;
  }
  if (threadIdx.x == 0) a.n_sel[pair] = ks;
  if (ks == 0) return;
  key_range_publish(kmax, kmin, sh);
  topk_clear(sh);
  lds_barrier();
  const TopK t = topk_find(pg, npg, ks, sh);
  const int32_t* pt = a.page_table + (size_t)b * maxp;
  auto put = [&](int p, int j) {
    if (p >= ks) return;  // (never: the cut keeps exactly ks pages)
    sel[p] = j;
    if (selp) selp[p] = pt[j];
  };
  if (t.mode == 2) topk_emit(pg, npg, t, sh, put);
  else topk_emit_masked(pg, npg, t, sh, put);
}

}  // namespace

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const size_t lds = (size_t)a.s.max_pages * 6;
  const hipError_t e = allow_lds((const void*)select_kernel, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(a.s.batch * a.s.n_kv_heads), dim3(SEL_T), lds, st, a);
  return hipGetLastError();
}

}  // namespace bkv
