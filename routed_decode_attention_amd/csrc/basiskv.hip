// C-ABI host layer: argument validation, workspace planning and kernel
// launches on the caller's stream.  The library keeps no device state; the
// only global is the thread-local error text.
#include <math.h>
#include <stdlib.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>
#include <mutex>


#include "../../include/basiskv.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BASISKV_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- debug mode (environment BASISKV_DEBUG=1): before its kernels, a call
// checks the device data it is about to read and returns BASISKV_E_DATA on a
// violation, with nothing else enqueued.  It synchronises the stream, so it
// is not for graph capture. ----
__device__ unsigned g_validate_flag;

bool debug_on() {
  const char* e = getenv("BASISKV_DEBUG");
  return e && e[0] == '1';
}

bkv::ValidateArgs validate_args(const bkv::Shape& s, const basiskv_cache* c) {
  bkv::ValidateArgs v = {};
  v.rows = s.batch;
  v.max_pages = s.max_pages;
  v.page_size = s.page_size;
  v.num_phys = s.num_pages;
  v.top_k = s.top_k;
  v.n_kv_heads = bkv::unit_shape(s).n_kv_heads;  // selection units per row
  v.page_table = c->page_table;
  return v;
}

int debug_check(bkv::ValidateArgs v, void* stream, const char* who) {
  if (!debug_on()) return BASISKV_OK;
  // one flag per device: checks from several host threads take turns
  static std::mutex mu;
  const std::lock_guard<std::mutex> lock(mu);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetSymbolAddress(reinterpret_cast<void**>(&v.flag), HIP_SYMBOL(g_validate_flag));
  if (e == hipSuccess) e = bkv::launch_zero_u32(v.flag, 1, st);
  if (e == hipSuccess) e = bkv::launch_validate(v, st);
  unsigned bits = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&bits, v.flag, sizeof bits, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "debug check");
  if (!bits) return BASISKV_OK;
  return fail(BASISKV_E_DATA, "%s: invalid device data:%s%s%s%s%s", who,
              bits & bkv::VALIDATE_SEQ_LEN ? " a sequence length out of range;" : "",
              bits & bkv::VALIDATE_PAGE ? " a page-table entry out of range;" : "",
              bits & bkv::VALIDATE_APPEND_PAGE ? " an append position's page unmapped;" : "",
              bits & bkv::VALIDATE_COUNT ? " a selection count outside [0, top_k];" : "",
              bits & bkv::VALIDATE_SELECTION ? " a selected page outside its sequence or pool;" : "");
}

// Validate dims and fill the kernels' shape.  Returns BASISKV_OK or an error.
int check_dims(const basiskv_dims* d, bkv::Shape* s) {
  if (!d) return fail(BASISKV_E_NULL, "dims is NULL");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->head_dim < 1 ||
      d->rank_v < 1 || d->rank_k < 1 || d->page_size < 1 || d->d_model < 1 || d->top_k < 1 ||
      d->max_pages_per_seq < 1 || d->num_phys_pages < 1)
    return fail(BASISKV_E_DIMS, "every dimension must be positive");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(BASISKV_E_DIMS, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if (d->rank_v > d->head_dim || d->rank_k > d->head_dim)
    return fail(BASISKV_E_DIMS, "ranks must not exceed head_dim");
  if (d->top_k > d->max_pages_per_seq)
    return fail(BASISKV_E_DIMS, "top_k (%d) exceeds max_pages_per_seq (%d)", d->top_k,
                d->max_pages_per_seq);
  if (d->dtype != BASISKV_F32 && d->dtype != BASISKV_BF16)
    return fail(BASISKV_E_DIMS, "unknown dtype %d", d->dtype);
  if (!(d->softmax_scale >= 0.f) || !isfinite(d->softmax_scale))
    return fail(BASISKV_E_DIMS, "softmax_scale must be finite and >= 0");
  if (d->sink_pages < 0 || d->local_pages < 0)
    return fail(BASISKV_E_DIMS, "sink_pages %d and local_pages %d must be >= 0", d->sink_pages, d->local_pages);
  if (d->group_mean != 0 && d->group_mean != 1) return fail(BASISKV_E_DIMS, "group_mean %d (0 or 1)", d->group_mean);
  if (d->head_select != 0 && d->head_select != 1) return fail(BASISKV_E_DIMS, "head_select %d (0 or 1)", d->head_select);
  const int group = d->n_q_heads / d->n_kv_heads;
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(BASISKV_E_UNSUPPORTED, "head_dim %d (supported: 64, 128)", d->head_dim);
  if (d->page_size != 16 && d->page_size != 32 && d->page_size != 64)
    return fail(BASISKV_E_UNSUPPORTED, "page_size %d (supported: 16, 32, 64)", d->page_size);
  if (d->rank_v % 16 != 0 || d->rank_v > bkv::MAX_RANK)
    return fail(BASISKV_E_UNSUPPORTED, "rank_v %d (multiple of 16, at most 64)", d->rank_v);
  if (d->rank_k % 4 != 0 || d->rank_k > bkv::MAX_RESID)
    return fail(BASISKV_E_UNSUPPORTED, "rank_k %d (multiple of 4, at most 64)", d->rank_k);
  if (group > bkv::MAX_GROUP)
    return fail(BASISKV_E_UNSUPPORTED, "%d query heads per KV head (at most 16)", group);
  if (d->max_pages_per_seq > bkv::MAX_PAGES)
    return fail(BASISKV_E_UNSUPPORTED, "max_pages_per_seq %d (at most %d)", d->max_pages_per_seq,
                bkv::MAX_PAGES);
  s->batch = d->batch;
  s->n_q_heads = d->n_q_heads;
  s->n_kv_heads = d->n_kv_heads;
  s->group = group;
  s->head_dim = d->head_dim;
  s->rank_v = d->rank_v;
  s->rank_k = d->rank_k;
  s->page_size = d->page_size;
  s->d_model = d->d_model;
  s->top_k = d->top_k;
  s->max_pages = d->max_pages_per_seq;
  s->num_pages = d->num_phys_pages;
  s->dtype = d->dtype;
  s->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->head_dim);
  s->cache_heads = d->n_kv_heads;
  s->unit_div = 1;
  s->head_select = d->head_select;
  return BASISKV_OK;
}

struct WsLayout {
  size_t part_acc, part_ml, z, pf_acc, pf_ml, total;
};

// Workspace: the attention splits' partials (latent sums, then max /
// denominator pairs), then latent rows (decode batch or prefill chunk), then
// (with prefill tokens) the prefill key ranges' partials.  Nothing in it
// carries over between calls.
WsLayout ws_layout(const bkv::Shape& s0, int max_prefill_tokens) {
  const bkv::Shape s = bkv::unit_shape(s0);
  const size_t pairs = (size_t)s.batch * s.n_kv_heads;
  const bkv::AttendPlan p = bkv::plan_attend(s);
  const size_t splits = pairs * p.n_wsplit * s.group;
  WsLayout L;
  L.part_acc = 0;
  L.part_ml = L.part_acc + align256(splits * s.rank_v * sizeof(float));
  L.z = L.part_ml + align256(splits * 2 * sizeof(float));
  size_t rows = (size_t)s.batch;
  if (max_prefill_tokens > 0 && (size_t)max_prefill_tokens > rows) rows = max_prefill_tokens;
  L.pf_acc = L.z + align256(rows * s.n_q_heads * s.rank_v * sizeof(float));
  const size_t pf_rows = max_prefill_tokens > 0 ? (size_t)max_prefill_tokens * s.n_q_heads * bkv::PREFILL_KSPLIT_MAX : 0;
  L.pf_ml = L.pf_acc + align256(pf_rows * s.rank_v * sizeof(float));
  L.total = L.pf_ml + align256(pf_rows * 2 * sizeof(float));
  return L;
}

int check_cache(const basiskv_cache* c, bool needs_k, bool needs_z, bool needs_s) {
  if (!c) return fail(BASISKV_E_NULL, "cache is NULL");
  if (!c->page_table || !c->summ || (needs_k && !c->K) || (needs_z && !c->Z) || (needs_s && !c->S))
    return fail(BASISKV_E_NULL, "a cache pointer is NULL");
  return BASISKV_OK;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Attention over the selection.  Several splits leave their partials in the
// workspace; with `merge` they are combined into z_out right away, otherwise
// the caller consumes them (the fused merge + projection).
// Selection done by the attention kernel's prologue (the decode step).
struct PrologueSelect {
  const float* scores = nullptr;
  int32_t *sel = nullptr, *n_sel = nullptr;
  int sink_pages = 0, local_pages = 0;
};

int do_attend(const bkv::Shape& s0, const basiskv_cache* cache, const int32_t* seq_lens, const void* q,
              const int32_t* sel, const int32_t* n_sel, void* ws, size_t ws_bytes, float* z_out,
              void* stream, const int32_t* sel_phys, bool merge, const PrologueSelect& ps = PrologueSelect()) {
  const bkv::Shape s = bkv::unit_shape(s0);  // pairs are selection units
  const WsLayout L = ws_layout(s, 0);
  if (ws_bytes < L.z)
    return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, attention needs %zu", ws_bytes, L.z);
  bkv::AttendArgs a;
  a.s = s;
  a.K = cache->K;
  a.Z = cache->Z;
  a.page_table = cache->page_table;
  a.seq_lens = seq_lens;
  a.q = q;
  a.sel = sel;
  a.n_sel = n_sel;
  a.sel_phys = sel_phys;
  a.scores = ps.scores;
  a.sel_out = ps.sel;
  a.n_sel_out = ps.n_sel;
  a.sink_pages = ps.sink_pages;
  a.local_pages = ps.local_pages;
  char* w = static_cast<char*>(ws);
  a.part_acc = reinterpret_cast<float*>(w + L.part_acc);
  a.part_ml = reinterpret_cast<float*>(w + L.part_ml);
  a.z_out = z_out;
  const bkv::AttendPlan p = bkv::plan_attend(s);
  a.n_wsplit = p.n_wsplit;
  a.pages_per_wave = p.pages_per_wave;
  a.waves = p.waves;
  a.scale_log2 = s.scale * 1.4426950408889634f;
  hipError_t e = bkv::launch_attend(a, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  if (merge && p.n_wsplit > 1) {
    bkv::MergeArgs m;
    m.s = s;
    m.part_acc = a.part_acc;
    m.part_ml = a.part_ml;
    m.n_wsplit = p.n_wsplit;
    m.z_out = z_out;
    e = bkv::launch_merge(m, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "split merge launch");
  }
  return BASISKV_OK;
}

int do_project(const bkv::Shape& s, const basiskv_factors* f, const float* z, int rows, float* out,
               void* stream) {
  bkv::ProjectArgs a;
  a.z = z;
  a.W = f->W_ofT;
  a.out = out;
  a.rows = rows;
  a.kdim = s.n_q_heads * s.rank_v;
  a.n = s.d_model;
  a.dtype = s.dtype;
  const hipError_t e = bkv::launch_project(a, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "projection launch");
}

// After the attention (n_wsplit splits per unit, partials at L in ws, or
// with one split the latents already in z): the merge of the splits and the
// output projection.  The fused merge-projection re-merges a row's splits in
// every column group and re-reads the weights in every row group: up to one
// MFMA row tile (16 rows) in groups of 2 rows, beyond in whole 16-row tiles
// (measured against the separate merge and projection: 70B 128K share 41.2
// against 42.2 us per step, ragged mix 35.7 against 38.2), which contractions
// over 256 still take.  s: the unit shape.
int merge_project(const bkv::Shape& s, const basiskv_factors* f, void* ws, const WsLayout& L, int n_wsplit,
                  float* z, float* z_out, float* out, void* stream) {
  char* w = static_cast<char*>(ws);
  const bool small = s.batch <= 16 && bkv::merge_project_supported(s);
  const bool rows16 = !small && bkv::merge_project_rows_supported(s);  // 16-row tiles
  const bool fused = n_wsplit > 1 && (small || rows16);
  if (!fused) {
    if (n_wsplit > 1) {
      bkv::MergeArgs m;
      m.s = s;
      m.part_acc = reinterpret_cast<const float*>(w + L.part_acc);
      m.part_ml = reinterpret_cast<const float*>(w + L.part_ml);
      m.n_wsplit = n_wsplit;
      m.z_out = z;
      const hipError_t e = bkv::launch_merge(m, as_stream(stream));
      if (e != hipSuccess) return hip_fail(e, "split merge launch");
    }
    return do_project(s, f, z, s.batch, out, stream);
  }
  bkv::MergeProjectArgs m;
  m.s = s;
  m.part_acc = reinterpret_cast<const float*>(w + L.part_acc);
  m.part_ml = reinterpret_cast<const float*>(w + L.part_ml);
  m.n_wsplit = n_wsplit;
  m.W = f->W_ofT;
  m.out = out;
  m.z_out = z_out;
  m.rows = s.batch;
  m.kdim = s.n_q_heads * s.rank_v;
  m.n = s.d_model;
  const hipError_t e = rows16 ? bkv::launch_merge_project_rows(m, as_stream(stream))
                              : bkv::launch_merge_project(m, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "merge-projection launch");
}

// Decode attention, the merge of its splits, then the output projection.
int attend_project(const bkv::Shape& s0, const basiskv_factors* f, const basiskv_cache* cache,
                   const int32_t* seq_lens, const void* q, const int32_t* sel, const int32_t* n_sel,
                   const int32_t* sel_phys, void* ws, size_t ws_bytes, float* z_out, float* out, void* stream,
                   const PrologueSelect& psel = PrologueSelect()) {
  const bkv::Shape s = bkv::unit_shape(s0);
  const WsLayout L = ws_layout(s, 0);
  float* z = z_out ? z_out : reinterpret_cast<float*>(static_cast<char*>(ws) + L.z);
  // the splits' partials stay in the workspace for merge_project
  const int rc = do_attend(s, cache, seq_lens, q, sel, n_sel, ws, ws_bytes, z, stream, sel_phys, false, psel);
  if (rc) return rc;
  return merge_project(s, f, ws, L, bkv::plan_attend(s).n_wsplit, z, z_out, out, stream);
}

int do_write(const bkv::Shape& s, const basiskv_factors* f, const basiskv_cache* c, const int32_t* pos,
             int seq, int start, int n_tok, const void* k, const void* v, void* stream) {
  bkv::WriteArgs a;
  a.s = s;
  a.B = f->B;
  a.P = f->P;
  a.R_enc = f->R_enc;
  a.K = c->K;
  a.Z = c->Z;
  a.S = c->S;
  a.summ = c->summ;
  a.page_table = c->page_table;
  a.k = k;
  a.v = v;
  a.pos = pos;
  a.seq = seq;
  a.start = start;
  a.n_tok = n_tok;
  const hipError_t e = bkv::launch_write(a, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "writer launch");
}

// Page scores (with the append fused when pos is given), then, when sel is
// given, the top-k selection.
int do_route(const bkv::Shape& s, const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
             const int32_t* pos, const void* k_new, const void* v_new, const int32_t* seq_lens, const void* q,
             int32_t* sel, int32_t* n_sel, float* scores, int32_t* sel_phys, void* stream) {
  if (!bkv::score_fits(s, pos != nullptr))
    return fail(BASISKV_E_UNSUPPORTED, "route: the appending workgroup's factors and page image exceed the LDS");
  bkv::ScoreArgs a;
  a.s = s;
  a.B = f->B;
  a.P = f->P;
  a.R_enc = f->R_enc;
  a.R_dec = f->R_dec;
  a.K = cache->K;
  a.Z = cache->Z;
  a.S = cache->S;
  a.summ = cache->summ;
  a.page_table = cache->page_table;
  a.seq_lens = seq_lens;
  a.q = q;
  a.pos = pos;
  a.k_new = k_new;
  a.v_new = v_new;
  a.scores = scores;
  a.group_mean = dims->group_mean;
  bkv::score_plan(s, pos != nullptr, &a.cluster, &a.per);
  hipError_t e = bkv::launch_score(a, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "score launch");
  if (!sel) return BASISKV_OK;
  bkv::SelectArgs sa;
  sa.s = bkv::unit_shape(s);
  sa.scores = scores;
  sa.page_table = cache->page_table;
  sa.seq_lens = seq_lens;
  sa.sel = sel;
  sa.n_sel = n_sel;
  sa.sel_phys = sel_phys;
  sa.sink_pages = dims->sink_pages;
  sa.local_pages = dims->local_pages;
  e = bkv::launch_select(sa, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "selection launch");
}

int check_step_args(const bkv::Shape& s, const basiskv_factors* f, const basiskv_cache* cache, const int32_t* pos,
                    const void* k_new, const void* v_new, const int32_t* seq_lens, const void* q, int32_t* sel,
                    int32_t* n_sel, float* scores, float* out, const char* who) {
  if (!f || !f->B || !f->P || !f->R_enc || !f->R_dec || !f->W_ofT)
    return fail(BASISKV_E_NULL, "%s: every factor is required", who);
  int rc = check_cache(cache, true, true, true);
  if (rc) return rc;
  if (!pos || !k_new || !v_new || !seq_lens || !q || !sel || !n_sel || !scores || !out)
    return fail(BASISKV_E_NULL, "%s: a required pointer is NULL", who);
  if (bkv::attend_lds_bytes(bkv::unit_shape(s), true) > 160 * 1024)
    return fail(BASISKV_E_UNSUPPORTED, "%s: max_pages_per_seq %d needs more LDS than a CU has for the "
                "attention's selection", who, s.max_pages);
  return BASISKV_OK;
}

// The decode layer step on a checked workspace of ws_bytes >= ws_layout(s, 0).total:
// append + scores, then attention with the selection in its prologue, then
// the split merge fused with the projection.
int decode_step(const bkv::Shape& s, const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                const int32_t* pos, const void* k_new, const void* v_new, const int32_t* seq_lens, const void* q,
                int32_t* sel, int32_t* n_sel, float* scores, void* ws, size_t ws_bytes, float* z_out, float* out,
                void* stream) {
  bkv::ValidateArgs va = validate_args(s, cache);
  va.seq_lens = seq_lens;
  va.pos = pos;
  int rc = debug_check(va, stream, "decode_step");
  if (rc) return rc;
  if ((rc = do_route(s, dims, f, cache, pos, k_new, v_new, seq_lens, q, nullptr, nullptr, scores, nullptr, stream)))
    return rc;
  PrologueSelect psel;
  psel.scores = scores;
  psel.sel = sel;
  psel.n_sel = n_sel;
  psel.sink_pages = dims->sink_pages;
  psel.local_pages = dims->local_pages;
  return attend_project(s, f, cache, seq_lens, q, nullptr, nullptr, nullptr, ws, ws_bytes, z_out, out, stream, psel);
}

// ---- scratch of the no-allocation decode step: one array per device, for
// callers that cannot allocate (graph capture, allocation-free serving
// loops).  In host code `scratch` is only a stand-in for the device symbol:
// its device address is looked up once per device and used everywhere. ----
static __device__ __align__(256) unsigned char scratch[BASISKV_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;

int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "decode_step_noalloc: hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(BASISKV_E_UNSUPPORTED, "device %d (at most %d)", dev, MAX_DEVICES);
  const std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "decode_step_noalloc: hipGetSymbolAddress(scratch)");
    addr[dev] = p;
  }
  *out = addr[dev];
  return BASISKV_OK;
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int basiskv_version(void) { return BASISKV_VERSION; }

const char* basiskv_strerror(int code) {
  switch (code) {
    case BASISKV_OK: return "ok";
    case BASISKV_E_NULL: return "a required pointer is NULL";
    case BASISKV_E_DIMS: return "inconsistent or non-positive dimensions";
    case BASISKV_E_UNSUPPORTED: return "shape not supported by the kernels";
    case BASISKV_E_WORKSPACE: return "workspace too small";
    case BASISKV_E_HIP: return "HIP error";
    case BASISKV_E_DATA: return "invalid device data";
    default: return "unknown error";
  }
}

const char* basiskv_last_error(void) { return g_err; }

int basiskv_fold_output(const basiskv_dims* dims, const float* B, const void* W_O, void* W_ofT,
                        void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!B || !W_O || !W_ofT) return fail(BASISKV_E_NULL, "fold: B, W_O and W_ofT are required");
  const hipError_t e = bkv::launch_fold(s, B, W_O, W_ofT, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "fold launch");
}

int basiskv_write(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                  int32_t seq, int32_t start, int32_t n_tok, const void* k, const void* v,
                  void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!f || !f->B || !f->P || !f->R_enc) return fail(BASISKV_E_NULL, "write: factors B, P, R_enc required");
  if ((rc = check_cache(cache, true, true, true))) return rc;
  if (n_tok < 0 || start < 0 || seq < 0 || seq >= s.batch)
    return fail(BASISKV_E_DIMS, "write: seq %d, start %d, n_tok %d out of range", seq, start, n_tok);
  if (n_tok == 0) return BASISKV_OK;
  if (!k || !v) return fail(BASISKV_E_NULL, "write: k and v are required");
  if ((int64_t)start + n_tok > (int64_t)s.max_pages * s.page_size)
    return fail(BASISKV_E_DIMS, "write: tokens beyond max_pages_per_seq * page_size");
  bkv::ValidateArgs va = validate_args(s, cache);
  va.rows = 1;
  va.chunk_seq = seq;
  va.chunk_first = start / s.page_size;
  va.chunk_pages = (start + n_tok - 1) / s.page_size - va.chunk_first + 1;
  if ((rc = debug_check(va, stream, "write"))) return rc;
  return do_write(s, f, cache, nullptr, seq, start, n_tok, k, v, stream);
}

int basiskv_append(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                   const int32_t* pos, const void* k_new, const void* v_new, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!f || !f->B || !f->P || !f->R_enc) return fail(BASISKV_E_NULL, "append: factors B, P, R_enc required");
  if ((rc = check_cache(cache, true, true, true))) return rc;
  if (!pos || !k_new || !v_new) return fail(BASISKV_E_NULL, "append: pos, k_new and v_new are required");
  bkv::ValidateArgs va = validate_args(s, cache);
  va.pos = pos;
  if ((rc = debug_check(va, stream, "append"))) return rc;
  return do_write(s, f, cache, pos, 0, 0, 1, k_new, v_new, stream);
}

int basiskv_route(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                  const int32_t* seq_lens, const void* q, int32_t* sel, int32_t* n_sel, float* scores,
                  int32_t* sel_phys, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!f || !f->P || !f->R_dec) return fail(BASISKV_E_NULL, "route: factors P and R_dec required");
  if ((rc = check_cache(cache, false, false, false))) return rc;
  if (!seq_lens || !q || !scores) return fail(BASISKV_E_NULL, "route: seq_lens, q and scores are required");
  if (!sel != !n_sel || (!sel && sel_phys))
    return fail(BASISKV_E_NULL, "route: sel and n_sel are both given or both NULL (then sel_phys is NULL)");
  bkv::ValidateArgs va = validate_args(s, cache);
  va.seq_lens = seq_lens;
  if ((rc = debug_check(va, stream, "route"))) return rc;
  return do_route(s, dims, f, cache, nullptr, nullptr, nullptr, seq_lens, q, sel, n_sel, scores, sel_phys, stream);
}

int basiskv_append_route(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                         const int32_t* pos, const void* k_new, const void* v_new, const int32_t* seq_lens,
                         const void* q, int32_t* sel, int32_t* n_sel, float* scores, int32_t* sel_phys,
                         void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!f || !f->B || !f->P || !f->R_enc || !f->R_dec)
    return fail(BASISKV_E_NULL, "append_route: factors B, P, R_enc and R_dec required");
  if ((rc = check_cache(cache, true, true, true))) return rc;
  if (!pos || !k_new || !v_new || !seq_lens || !q || !scores)
    return fail(BASISKV_E_NULL, "append_route: pos, k_new, v_new, seq_lens, q and scores are required");
  if (!sel != !n_sel || (!sel && sel_phys))
    return fail(BASISKV_E_NULL, "append_route: sel and n_sel are both given or both NULL (then sel_phys is NULL)");
  bkv::ValidateArgs va = validate_args(s, cache);
  va.seq_lens = seq_lens;
  va.pos = pos;
  if ((rc = debug_check(va, stream, "append_route"))) return rc;
  return do_route(s, dims, f, cache, pos, k_new, v_new, seq_lens, q, sel, n_sel, scores, sel_phys, stream);
}

size_t basiskv_workspace_bytes(const basiskv_dims* dims, int32_t max_prefill_tokens) {
  bkv::Shape s;
  if (check_dims(dims, &s)) return 0;
  return ws_layout(s, max_prefill_tokens).total;
}

int basiskv_workspace_init(const basiskv_dims* dims, void* ws, size_t ws_bytes, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!ws) return fail(BASISKV_E_NULL, "workspace is NULL");
  const WsLayout L = ws_layout(s, 0);
  if (ws_bytes < L.total) return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, needs %zu", ws_bytes, L.total);
  const hipError_t e = bkv::launch_zero_u32(static_cast<unsigned*>(ws), ws_bytes / sizeof(unsigned),
                                            as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "workspace init");
}

int basiskv_attend(const basiskv_dims* dims, const basiskv_cache* cache, const int32_t* seq_lens,
                   const void* q, const int32_t* sel, const int32_t* n_sel, const int32_t* sel_phys, void* ws,
                   size_t ws_bytes, float* z_out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = check_cache(cache, true, true, false))) return rc;
  if (!seq_lens || !q || !sel || !n_sel || !ws)
    return fail(BASISKV_E_NULL, "attend: seq_lens, q, sel, n_sel and ws are required");
  if (ws_bytes < ws_layout(s, 0).z)
    return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, attention needs %zu", ws_bytes, ws_layout(s, 0).z);
  bkv::ValidateArgs va = validate_args(s, cache);
  va.seq_lens = seq_lens;
  va.sel = sel;
  va.n_sel = n_sel;
  va.sel_phys = sel_phys;
  if ((rc = debug_check(va, stream, "attend"))) return rc;
  return do_attend(s, cache, seq_lens, q, sel, n_sel, ws, ws_bytes, z_out, stream, sel_phys, z_out != nullptr);
}

int basiskv_attend_splits(const basiskv_dims* dims) {
  bkv::Shape s;
  const int rc = check_dims(dims, &s);
  if (rc) return rc;
  return bkv::plan_attend(bkv::unit_shape(s)).n_wsplit;
}

int basiskv_project(const basiskv_dims* dims, const basiskv_factors* f, const float* z, int32_t rows,
                    float* out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (rows < 0) return fail(BASISKV_E_DIMS, "project: rows %d", rows);
  if (!f || !f->W_ofT || !z || !out) return fail(BASISKV_E_NULL, "project: W_ofT, z and out are required");
  return do_project(s, f, z, rows, out, stream);
}

int basiskv_decode(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                   const int32_t* seq_lens, const void* q, const int32_t* sel, const int32_t* n_sel,
                   const int32_t* sel_phys, void* ws, size_t ws_bytes, float* z_out, float* out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = check_cache(cache, true, true, false))) return rc;
  if (!f || !f->W_ofT) return fail(BASISKV_E_NULL, "decode: W_ofT is required");
  if (!seq_lens || !q || !sel || !n_sel || !ws || !out)
    return fail(BASISKV_E_NULL, "decode: seq_lens, q, sel, n_sel, ws and out are required");
  const WsLayout L = ws_layout(s, 0);
  if (ws_bytes < L.total)
    return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, decode needs %zu", ws_bytes, L.total);
  bkv::ValidateArgs va = validate_args(s, cache);
  va.seq_lens = seq_lens;
  va.sel = sel;
  va.n_sel = n_sel;
  va.sel_phys = sel_phys;
  if ((rc = debug_check(va, stream, "decode"))) return rc;
  return attend_project(s, f, cache, seq_lens, q, sel, n_sel, sel_phys, ws, ws_bytes, z_out, out, stream);
}

int basiskv_decode_step(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                        const int32_t* pos, const void* k_new, const void* v_new, const int32_t* seq_lens,
                        const void* q, int32_t* sel, int32_t* n_sel, float* scores, void* ws, size_t ws_bytes,
                        float* z_out, float* out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = check_step_args(s, f, cache, pos, k_new, v_new, seq_lens, q, sel, n_sel, scores, out, "decode_step")))
    return rc;
  if (!ws) return fail(BASISKV_E_NULL, "decode_step: ws is required");
  const WsLayout L = ws_layout(s, 0);
  if (ws_bytes < L.total)
    return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, decode needs %zu", ws_bytes, L.total);
  return decode_step(s, dims, f, cache, pos, k_new, v_new, seq_lens, q, sel, n_sel, scores, ws, ws_bytes, z_out,
                     out, stream);
}

int basiskv_decode_step_noalloc(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                                const int32_t* pos, const void* k_new, const void* v_new, const int32_t* seq_lens,
                                const void* q, int32_t* sel, int32_t* n_sel, float* scores, float* z_out,
                                float* out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if ((rc = check_step_args(s, f, cache, pos, k_new, v_new, seq_lens, q, sel, n_sel, scores, out,
                            "decode_step_noalloc")))
    return rc;
  const WsLayout L = ws_layout(s, 0);
  if (L.total > BASISKV_NOALLOC_SCRATCH_BYTES)
    return fail(BASISKV_E_WORKSPACE, "decode_step_noalloc: these dims need %zu bytes of scratch, the library "
                "holds %zu per device (use basiskv_decode_step with a workspace)", L.total,
                (size_t)BASISKV_NOALLOC_SCRATCH_BYTES);
  // nothing in the array needs to start at any value: every byte a call
  // reads it has written before, in the same call
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return decode_step(s, dims, f, cache, pos, k_new, v_new, seq_lens, q, sel, n_sel, scores, ws, L.total, z_out,
                     out, stream);
}

int basiskv_stream_read(const void* src, size_t bytes, float* sink, int32_t n_sink, void* stream) {
  if (!src || !sink) return fail(BASISKV_E_NULL, "stream_read: src and sink are required");
  if (bytes % 4 != 0 || n_sink < 1 || (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return fail(BASISKV_E_DIMS, "stream_read: bytes %zu (multiple of 4), n_sink %d (>= 1), src 16-byte aligned",
                bytes, (int)n_sink);
  const hipError_t e = bkv::launch_stream_read(src, bytes, sink, n_sink, as_stream(stream));
  return e == hipSuccess ? BASISKV_OK : hip_fail(e, "stream-read launch");
}

int basiskv_prefill(const basiskv_dims* dims, const basiskv_factors* f, const basiskv_cache* cache,
                    int32_t seq, int32_t start_pos, int32_t n_tok, const void* q, const void* k,
                    const void* v, void* ws, size_t ws_bytes, float* z_out, float* out, void* stream) {
  bkv::Shape s;
  int rc = check_dims(dims, &s);
  if (rc) return rc;
  if (!f || !f->B || !f->P || !f->R_enc || !f->W_ofT)
    return fail(BASISKV_E_NULL, "prefill: factors B, P, R_enc and W_ofT are required");
  if ((rc = check_cache(cache, true, true, true))) return rc;
  if (n_tok < 0 || start_pos < 0 || seq < 0 || seq >= s.batch)
    return fail(BASISKV_E_DIMS, "prefill: seq %d, start %d, n_tok %d out of range", seq, start_pos, n_tok);
  if ((int64_t)start_pos + n_tok > (int64_t)s.max_pages * s.page_size)
    return fail(BASISKV_E_DIMS, "prefill: tokens beyond max_pages_per_seq * page_size");
  if (n_tok == 0) return BASISKV_OK;
  if (!q || !k || !v || !out || !ws) return fail(BASISKV_E_NULL, "prefill: q, k, v, ws and out are required");
  const WsLayout L = ws_layout(s, n_tok);
  if (ws_bytes < L.total)
    return fail(BASISKV_E_WORKSPACE, "workspace of %zu bytes, a %d-token prefill needs %zu", ws_bytes,
                n_tok, L.total);
  bkv::ValidateArgs va = validate_args(s, cache);
  va.rows = 1;
  va.chunk_seq = seq;
  va.chunk_first = 0;  // the chunk attends to every earlier page of its row
  va.chunk_pages = (start_pos + n_tok - 1) / s.page_size + 1;
  if ((rc = debug_check(va, stream, "prefill"))) return rc;
  if ((rc = do_write(s, f, cache, nullptr, seq, start_pos, n_tok, k, v, stream))) return rc;
  float* z = z_out ? z_out : reinterpret_cast<float*>(static_cast<char*>(ws) + L.z);
  bkv::PrefillArgs a;
  a.s = s;
  a.K = cache->K;
  a.Z = cache->Z;
  a.page_table = cache->page_table;
  a.q = q;
  a.z_out = z;
  a.seq = seq;
  a.start = start_pos;
  a.n_tok = n_tok;
  a.scale_log2 = s.scale * 1.4426950408889634f;
  bkv::plan_prefill(s, start_pos, n_tok, &a.n_ksplit, &a.split_pages);
  a.part_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + L.pf_acc);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) + L.pf_ml);
  const hipError_t e = bkv::launch_prefill_attend(a, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill attention launch");
  return do_project(s, f, z, n_tok, out, stream);
}

}  // extern "C"
#pragma GCC visibility pop
