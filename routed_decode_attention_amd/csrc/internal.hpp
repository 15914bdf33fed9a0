// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bkv {

constexpr int MAX_GROUP = 16;      // query heads per KV head handled by one wave
constexpr int MAX_RANK = 64;       // latent width bound
constexpr int MAX_RESID = 64;      // residual width bound
constexpr int MAX_PAGES = 8192;    // page-table columns the router's LDS holds
constexpr int ATTEND_WAVES_MAX = 8;  // waves per attention workgroup (4 or 8 planned)

struct Shape {
  int batch, n_q_heads, n_kv_heads, group, head_dim, rank_v, rank_k, page_size;
  int d_model, top_k, max_pages, num_pages, dtype;
  float scale;
  // The cache pools hold cache_heads KV heads; head g of this shape reads
  // cache head g / unit_div.  As the caller gives it (head_select 0 or 1):
  // cache_heads = n_kv_heads, unit_div = 1.
  int cache_heads, unit_div;
  int head_select;  // every query head selects its own pages (see unit_shape)
};

// The shape the selection and the attention see.  With head_select every
// query head is a selection unit of its own: n_kv_heads becomes n_q_heads,
// group 1, and unit g reads cache head g / group.  Otherwise s itself.
inline Shape unit_shape(const Shape& s) {
  if (!s.head_select) return s;
  Shape u = s;
  u.n_kv_heads = s.n_q_heads;
  u.group = 1;
  u.unit_div = s.group;
  u.head_select = 0;
  return u;
}

struct WriteArgs {
  Shape s;
  const float *B, *P, *R_enc;
  void *K, *Z, *S;
  float* summ;
  const int32_t* page_table;
  const void *k, *v;
  // append mode: pos != nullptr, one token per row b at pos[b]
  const int32_t* pos;
  // chunk mode: row `seq`, tokens [start, start+n_tok)
  int seq, start, n_tok;
};

// Page scores (and the fused decode-step append): score_kernel.hpp.
struct ScoreArgs {
  Shape s;
  const float *B, *P, *R_enc, *R_dec;
  void *K, *Z, *S;            // written only by the fused append
  float* summ;
  const int32_t *page_table, *seq_lens;
  const void* q;
  const int32_t* pos;         // fused append of one token per row at pos[b]; nullptr: scores only
  const void *k_new, *v_new;
  float* scores;              // [batch][units][max_pages], units: n_kv_heads (or n_q_heads with s.head_select)
  int group_mean;             // a page's score over the group's query heads: 0 max, 1 mean
  int cluster;                // workgroups per (sequence, KV head): [appender] + scorers
  int per;                    // pages per scoring workgroup (<= 256)
};

// Workgroups per (sequence, KV head) and pages per scoring workgroup.
void score_plan(const Shape& s, bool append, int* cluster, int* per);
bool score_fits(const Shape& s, bool append);  // the appending workgroup's LDS fits one CU

// Top-k selection over the scores: select.hip (and the attention prologue).
struct SelectArgs {
  Shape s;
  const float* scores;
  const int32_t *page_table, *seq_lens;
  int32_t *sel, *n_sel;
  int32_t* sel_phys;          // optional: page_table entries of sel
  int sink_pages, local_pages;  // pages always kept at either end of a sequence (0, 0: plain top-k)
};

struct AttendArgs {
  Shape s;
  const void *K, *Z;
  const int32_t *page_table, *seq_lens;
  const void* q;
  const int32_t *sel, *n_sel;
  const int32_t* sel_phys;  // physical ids of sel (nullptr: looked up in page_table)
  // selection in the prologue (scores != nullptr): every workgroup selects
  // its pair's pages from the scores; split 0 writes sel / n_sel (outputs)
  const float* scores;
  int32_t *sel_out, *n_sel_out;
  int sink_pages, local_pages;
  float* part_acc;          // [pairs][n_wsplit][group][rank_v]  split partial sums
  float* part_ml;           // [pairs][n_wsplit][group][2]       split (max, denominator)
  float* z_out;             // [batch][n_q_heads][rank_v], written directly when n_wsplit == 1
  int n_wsplit, pages_per_wave, waves;
  float scale_log2;         // softmax scale * log2(e)
};

// Combining the split partials of AttendArgs into the normalised latent.
struct MergeArgs {
  Shape s;
  const float *part_acc, *part_ml;
  int n_wsplit;
  float* z_out;             // [batch][n_q_heads][rank_v]
};

// The split merge of AttendArgs' partials fused with the projection (decode).
struct MergeProjectArgs {
  Shape s;
  const float *part_acc, *part_ml;
  int n_wsplit;
  const void* W;            // W_ofT [n][kdim] bf16
  float* out;               // [rows][n]
  float* z_out;             // optional [rows][kdim]: the merged latents
  int rows, kdim, n;
};

struct ProjectArgs {
  const float* z;           // [rows][kdim] fp32
  const void* W;            // [n][kdim] dtype
  float* out;               // [rows][n]
  int rows, kdim, n, dtype;
};

struct PrefillArgs {
  Shape s;
  const void *K, *Z;
  const int32_t* page_table;
  const void* q;            // [n_tok][n_q_heads][head_dim]
  float* z_out;             // [n_tok][n_q_heads][rank_v]
  int seq, start, n_tok;
  float scale_log2;
  // the key pages split into ranges of split_pages, n_ksplit of them (1: no
  // split, z written directly); partials [n_tok * n_q_heads][n_ksplit][rank_v]
  // and [..][n_ksplit][2] (max, denominator), merged into z_out afterwards
  int n_ksplit, split_pages;
  float *part_acc, *part_ml;
};
constexpr int PREFILL_KSPLIT_MAX = 8;
// Key-range splits of a prefill chunk: about 16 pages each (or
// BASISKV_PREFILL_SPLIT_PAGES), at most PREFILL_KSPLIT_MAX; 1 where the
// matrix-core kernel does not run.
void plan_prefill(const Shape& s, int start, int n_tok, int* n_ksplit, int* split_pages);

// Raise a kernel's dynamic-LDS limit when a launch needs more than the
// default allows alongside its static arrays (gfx950 has 160 KiB per CU).
inline hipError_t allow_lds(const void* kernel, size_t dynamic_bytes) {
  if (dynamic_bytes <= 32 * 1024) return hipSuccess;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)dynamic_bytes);
}

// Host-side planning shared by workspace sizing and launches.
struct AttendPlan {
  int pages_per_wave, n_wsplit, waves;
};
AttendPlan plan_attend(const Shape& s);
size_t attend_lds_bytes(const Shape& s, bool select);  // dynamic LDS of the attention kernel

bool attend_mfma_supported(const Shape& s);
bool project_mfma_supported(int kdim, int n, int dtype);
bool prefill_mfma_supported(const Shape& s);

hipError_t launch_fold(const Shape& s, const float* B, const void* W_O, void* W_ofT, hipStream_t st);
hipError_t launch_write(const WriteArgs& a, hipStream_t st);
hipError_t launch_score(const ScoreArgs& a, hipStream_t st);
hipError_t launch_score_f32(const ScoreArgs& a, hipStream_t st);   // by storage dtype
hipError_t launch_score_bf16(const ScoreArgs& a, hipStream_t st);
hipError_t launch_select(const SelectArgs& a, hipStream_t st);
hipError_t launch_attend(const AttendArgs& a, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, hipStream_t st);
bool merge_project_supported(const Shape& s);
hipError_t launch_merge_project(const MergeProjectArgs& a, hipStream_t st);
bool merge_project_rows_supported(const Shape& s);  // beyond 16 rows: 16-row tiles
hipError_t launch_merge_project_rows(const MergeProjectArgs& a, hipStream_t st);
hipError_t launch_project(const ProjectArgs& a, hipStream_t st);
hipError_t launch_prefill_attend(const PrefillArgs& a, hipStream_t st);
hipError_t launch_zero_u32(unsigned* p, size_t n, hipStream_t st);

// Debug-mode check of the device data a call reads (see validate.hip).
enum : unsigned {
  VALIDATE_SEQ_LEN = 1,      // a sequence length outside [0, max_pages * page_size]
  VALIDATE_PAGE = 2,         // a page-table entry a call reads outside [0, num_phys_pages)
  VALIDATE_APPEND_PAGE = 4,  // the page-table entry of an append position
  VALIDATE_COUNT = 8,        // a selection count outside [0, top_k]
  VALIDATE_SELECTION = 16,   // a selected page outside the sequence, or its physical id out of range
};
struct ValidateArgs {
  int rows, max_pages, page_size, num_phys, top_k, n_kv_heads;
  const int32_t* page_table;
  const int32_t *seq_lens, *pos, *sel, *n_sel, *sel_phys;  // each nullable
  int chunk_seq, chunk_first, chunk_pages;                 // pages of one row (chunk_pages 0: none)
  unsigned* flag;
};
hipError_t launch_validate(const ValidateArgs& v, hipStream_t st);
hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, int n_sink, hipStream_t st);

}  // namespace bkv
