/*
 * basiskv.h - C ABI of the routed latent decode library for MI355X (gfx950).
 *
 * The method (weekinpapers "BasisKV: Value Latents for Communication and Key
 * Routing", Abstract; kongchang article on BasisKV, sections on binding the
 * Value compression to the output projection and on Value-latent Key
 * routing) keeps each cached Value only as a rank-r latent z = v.B, folds the
 * value basis into this GPU's slice of the output projection, predicts page
 * scores for Key routing from the latents plus a Key-specific low-rank
 * residual, and reads the exact Keys back only for the top-k pages to score
 * q.k exactly.  Decode appends the new token before attending
 * (machinelearning.ru "KV-кэширование", "Фаза Decode"); prefill writes a
 * chunk of prompt tokens and attends causally ("Фаза Prefill"); attention is
 * softmax(q.k / sqrt(d_h)) weighted ("Математическая формализация").  The
 * cache is paged ("Форматы" on the same page) and several query heads share
 * one KV head (Baidu article "KV cache compression architectures", GQA).
 *
 * Everything here is one GPU's tensor-parallel share: its query heads, their
 * KV heads and its rows of the output projection.  No collective is issued.
 *
 * ---------------------------------------------------------------------------
 * Conventions
 *   - All pointers are DEVICE pointers unless marked (host).  The structs
 *     themselves are host memory, read during the call only.
 *   - The caller owns every buffer.  The library never allocates or frees
 *     device memory and keeps no state between calls.
 *   - Every call validates its arguments on the host, then only enqueues
 *     kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns.  Ordering between calls is the stream's order.  An error
 *     return means nothing was enqueued (except BASISKV_E_HIP, where a launch
 *     failed and earlier kernels of the same call may have been enqueued).
 *   - Contents of device data (page ids, lengths, positions) are not checked;
 *     out-of-range values are undefined behaviour.
 *   - Calls are thread-safe; the only global is the thread-local error text.
 *
 * Data layout (row-major, contiguous; dtype = storage dtype, fp32 or bf16):
 *   K pool      [num_phys_pages][n_kv_heads][page_size][head_dim]   dtype  exact Keys
 *   Z pool      [num_phys_pages][n_kv_heads][rank_v][page_size]     dtype  Value latents,
 *               channel-major inside a page (a page's latent channel is contiguous)
 *   S pool      [num_phys_pages][n_kv_heads][page_size][rank_k]     dtype  Key residuals
 *   summ        [num_phys_pages][n_kv_heads][rank_v + rank_k]       fp32   per-page sums of
 *               the stored latents (first rank_v) and residuals (last rank_k)
 *   page_table  [batch][max_pages_per_seq]  int32  physical page of logical page j
 *   seq_lens    [batch]                     int32  tokens in the cache per sequence
 *   q           [rows][n_q_heads][head_dim] dtype
 *   factors     B [n_kv_heads][head_dim][rank_v], P [n_kv_heads][rank_v][head_dim],
 *               R_enc [n_kv_heads][head_dim][rank_k], R_dec [n_kv_heads][rank_k][head_dim]
 *               fp32; W_ofT [d_model][n_q_heads*rank_v] dtype (the folded output
 *               projection, stored transposed like a linear layer's weight)
 *   Query head h belongs to KV head h / (n_q_heads / n_kv_heads).
 *
 * Page sums, scores and selection (per sequence b and KV head g, n = seq_lens[b],
 * n_pg = ceil(n / page_size), cnt_j = min(page_size, n - j*page_size)):
 *   score_h(j) = scale * (P.q_h . sumz_j + R_dec.q_h . sums_j) / cnt_j
 *   score(j)   = max over the query heads h of KV head g (their mean with group_mean)
 *   the min(top_k, n_pg) highest scores are selected, ties to the smaller j;
 *   sel lists them in ascending j, padded with -1.
 *   Forced pages (sink_pages, local_pages >= 0, both 0 for plain top-k): pages
 *   j < sink_pages and j >= n_pg - local_pages rank above every score (among
 *   themselves the smaller j first), so they are kept whenever they fit in
 *   top_k; scores are reported unchanged.
 * Selection units: by default a unit is a (sequence b, KV head g) pair and
 * its score is score(j) above; with head_select = 1 every query head h is a
 * unit of its own, scored by score_h(j) alone (group_mean has no effect),
 * and attends over its own pages of KV head h / group (the pages leave the
 * GQA granularity of routing open: kongchang article, Value-latent Key
 * routing).  U = n_kv_heads (or n_q_heads) units per sequence; the router's
 * scores, sel, n_sel and sel_phys below are [batch][U][...], and "pair"
 * below means a unit.
 * ---------------------------------------------------------------------------
 */
#ifndef BASISKV_H
#define BASISKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BASISKV_VERSION 4

enum {
  BASISKV_OK = 0,
  BASISKV_E_NULL = -1,        /* a required pointer is NULL                           */
  BASISKV_E_DIMS = -2,        /* inconsistent or non-positive dimensions              */
  BASISKV_E_UNSUPPORTED = -3, /* valid, but no kernel for this shape                  */
  BASISKV_E_WORKSPACE = -4,   /* workspace too small                                  */
  BASISKV_E_HIP = -5,         /* a HIP call or launch failed (see basiskv_last_error) */
  BASISKV_E_DATA = -6         /* invalid device data (debug mode only, see below)    */
};

/*
 * Debug mode: with the environment variable BASISKV_DEBUG=1, every call that
 * reads sequence lengths, page-table entries, append positions or a
 * selection first checks, on the device, the values it is about to use
 * (lengths within [0, max_pages_per_seq * page_size]; the page-table entry
 * of every page a length, an append position or a chunk reaches within
 * [0, num_phys_pages); selection counts within [0, top_k], selected pages
 * below the sequence's page count and their physical ids within the pool),
 * synchronises the stream, and returns BASISKV_E_DATA with nothing else
 * enqueued when one is violated (basiskv_last_error says which).  Without
 * it these values are not checked and a violation is undefined behaviour.
 * Debug mode synchronises, so it does not suit graph capture.  The checks of
 * calls made from several host threads run one at a time: the library holds
 * one check flag per device.
 */

enum { BASISKV_F32 = 0, BASISKV_BF16 = 1 };

/* Shapes of one GPU's share.  Host struct. */
typedef struct {
  int32_t batch;              /* rows of page_table (sequences)                       */
  int32_t n_q_heads;          /* query heads on this GPU                              */
  int32_t n_kv_heads;         /* KV heads on this GPU; n_q_heads % n_kv_heads == 0    */
  int32_t head_dim;           /* d_h: 64 or 128                                       */
  int32_t rank_v;             /* r: latent width, multiple of 16, <= 64, <= head_dim  */
  int32_t rank_k;             /* r_k: residual width, multiple of 4, <= 64            */
  int32_t page_size;          /* tokens per page: 16, 32 or 64                        */
  int32_t d_model;            /* output width of this GPU's projection slice          */
  int32_t top_k;              /* pages selected per selection unit (see above)       */
  int32_t max_pages_per_seq;  /* columns of page_table, <= 8192                       */
  int32_t num_phys_pages;     /* pages in each pool                                   */
  int32_t dtype;              /* BASISKV_F32 or BASISKV_BF16                          */
  float softmax_scale;        /* 0 -> 1/sqrt(head_dim)                                */
  int32_t sink_pages;         /* routing: the first sink_pages pages are always kept  */
  int32_t local_pages;        /* routing: the last local_pages pages are always kept  */
  int32_t group_mean;         /* routing: 0 = a page's score is the max over the KV
                                 head's query heads, 1 = their mean                  */
  int32_t head_select;        /* routing: 0 = one selection per (sequence, KV head);
                                 1 = one per (sequence, query head), see above       */
} basiskv_dims;

/* Factors.  Host struct of device pointers; read only. */
typedef struct {
  const float *B, *P, *R_enc, *R_dec;
  const void *W_ofT;          /* [d_model][n_q_heads*rank_v] dtype                    */
} basiskv_factors;

/* Paged cache.  Host struct of device pointers. */
typedef struct {
  void *K, *Z, *S;
  float *summ;
  const int32_t *page_table;
} basiskv_cache;

/* Library version (BASISKV_VERSION).  Host. */
int basiskv_version(void);

/* Static text for an error code.  Host. */
const char *basiskv_strerror(int code);

/* Detail of the last error on the calling thread ("" if none).  Host. */
const char *basiskv_last_error(void);

/*
 * Fold the value basis into the output projection (Abstract, observation (ii);
 * kongchang article, output-projection binding):
 *   W_ofT[c][h*rank_v + j] = round_dtype( sum_i B[g(h)][i][j] * W_O[h*head_dim + i][c] )
 * W_O [n_q_heads*head_dim][d_model] dtype; W_ofT as in the layout above.
 * Setup-time call; fp32 accumulation, round-to-nearest-even.
 */
int basiskv_fold_output(const basiskv_dims *dims, const float *B, const void *W_O,
                        void *W_ofT, void *stream);

/*
 * Cache writer for a run of tokens of one sequence (prefill chunks, or any
 * batch of appends to one row).  For each token position p in
 * [start, start+n_tok) and KV head g, with k = k[p-start][g], v = v[p-start][g]:
 *   z~ = round(v.B[g]);  s~ = round((k - z~.P[g]).R_enc[g]);
 * k, z~ and s~ go to slot p % page_size of page page_table[seq][p / page_size].
 * Then each touched page's sums are set to the fp32 sums of its stored
 * latents and residuals over slots [0, last written slot] (fp32 storage: in
 * slot order; bf16: the slots before the last on the matrix cores, then the
 * last slot added, the same way for appends and chunks).
 * The caller maps the pages first.  k, v: [n_tok][n_kv_heads][head_dim] dtype.
 */
int basiskv_write(const basiskv_dims *dims, const basiskv_factors *f,
                  const basiskv_cache *cache, int32_t seq, int32_t start, int32_t n_tok,
                  const void *k, const void *v, void *stream);

/*
 * Decode-step append: the writer above for one token per sequence, at
 * position pos[b] of row b (pos is a device array [batch]; pos[b] < 0 skips
 * row b).  k_new, v_new: [batch][n_kv_heads][head_dim] dtype.  The caller
 * maps page pos[b] / page_size and afterwards sets seq_lens[b] = pos[b] + 1.
 * Writing a position again rewrites its slot and the page sums identically.
 */
int basiskv_append(const basiskv_dims *dims, const basiskv_factors *f,
                   const basiskv_cache *cache, const int32_t *pos, const void *k_new,
                   const void *v_new, void *stream);

/*
 * Router (Abstract: the Value latents predict the Key information needed for
 * routing, a Key residual stores the rest; kongchang article, coarse routing
 * then exact scoring).  Reads P, R_dec, summ, page_table, seq_lens and
 * q [batch][n_q_heads][head_dim]; writes
 *   scores [batch][U][max_pages_per_seq] fp32 (required): the unit's score(j)
 *          for j < n_pg; entries j >= n_pg are left unspecified;
 *   sel    [batch][U][top_k] int32 ascending logical pages, -1 padded;
 *   n_sel  [batch][U] int32 = min(top_k, n_pg);
 *   sel_phys (nullable) [batch][U][top_k] int32: page_table entries of
 *          sel (-1 padded), which basiskv_attend/decode may take to skip the
 *          page-table lookup.
 * sel and n_sel are both given or both NULL; NULL asks for the scores alone
 * (sel_phys must then be NULL too).
 * Two launches: the scores (a cluster of workgroups per (sequence, KV head),
 * each scoring a few dozen pages), then the selection (a workgroup per
 * unit), which the scores-only form leaves out.  Needs no
 * workspace.
 */
int basiskv_route(const basiskv_dims *dims, const basiskv_factors *f,
                  const basiskv_cache *cache, const int32_t *seq_lens, const void *q,
                  int32_t *sel, int32_t *n_sel, float *scores, int32_t *sel_phys, void *stream);

/*
 * basiskv_append followed by basiskv_route: the append is fused into the
 * scoring launch (the decode step appends its token before attending).
 * Arguments as in the two calls; the factors B, P, R_enc and R_dec are all
 * required.
 */
int basiskv_append_route(const basiskv_dims *dims, const basiskv_factors *f,
                         const basiskv_cache *cache, const int32_t *pos, const void *k_new,
                         const void *v_new, const int32_t *seq_lens, const void *q,
                         int32_t *sel, int32_t *n_sel, float *scores, int32_t *sel_phys,
                         void *stream);

/*
 * Device workspace, in bytes, that basiskv_attend/decode/decode_step (batch
 * rows) and basiskv_prefill (up to max_prefill_tokens queries) need.  Host
 * function.  It carries the attention splits' partial results and
 * intermediate latents between the launches of one call; nothing in it
 * carries over between calls and it needs no initialisation.  Calls that
 * share a workspace must not overlap in time.
 */
size_t basiskv_workspace_bytes(const basiskv_dims *dims, int32_t max_prefill_tokens);

/* Zero-fill a workspace with a fill kernel (safe under graph capture); not
 * needed before use. */
int basiskv_workspace_init(const basiskv_dims *dims, void *ws, size_t ws_bytes, void *stream);

/*
 * Routed exact attention over the selected pages (Abstract: original Keys
 * retrieved only for the selected pages to compute exact QK scores).  For
 * query head h of KV head g and sequence b, u its unit (g, or h with
 * head_select):
 *   s_t = scale * q_h . k_t   for every token t < seq_lens[b] of every page
 *                             listed in sel[b][u][0 .. n_sel[b][u])
 *   z_out[b][h] = sum_t softmax(s)_t * z~_t          (fp32 [batch][n_q_heads][rank_v])
 * A sequence with no selected page gets z_out = 0.  sel_phys (nullable): the
 * physical ids of sel as basiskv_route writes them; NULL looks them up.
 * The selection of each unit is processed in splits whose
 * partial results are combined afterwards (flash-decoding style).  z_out may
 * be NULL: the combination is then left to the caller and the partials stay
 * at the start of ws, fp32 [batch*U][n_split][Gu][rank_v] partial
 * sums sum_t 2^(s_t*log2(e) - m) z~_t, followed (at the next 256-byte
 * boundary) by [batch*U][n_split][Gu][2] pairs (m, sum_t
 * 2^(s_t*log2(e) - m)) with m the split's max of s_t*log2(e) (-inf for an
 * empty split); Gu = group (1 with head_select), n_split =
 * basiskv_attend_splits(dims).
 */
int basiskv_attend(const basiskv_dims *dims, const basiskv_cache *cache,
                   const int32_t *seq_lens, const void *q, const int32_t *sel,
                   const int32_t *n_sel, const int32_t *sel_phys, void *ws, size_t ws_bytes,
                   float *z_out, void *stream);

/* Number of splits per selection unit that basiskv_attend plans for
 * these dims (>= 1), or a negative error code.  Host function. */
int basiskv_attend_splits(const basiskv_dims *dims);

/*
 * Output projection through the folded weights: out[m][c] = sum_x z[m][x] * W_ofT[c][x]
 * for m < rows (z fp32 [rows][n_q_heads*rank_v], out fp32 [rows][d_model]).
 * bf16 storage: z is rounded to bf16 and multiplied on the matrix cores with
 * fp32 accumulation.  This GPU's partial of the layer output (no all-reduce).
 */
int basiskv_project(const basiskv_dims *dims, const basiskv_factors *f, const float *z,
                    int32_t rows, float *out, void *stream);

/*
 * One decode layer step after the append: basiskv_attend then basiskv_project
 * over the batch.  z_out and sel_phys may be NULL (the latents then live in
 * the workspace).  out: fp32 [batch][d_model].
 */
int basiskv_decode(const basiskv_dims *dims, const basiskv_factors *f,
                   const basiskv_cache *cache, const int32_t *seq_lens, const void *q,
                   const int32_t *sel, const int32_t *n_sel, const int32_t *sel_phys, void *ws,
                   size_t ws_bytes, float *z_out, float *out, void *stream);

/*
 * The whole decode layer step in three launches: the append fused with the
 * page scores; the attention, whose workgroups each select their pair's
 * top-k pages from the scores before reading the selected pages; the split
 * merge fused with the projection.  sel, n_sel and scores are written as by
 * basiskv_route; z_out may be NULL.
 */
int basiskv_decode_step(const basiskv_dims *dims, const basiskv_factors *f,
                        const basiskv_cache *cache, const int32_t *pos, const void *k_new,
                        const void *v_new, const int32_t *seq_lens, const void *q,
                        int32_t *sel, int32_t *n_sel, float *scores, void *ws, size_t ws_bytes,
                        float *z_out, float *out, void *stream);

/*
 * basiskv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, allocation-free serving
 * loops, harnesses that forbid hipMalloc).  Arguments and results as in
 * basiskv_decode_step.  Its scratch (what basiskv_decode_step keeps in the
 * workspace) is a file-scope device array of BASISKV_NOALLOC_SCRATCH_BYTES
 * bytes that the library holds on each device it runs on until the process
 * ends; dims whose workspace (basiskv_workspace_bytes(dims, 0)) exceeds it are
 * rejected with BASISKV_E_WORKSPACE before anything is enqueued.  The call
 * allocates nothing: it runs basiskv_decode_step's kernels on the array
 * (every byte a call reads there it has written earlier in the same call, so
 * nothing needs clearing).  Every call on a device shares that device's
 * array, which keeps the last call's contents:
 * calls that overlap in time on one device (other streams or threads) race
 * and their results are undefined.
 */
#define BASISKV_NOALLOC_SCRATCH_BYTES (4u << 20)
int basiskv_decode_step_noalloc(const basiskv_dims *dims, const basiskv_factors *f,
                                const basiskv_cache *cache, const int32_t *pos, const void *k_new,
                                const void *v_new, const int32_t *seq_lens, const void *q,
                                int32_t *sel, int32_t *n_sel, float *scores, float *z_out, float *out,
                                void *stream);

/*
 * Prefill chunk of one sequence: basiskv_write of tokens [start_pos,
 * start_pos+n_tok), then causal attention of the chunk's queries over every
 * earlier token of the sequence and themselves (all pages, no routing), then
 * the projection.  q: [n_tok][n_q_heads][head_dim]; k, v: [n_tok][n_kv_heads][head_dim];
 * z_out (nullable) fp32 [n_tok][n_q_heads][rank_v]; out fp32 [n_tok][d_model].
 * n_tok <= the max_prefill_tokens the workspace was sized for.
 */
int basiskv_prefill(const basiskv_dims *dims, const basiskv_factors *f,
                    const basiskv_cache *cache, int32_t seq, int32_t start_pos, int32_t n_tok,
                    const void *q, const void *k, const void *v, void *ws, size_t ws_bytes,
                    float *z_out, float *out, void *stream);

/*
 * Measurement aid beside the method: reads `bytes` bytes of src (16-byte
 * aligned device memory; bytes a multiple of 4) once, with 16-byte loads
 * spread over n_sink >= 1 workgroups of 256 threads, and writes each
 * workgroup's fp32 sum of the words read as floats to sink[0 .. n_sink)
 * (sink: device, caller-owned).  Timing it over a buffer well beyond the
 * 256 MB Infinity Cache gives the achievable HBM read bandwidth that the
 * attention kernel's rate is compared with.  Errors: E_NULL (src or sink
 * NULL), E_DIMS (bytes not a multiple of 4, n_sink < 1, src misaligned).
 */
int basiskv_stream_read(const void *src, size_t bytes, float *sink, int32_t n_sink, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* BASISKV_H */
