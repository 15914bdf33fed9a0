/*
 * oracle.h - plain fp64 CPU oracle of BasisKV's per-GPU routed latent decode.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may call this library.  The GPU library never links,
 * loads or calls it, and the two share no source.
 *
 * What it computes, and the passages it follows (weekinpapers "BasisKV: Value
 * Latents for Communication and Key Routing", Abstract; kongchang article on
 * BasisKV, sections on the output-projection binding and on Value-latent Key
 * routing; machinelearning.ru "KV-кэширование", sections "Математическая
 * формализация" and "Фаза Prefill"/"Фаза Decode"):
 *   writer  - a Value is stored only as its latent z = v.B (rounded to the
 *             storage dtype); a Key residual s = (k - z~.P).R_enc is stored
 *             beside it; the exact Key is stored too; each page keeps the
 *             sums of its stored latents and residuals.
 *   route   - per query head, page score = scale * q . mean_t(z~_t.P + s~_t.R_dec)
 *             evaluated from the page sums; the group's score is the max over
 *             its query heads (or their mean); the top-k pages are kept, per
 *             KV head (or, with head_select, per query head).
 *   decode  - exact q.k on the selected pages only, softmax over their valid
 *             tokens, weighted sum of the stored latents, then the projection
 *             through W_of = B^T.W_O (the value basis folded into the output
 *             projection).
 *   prefill - write the chunk, then causal attention over all earlier tokens.
 *
 * Data layout (identical to the GPU library's, written independently):
 *   K pool   [num_pages][H_kv][ps][d_h]        storage dtype
 *   Z pool   [num_pages][H_kv][r][ps]          storage dtype (latent, r-major in a page)
 *   S pool   [num_pages][H_kv][ps][r_k]        storage dtype
 *   summ     [num_pages][H_kv][r + r_k]        fp32 sums of stored z~ then s~
 *   page_table [batch][max_pages]              int32 physical page id
 *   factors: B [H_kv][d_h][r], P [H_kv][r][d_h], R_enc [H_kv][d_h][r_k],
 *            R_dec [H_kv][r_k][d_h] (fp32); W_O [H_q*d_h][d_model] and
 *            W_of^T [d_model][H_q*r] in storage dtype.
 * dtype 0 = fp32, 1 = bf16 (uint16 bit patterns).
 */
#ifndef BASISKV_ORACLE_H
#define BASISKV_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, n_q_heads, n_kv_heads, head_dim, rank_v, rank_k, page_size;
  int32_t d_model, top_k, max_pages, num_pages, dtype;
  double scale;           /* softmax scale, e.g. 1/sqrt(d_h) */
  int32_t sink_pages, local_pages;  /* routing: pages always kept at either end */
  int32_t group_mean;               /* routing: group score = mean over its query heads (else max) */
  int32_t head_select;              /* routing: 1 = every query head selects its own pages */
} ora_dims;

typedef struct {
  void *K, *Z, *S;
  float *summ;
  const int32_t *page_table;
} ora_cache;

/* Round a real value to the nearest bf16, ties to even; returns the bits. */
uint16_t ora_round_bf16(double x);

/* W_of^T[c][h*r + j] = round(sum_i B[g(h)][i][j] * W_O[h*d_h + i][c]). */
void ora_fold(const ora_dims *d, const float *B, const void *W_O, void *W_ofT);

/* Write tokens [start, start+n) of sequence `seq` (k, v: [n][H_kv][d_h]),
 * then set every touched page's sums to the fp64 sum (rounded to fp32) over
 * its slots [0, valid). */
void ora_write(const ora_dims *d, const float *B, const float *P, const float *R_enc,
               const ora_cache *c, int32_t seq, int32_t start, int32_t n,
               const void *k, const void *v);

/* Router.  A selection unit is a (sequence, KV head) pair scored over the
 * KV head's query heads, or with head_select a (sequence, query head) pair
 * scored by that head alone; U = H_kv (or H_q) units per sequence.
 * sel [batch][U][top_k] ascending logical ids, -1 padded; n_sel [batch][U];
 * scores [batch][U][max_pages] fp32 unit scores (-inf beyond the sequence's
 * pages). */
void ora_route(const ora_dims *d, const float *P, const float *R_dec, const ora_cache *c,
               const int32_t *seq_lens, const void *q, int32_t *sel, int32_t *n_sel,
               float *scores);

/* Decode over a given selection (per unit, as the router lists it): every
 * query head of a unit attends over the unit's pages.  z_out [batch][H_q][r],
 * out [batch][d_model]. */
void ora_decode(const ora_dims *d, const void *W_ofT, const ora_cache *c,
                const int32_t *seq_lens, const void *q, const int32_t *sel,
                const int32_t *n_sel, double *z_out, double *out);

/* Causal attention of sequence `seq` for the query positions pos[0..n):
 * every token t <= pos[i] of every page is attended.  q: [n][H_q][d_h];
 * z_out [n][H_q][r], out [n][d_model]. */
void ora_attend_causal(const ora_dims *d, const void *W_ofT, const ora_cache *c,
                       int32_t seq, const int32_t *pos, int32_t n, const void *q,
                       double *z_out, double *out);

#ifdef __cplusplus
}
#endif
#endif
