/*
 * oracle.c - plain fp64 CPU oracle of BasisKV's per-GPU routed latent decode.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline timing).  Slow on
 * purpose: straight loops in the order the method states its steps, fp64
 * arithmetic, rounding only where a value is stored.  See oracle.h for the
 * data layout and the passages each function follows.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ---- storage dtype helpers ------------------------------------------------ */

uint16_t ora_round_bf16(double x) {
  /* bf16: 1 sign, 8 exponent, 7 fraction bits.  A normal value carries 8
   * significant bits, so its quantum is 2^(e-8) where x = m*2^e, m in [0.5,1);
   * below 2^-126 the quantum is fixed at 2^-133.  nearbyint rounds to nearest,
   * ties to even, in the default floating-point environment. */
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7F80;
  int e;
  frexp(a, &e);
  int qexp = (e - 1 >= -126) ? e - 8 : -133;
  double r = ldexp(nearbyint(ldexp(a, -qexp)), qexp);
  const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
  if (r > max_finite) return sign | 0x7F80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

static double ld(const void *base, size_t i, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[i];
  uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round x to the storage dtype and return the stored value as a real. */
static double st(void *base, size_t i, int dtype, double x) {
  if (dtype == 0) {
    float f = (float)x;
    ((float *)base)[i] = f;
    return (double)f;
  }
  uint16_t h = ora_round_bf16(x);
  ((uint16_t *)base)[i] = h;
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static void copy_elem(void *dst, size_t di, const void *src, size_t si, int dtype) {
  if (dtype == 0) ((float *)dst)[di] = ((const float *)src)[si];
  else ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
}

/* ---- index helpers ---------------------------------------------------------- */

static size_t k_idx(const ora_dims *d, int phys, int g, int t, int i) {
  return (((size_t)phys * d->n_kv_heads + g) * d->page_size + t) * d->head_dim + i;
}
static size_t z_idx(const ora_dims *d, int phys, int g, int j, int t) {
  return (((size_t)phys * d->n_kv_heads + g) * d->rank_v + j) * d->page_size + t;
}
static size_t s_idx(const ora_dims *d, int phys, int g, int t, int j) {
  return (((size_t)phys * d->n_kv_heads + g) * d->page_size + t) * d->rank_k + j;
}
static size_t summ_idx(const ora_dims *d, int phys, int g, int j) {
  return ((size_t)phys * d->n_kv_heads + g) * (d->rank_v + d->rank_k) + j;
}
static int phys_of(const ora_dims *d, const ora_cache *c, int seq, int page) {
  return c->page_table[(size_t)seq * d->max_pages + page];
}

/* ---- output projection with the value basis folded in -------------------- */

void ora_fold(const ora_dims *d, const float *B, const void *W_O, void *W_ofT) {
  const int D = d->head_dim, R = d->rank_v, G = d->n_q_heads / d->n_kv_heads;
  const int KW = d->n_q_heads * R;
#pragma omp parallel for schedule(static)
  for (int col = 0; col < d->d_model; ++col)
    for (int h = 0; h < d->n_q_heads; ++h) {
      int g = h / G;
      for (int j = 0; j < R; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i)
          acc += (double)B[((size_t)g * D + i) * R + j] *
                 ld(W_O, ((size_t)h * D + i) * d->d_model + col, d->dtype);
        st(W_ofT, (size_t)col * KW + (size_t)h * R + j, d->dtype, acc);
      }
    }
}

/* ---- writer ------------------------------------------------------------------ */

static void write_token(const ora_dims *d, const float *B, const float *P, const float *R_enc,
                        const ora_cache *c, int seq, int pos, int g, const void *k,
                        const void *v, size_t row) {
  const int D = d->head_dim, R = d->rank_v, RK = d->rank_k, ps = d->page_size;
  int phys = phys_of(d, c, seq, pos / ps), slot = pos % ps;
  double *z = malloc(sizeof(double) * (size_t)(R + D + RK));
  double *e = z + R, *s = e + D;
  /* latent of the Value: z = v . B, stored rounded */
  for (int j = 0; j < R; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i)
      acc += ld(v, row * D + i, d->dtype) * (double)B[((size_t)g * D + i) * R + j];
    z[j] = st(c->Z, z_idx(d, phys, g, j, slot), d->dtype, acc);
  }
  /* what the stored latent predicts of the Key, and the Key's remainder */
  for (int i = 0; i < D; ++i) {
    double khat = 0.0;
    for (int j = 0; j < R; ++j) khat += z[j] * (double)P[((size_t)g * R + j) * D + i];
    e[i] = ld(k, row * D + i, d->dtype) - khat;
  }
  /* the Key-specific residual, stored rounded */
  for (int j = 0; j < RK; ++j) {
    double acc = 0.0;
    for (int i = 0; i < D; ++i) acc += e[i] * (double)R_enc[((size_t)g * D + i) * RK + j];
    s[j] = st(c->S, s_idx(d, phys, g, slot, j), d->dtype, acc);
  }
  /* the exact Key */
  for (int i = 0; i < D; ++i) copy_elem(c->K, k_idx(d, phys, g, slot, i), k, row * D + i, d->dtype);
  free(z);
}

static void page_sums(const ora_dims *d, const ora_cache *c, int phys, int g, int valid) {
  const int R = d->rank_v, RK = d->rank_k;
  for (int j = 0; j < R; ++j) {
    double acc = 0.0;
    for (int t = 0; t < valid; ++t) acc += ld(c->Z, z_idx(d, phys, g, j, t), d->dtype);
    c->summ[summ_idx(d, phys, g, j)] = (float)acc;
  }
  for (int j = 0; j < RK; ++j) {
    double acc = 0.0;
    for (int t = 0; t < valid; ++t) acc += ld(c->S, s_idx(d, phys, g, t, j), d->dtype);
    c->summ[summ_idx(d, phys, g, R + j)] = (float)acc;
  }
}

void ora_write(const ora_dims *d, const float *B, const float *P, const float *R_enc,
               const ora_cache *c, int32_t seq, int32_t start, int32_t n, const void *k,
               const void *v) {
  if (n <= 0) return;
  const int H = d->n_kv_heads, ps = d->page_size;
#pragma omp parallel for schedule(static)
  for (long it = 0; it < (long)n * H; ++it) {
    int t = (int)(it / H), g = (int)(it % H);
    write_token(d, B, P, R_enc, c, seq, start + t, g, k, v, (size_t)t * H + g);
  }
  int end = start + n;
  int p0 = start / ps, p1 = (end - 1) / ps;
#pragma omp parallel for schedule(static)
  for (long it = 0; it < (long)(p1 - p0 + 1) * H; ++it) {
    int page = p0 + (int)(it / H), g = (int)(it % H);
    int valid = end - page * ps;
    if (valid > ps) valid = ps;
    page_sums(d, c, phys_of(d, c, seq, page), g, valid);
  }
}

/* ---- router -------------------------------------------------------------- */

typedef struct {
  float score;
  int page;
  int forced; /* kept whatever its score: one of the first sink_pages or last local_pages */
} ranked;

/* forced pages first, then the higher score; ties to the smaller page */
static int by_score_then_page(const void *a, const void *b) {
  const ranked *x = a, *y = b;
  if (x->forced != y->forced) return x->forced ? -1 : 1;
  if (!x->forced) {
    if (x->score > y->score) return -1;
    if (x->score < y->score) return 1;
  }
  return (x->page > y->page) - (x->page < y->page);
}

static int ascending_int(const void *a, const void *b) {
  int x = *(const int *)a, y = *(const int *)b;
  return (x > y) - (x < y);
}

void ora_route(const ora_dims *d, const float *P, const float *R_dec, const ora_cache *c,
               const int32_t *seq_lens, const void *q, int32_t *sel, int32_t *n_sel,
               float *scores) {
  const int D = d->head_dim, R = d->rank_v, RK = d->rank_k, ps = d->page_size;
  const int H = d->n_kv_heads, G = d->n_q_heads / H;
  /* selection units per sequence, and the query heads scored in a unit */
  const int U = d->head_select ? d->n_q_heads : H, GU = d->head_select ? 1 : G;
#pragma omp parallel for schedule(dynamic)
  for (long unit = 0; unit < (long)d->batch * U; ++unit) {
    int b = (int)(unit / U), u = (int)(unit % U);
    int g = d->head_select ? u / G : u;      /* the unit's KV head */
    int h0 = d->head_select ? u : g * G;     /* its first query head */
    int n = seq_lens[b];
    int npg = (n + ps - 1) / ps;
    int keff = d->top_k < npg ? d->top_k : npg;
    double *qz = malloc(sizeof(double) * (size_t)GU * (R + RK));
    ranked *rk = malloc(sizeof(ranked) * (size_t)(npg > 0 ? npg : 1));
    /* the query seen through the latent predictor and through the residual decoder */
    for (int hh = 0; hh < GU; ++hh) {
      int h = h0 + hh;
      for (int j = 0; j < R; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i)
          acc += (double)P[((size_t)g * R + j) * D + i] * ld(q, ((size_t)b * d->n_q_heads + h) * D + i, d->dtype);
        qz[(size_t)hh * (R + RK) + j] = acc;
      }
      for (int j = 0; j < RK; ++j) {
        double acc = 0.0;
        for (int i = 0; i < D; ++i)
          acc += (double)R_dec[((size_t)g * RK + j) * D + i] * ld(q, ((size_t)b * d->n_q_heads + h) * D + i, d->dtype);
        qz[(size_t)hh * (R + RK) + R + j] = acc;
      }
    }
    float *srow = scores ? scores + unit * d->max_pages : NULL;
    for (int j = 0; j < npg; ++j) {
      int phys = phys_of(d, c, b, j);
      int cnt = n - j * ps < ps ? n - j * ps : ps;
      double best = -INFINITY, sum = 0.0;
      for (int hh = 0; hh < GU; ++hh) {
        double dot = 0.0;
        for (int x = 0; x < R + RK; ++x)
          dot += qz[(size_t)hh * (R + RK) + x] * (double)c->summ[summ_idx(d, phys, g, x)];
        double sc = d->scale * dot / cnt;
        if (sc > best) best = sc;
        sum += sc;
      }
      if (d->group_mean) best = sum / GU; /* the group's mean instead of its max */
      rk[j].score = (float)best;
      if (rk[j].score == 0.0f) rk[j].score = 0.0f; /* one zero */
      rk[j].page = j;
      rk[j].forced = j < d->sink_pages || j >= npg - d->local_pages;
      if (srow) srow[j] = rk[j].score;
    }
    if (srow)
      for (int j = npg; j < d->max_pages; ++j) srow[j] = -INFINITY;
    qsort(rk, (size_t)npg, sizeof(ranked), by_score_then_page);
    int32_t *out = sel + unit * d->top_k;
    for (int i = 0; i < keff; ++i) out[i] = rk[i].page;
    qsort(out, (size_t)keff, sizeof(int32_t), ascending_int);
    for (int i = keff; i < d->top_k; ++i) out[i] = -1;
    n_sel[unit] = keff;
    free(qz);
    free(rk);
  }
}

/* ---- attention over a set of cached tokens ----------------------------------- */

/* Softmax attention of one query head over the tokens listed in (phys[], cnt[])
 * pages; writes the normalised latent average zhat[R]. */
static void attend_pages(const ora_dims *d, const ora_cache *c, int g, const void *q,
                         size_t qrow, const int *phys, const int *cnt, int np,
                         double *zhat) {
  const int D = d->head_dim, R = d->rank_v;
  int ntok = 0;
  for (int p = 0; p < np; ++p) ntok += cnt[p];
  for (int j = 0; j < R; ++j) zhat[j] = 0.0;
  if (ntok == 0) return;
  double *s = malloc(sizeof(double) * (size_t)ntok);
  int x = 0;
  double m = -INFINITY;
  for (int p = 0; p < np; ++p)
    for (int t = 0; t < cnt[p]; ++t) {
      double acc = 0.0;
      for (int i = 0; i < D; ++i)
        acc += ld(q, qrow * D + i, d->dtype) * ld(c->K, k_idx(d, phys[p], g, t, i), d->dtype);
      s[x] = d->scale * acc;
      if (s[x] > m) m = s[x];
      ++x;
    }
  double l = 0.0;
  for (x = 0; x < ntok; ++x) {
    s[x] = exp(s[x] - m);
    l += s[x];
  }
  x = 0;
  for (int p = 0; p < np; ++p)
    for (int t = 0; t < cnt[p]; ++t, ++x)
      for (int j = 0; j < R; ++j) zhat[j] += s[x] / l * ld(c->Z, z_idx(d, phys[p], g, j, t), d->dtype);
  free(s);
}

static void project(const ora_dims *d, const void *W_ofT, const double *zrow, double *out) {
  const int KW = d->n_q_heads * d->rank_v;
  for (int col = 0; col < d->d_model; ++col) {
    double acc = 0.0;
    for (int x = 0; x < KW; ++x) acc += zrow[x] * ld(W_ofT, (size_t)col * KW + x, d->dtype);
    out[col] = acc;
  }
}

void ora_decode(const ora_dims *d, const void *W_ofT, const ora_cache *c,
                const int32_t *seq_lens, const void *q, const int32_t *sel,
                const int32_t *n_sel, double *z_out, double *out) {
  const int R = d->rank_v, ps = d->page_size;
  const int H = d->n_kv_heads, G = d->n_q_heads / H;
  const int U = d->head_select ? d->n_q_heads : H, GU = d->head_select ? 1 : G;
#pragma omp parallel for schedule(dynamic)
  for (long unit = 0; unit < (long)d->batch * U; ++unit) {
    int b = (int)(unit / U), u = (int)(unit % U);
    int g = d->head_select ? u / G : u;
    int h0 = d->head_select ? u : g * G;
    int n = seq_lens[b];
    int ns = n > 0 ? n_sel[unit] : 0;
    int *phys = malloc(sizeof(int) * (size_t)(ns > 0 ? 2 * ns : 1));
    int *cnt = phys + ns;
    for (int i = 0; i < ns; ++i) {
      int j = sel[unit * d->top_k + i];
      phys[i] = phys_of(d, c, b, j);
      cnt[i] = n - j * ps < ps ? n - j * ps : ps;
    }
    for (int hh = 0; hh < GU; ++hh) {
      int h = h0 + hh;
      attend_pages(d, c, g, q, (size_t)b * d->n_q_heads + h, phys, cnt, ns,
                   z_out + ((size_t)b * d->n_q_heads + h) * R);
    }
    free(phys);
  }
#pragma omp parallel for schedule(static)
  for (int b = 0; b < d->batch; ++b)
    project(d, W_ofT, z_out + (size_t)b * d->n_q_heads * R, out + (size_t)b * d->d_model);
}

void ora_attend_causal(const ora_dims *d, const void *W_ofT, const ora_cache *c,
                       int32_t seq, const int32_t *pos, int32_t n, const void *q,
                       double *z_out, double *out) {
  const int R = d->rank_v, ps = d->page_size;
  const int H = d->n_kv_heads, G = d->n_q_heads / H;
#pragma omp parallel for schedule(dynamic)
  for (long it = 0; it < (long)n * d->n_q_heads; ++it) {
    int row = (int)(it / d->n_q_heads), h = (int)(it % d->n_q_heads);
    int p = pos[row], len = p + 1;
    int np = (len + ps - 1) / ps;
    int *phys = malloc(sizeof(int) * (size_t)2 * np);
    int *cnt = phys + np;
    for (int j = 0; j < np; ++j) {
      phys[j] = phys_of(d, c, seq, j);
      cnt[j] = len - j * ps < ps ? len - j * ps : ps;
    }
    attend_pages(d, c, h / G, q, (size_t)row * d->n_q_heads + h, phys, cnt, np,
                 z_out + ((size_t)row * d->n_q_heads + h) * R);
    free(phys);
  }
#pragma omp parallel for schedule(static)
  for (int row = 0; row < n; ++row)
    project(d, W_ofT, z_out + (size_t)row * d->n_q_heads * R, out + (size_t)row * d->d_model);
}
