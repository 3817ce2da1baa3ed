/*
 * CPU oracle for the DeepSeek Sparse Attention (DSA) decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table
 * or constant with the GPU path and is never called by it.
 *
 * Plain loops in float64, written from the definitions on these pages:
 *  - "MTP and sparse attention: NSA and DSA", DSA bullet: the index score
 *    I(t,s) = sum_j w(t,j) * ReLU(q(t,j) . k(s)) over 64 indexer heads of 128
 *    dims, in FP8 with a 4-byte scale per cached key (the cache accounting
 *    listing: 128 + 4 bytes per token); each query keeps its 2048
 *    highest-scoring tokens and runs absorbed-form MLA over only those
 *    (per-pair cost 2*H*(512+64) + 2*H*512: scores over the 576-wide latent,
 *    values are its first 512 dims).
 *  - "[SGLang] NSA", init_forward_metadata: cached lengths include the new
 *    (draft) rows; in an extend of n rows onto a cache of L tokens, row i sees
 *    L - n + 1 + i tokens (3 rows at L = 10 see 8, 9, 10).
 *  - "[SGLang] NSA", NSAMetadata: page tables map a request's token
 *    positions to physical pages of 64 tokens.
 *  - "MTP and sparse attention: NSA and DSA", new demands on inference
 *    engines, and "[SGLang] NSA", forward_decode: the step's new tokens are
 *    written into the paged latent cache and, FP8-quantised with a per-key
 *    scale, into the indexer-key cache (oracle_cache_append).
 * Ties in the selection go to the lower position.  FP8 values are OCP
 * e4m3fn (the pages say FP8 / E4M3 only; e4m3fn is the reading taken).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---- number formats ---------------------------------------------------- */

/* OCP e4m3fn: sign, 4-bit exponent with bias 7, 3-bit mantissa.  Exponent
 * field 0 holds subnormals m/8 * 2^-6; field 15 with mantissa 7 is NaN;
 * there is no infinity. */
double oracle_e4m3_decode(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* bf16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* ---- batch metadata ------------------------------------------------------ */

typedef struct {
  int32_t B;
  const int32_t* cu_q;       /* [B+1] cumulative query rows */
  const int32_t* seqlens_k;  /* [B]   cached tokens, new rows included */
  const int32_t* page_table; /* [B * max_pages] */
  int32_t max_pages;
  int32_t page_size;
} oracle_batch;

int32_t oracle_row_request(const oracle_batch* bt, int32_t t) {
  for (int32_t b = 0; b < bt->B; ++b)
    if (t >= bt->cu_q[b] && t < bt->cu_q[b + 1]) return b;
  return -1;
}

/* row j of request b sees L_b - n_b + 1 + j tokens */
int64_t oracle_row_visible(const oracle_batch* bt, int32_t t) {
  int32_t b = oracle_row_request(bt, t);
  if (b < 0) return 0;
  int64_t n = bt->cu_q[b + 1] - bt->cu_q[b];
  int64_t j = t - bt->cu_q[b];
  int64_t v = (int64_t)bt->seqlens_k[b] - n + 1 + j;
  return v > 0 ? v : 0;
}

int64_t oracle_slot(const oracle_batch* bt, int32_t b, int64_t s) {
  int64_t page = bt->page_table[(int64_t)b * bt->max_pages + s / bt->page_size];
  return page * bt->page_size + s % bt->page_size;
}

/* A page id outside the pool [0, num_pages) names no cached token: the
 * positions it maps hold no key and no latent row (reading taken here, as
 * the pages' page tables only ever name allocated pages). */
int oracle_page_valid(const oracle_batch* bt, int32_t b, int64_t s, int64_t num_pages) {
  int64_t page = bt->page_table[(int64_t)b * bt->max_pages + s / bt->page_size];
  return page >= 0 && page < num_pages;
}

/* ---- work splitting ------------------------------------------------------ */

typedef void (*item_fn)(void* ctx, int64_t item);
typedef struct {
  item_fn fn;
  void* ctx;
  int64_t n;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void* pool_worker(void* p) {
  pool_t* pl = (pool_t*)p;
  for (;;) {
    pthread_mutex_lock(&pl->mu);
    int64_t i = pl->next++;
    pthread_mutex_unlock(&pl->mu);
    if (i >= pl->n) break;
    pl->fn(pl->ctx, i);
  }
  return NULL;
}

/* Runs fn(ctx, i) for i in [0, n) on `threads` threads.  Items are
 * independent and write disjoint outputs, so results do not depend on the
 * thread count. */
static void run_items(int64_t n, int threads, item_fn fn, void* ctx) {
  if (threads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    threads = c > 0 ? (int)c : 1;
  }
  if (threads > 512) threads = 512;
  if (threads > n) threads = (int)(n > 0 ? n : 1);
  pool_t pl;
  pl.fn = fn;
  pl.ctx = ctx;
  pl.n = n;
  pl.next = 0;
  pthread_mutex_init(&pl.mu, NULL);
  if (threads == 1) {
    pool_worker(&pl);
  } else {
    pthread_t th[512];
    for (int i = 0; i < threads; ++i) pthread_create(&th[i], NULL, pool_worker, &pl);
    for (int i = 0; i < threads; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&pl.mu);
}

/* ---- index score ----------------------------------------------------------
 * I(t,s) = sum_h w(t,h) * max(0, sum_d q(t,h,d) * k(s,d)) with
 * q = q_scale(t) * e4m3(q8), k = k_scale(s) * e4m3(k8); d and h summed in
 * ascending order.  Written for s < v_t; other entries are left as they are.
 * A position on a page outside the pool has no key: it scores -infinity, so
 * it ranks below every real score (and is selected only by a row with fewer
 * than k keyed positions).
 */
#define KEY_CHUNK 4096

typedef struct {
  const oracle_batch* bt;
  int32_t H, D;
  const uint8_t* q8;
  const float* q_scale;
  const float* w;
  const uint8_t* k8;
  const float* k_scale;
  const int32_t* rows;
  int32_t n_rows;
  double* out;
  int64_t ld;
  int64_t chunks_per_row;
  int64_t num_pages;
} score_ctx;

static void score_item(void* p, int64_t item) {
  score_ctx* c = (score_ctx*)p;
  int64_t i = item / c->chunks_per_row;
  int64_t ch = item % c->chunks_per_row;
  int32_t t = c->rows[i];
  int32_t b = oracle_row_request(c->bt, t);
  if (b < 0) return;
  int64_t v = oracle_row_visible(c->bt, t);
  int64_t s0 = ch * KEY_CHUNK, s1 = s0 + KEY_CHUNK < v ? s0 + KEY_CHUNK : v;
  if (s0 >= s1) return;
  int32_t H = c->H, D = c->D;
  double* q = (double*)malloc(sizeof(double) * (size_t)H * (size_t)D);
  double* k = (double*)malloc(sizeof(double) * (size_t)D);
  double qs = (double)c->q_scale[t];
  for (int64_t e = 0; e < (int64_t)H * D; ++e)
    q[e] = qs * oracle_e4m3_decode(c->q8[(int64_t)t * H * D + e]);
  for (int64_t s = s0; s < s1; ++s) {
    if (!oracle_page_valid(c->bt, b, s, c->num_pages)) {
      c->out[i * c->ld + s] = -INFINITY;
      continue;
    }
    int64_t slot = oracle_slot(c->bt, b, s);
    double ks = (double)c->k_scale[slot];
    for (int d = 0; d < D; ++d) k[d] = ks * oracle_e4m3_decode(c->k8[slot * D + d]);
    double I = 0.0;
    for (int h = 0; h < H; ++h) {
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += q[(int64_t)h * D + d] * k[d];
      double relu = dot > 0.0 ? dot : 0.0;
      I += (double)c->w[(int64_t)t * H + h] * relu;
    }
    c->out[i * c->ld + s] = I;
  }
  free(q);
  free(k);
}

void oracle_index_score(const oracle_batch* bt, int64_t num_pages, int32_t H, int32_t D,
                        const uint8_t* q8, const float* q_scale, const float* w,
                        const uint8_t* k8, const float* k_scale, const int32_t* rows,
                        int32_t n_rows, double* out, int64_t ld, int threads) {
  int64_t maxv = 0;
  for (int32_t i = 0; i < n_rows; ++i) {
    int64_t v = oracle_row_visible(bt, rows[i]);
    if (v > maxv) maxv = v;
  }
  score_ctx c = {bt, H, D, q8, q_scale, w, k8, k_scale, rows, n_rows, out, ld,
                 (maxv + KEY_CHUNK - 1) / KEY_CHUNK, num_pages};
  if (c.chunks_per_row == 0) return;
  run_items((int64_t)n_rows * c.chunks_per_row, threads, score_item, &c);
}

/* ---- top-k -----------------------------------------------------------------
 * Order the v visible positions by (score descending, position ascending)
 * and keep the first K = min(k, v).  sel[0..K) holds them in that order and
 * sel[K..k) = -1.  kth = score of the K-th kept position (NaN when K = 0).
 * flags[s] (s < v) = 1 when |I(s) - kth| <= band * |kth|: positions whose
 * membership a float32 score may legitimately flip.
 */
typedef struct {
  double score;
  int64_t pos;
} scored_t;

static int cmp_scored(const void* a, const void* b) {
  const scored_t* x = (const scored_t*)a;
  const scored_t* y = (const scored_t*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return x->pos < y->pos ? -1 : (x->pos > y->pos ? 1 : 0);
}

int32_t oracle_topk(const double* scores, int64_t v, int32_t k, double band, int32_t* sel,
                    uint8_t* flags, double* kth) {
  int64_t K = v < k ? v : k;
  if (K < 0) K = 0;
  scored_t* a = (scored_t*)malloc(sizeof(scored_t) * (size_t)(v > 0 ? v : 1));
  for (int64_t s = 0; s < v; ++s) {
    a[s].score = scores[s] == 0.0 ? 0.0 : scores[s]; /* -0.0 counts as +0.0 */
    a[s].pos = s;
  }
  qsort(a, (size_t)v, sizeof(scored_t), cmp_scored);
  for (int64_t j = 0; j < k; ++j) sel[j] = j < K ? (int32_t)a[j].pos : -1;
  double kv = K > 0 ? a[K - 1].score : NAN;
  if (kth) *kth = kv;
  if (flags) {
    for (int64_t s = 0; s < v; ++s) {
      double x = scores[s] == 0.0 ? 0.0 : scores[s];
      flags[s] = (K > 0 && fabs(x - kv) <= band * fabs(kv)) ? 1 : 0;
    }
  }
  free(a);
  return (int32_t)K;
}

typedef struct {
  const double* scores;
  int64_t ld;
  const int64_t* v;
  int32_t k;
  double band;
  int32_t* sel;
  uint8_t* flags;
  int64_t ldf;
  double* kth;
  int32_t* K;
} topk_ctx;

static void topk_item(void* p, int64_t i) {
  topk_ctx* c = (topk_ctx*)p;
  int32_t K = oracle_topk(c->scores + i * c->ld, c->v[i], c->k, c->band, c->sel + i * c->k,
                          c->flags ? c->flags + i * c->ldf : NULL, c->kth + i);
  if (c->K) c->K[i] = K;
}

void oracle_topk_rows(const double* scores, int64_t ld, const int64_t* v, int32_t n_rows,
                      int32_t k, double band, int32_t* sel, uint8_t* flags, int64_t ldf,
                      double* kth, int32_t* K, int threads) {
  topk_ctx c = {scores, ld, v, k, band, sel, flags, ldf, kth, K};
  run_items(n_rows, threads, topk_item, &c);
}

/* ---- attention ----------------------------------------------------------------
 * Absorbed-form MLA for one (row, head) over a set of positions S:
 *   z(s) = sm_scale * sum_{d < D} q(t,h,d) * kv(s,d)       (D = 576)
 *   p(s) = exp(z(s) - m) / sum_{s'} exp(z(s') - m),  m = max z
 *   o(t,h,d) = sum_s p(s) * kv(s,d)  for d < Dv (Dv = 512)
 *   lse(t,h) = m + ln sum_s exp(z(s) - m)
 * An empty S gives o = 0 and lse = -inf.  Positions on a page outside the
 * pool have no latent row and are left out of S.
 */
typedef struct {
  const oracle_batch* bt;
  int32_t H, D, Dv;
  const uint16_t* q;
  const uint16_t* kv;
  const int32_t* idx; /* [n_rows][k] positions, or NULL for dense */
  int32_t k;
  double sm_scale;
  const int32_t* rows;
  double* out;
  double* lse;
  int64_t num_pages;
} mla_ctx;

static void mla_item(void* p, int64_t item) {
  mla_ctx* c = (mla_ctx*)p;
  int64_t i = item / c->H;
  int32_t h = (int32_t)(item % c->H);
  int32_t t = c->rows[i];
  int32_t b = oracle_row_request(c->bt, t);
  int64_t v = b < 0 ? 0 : oracle_row_visible(c->bt, t);
  int32_t D = c->D, Dv = c->Dv;
  double* o = c->out + (i * c->H + h) * Dv;
  for (int d = 0; d < Dv; ++d) o[d] = 0.0;

  /* the position list S */
  int64_t n = 0;
  int64_t cap = c->idx ? c->k : v;
  int64_t* S = (int64_t*)malloc(sizeof(int64_t) * (size_t)(cap > 0 ? cap : 1));
  if (c->idx) {
    for (int32_t j = 0; j < c->k; ++j) {
      int32_t s = c->idx[i * c->k + j];
      if (s >= 0 && s < v && oracle_page_valid(c->bt, b, s, c->num_pages)) S[n++] = s;
    }
  } else {
    for (int64_t s = 0; s < v; ++s)
      if (oracle_page_valid(c->bt, b, s, c->num_pages)) S[n++] = s;
  }
  if (n == 0) {
    c->lse[i * c->H + h] = -INFINITY;
    free(S);
    return;
  }
  double* qh = (double*)malloc(sizeof(double) * (size_t)D);
  for (int d = 0; d < D; ++d)
    qh[d] = oracle_bf16_decode(c->q[((int64_t)t * c->H + h) * D + d]);
  double* z = (double*)malloc(sizeof(double) * (size_t)n);
  double m = -INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    const uint16_t* row = c->kv + oracle_slot(c->bt, b, S[j]) * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += qh[d] * oracle_bf16_decode(row[d]);
    z[j] = c->sm_scale * dot;
    if (z[j] > m) m = z[j];
  }
  double sum = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    z[j] = exp(z[j] - m);
    sum += z[j];
  }
  for (int64_t j = 0; j < n; ++j) {
    const uint16_t* row = c->kv + oracle_slot(c->bt, b, S[j]) * D;
    double pj = z[j] / sum;
    for (int d = 0; d < Dv; ++d) o[d] += pj * oracle_bf16_decode(row[d]);
  }
  c->lse[i * c->H + h] = m + log(sum);
  free(z);
  free(qh);
  free(S);
}

void oracle_sparse_mla(const oracle_batch* bt, int64_t num_pages, int32_t H, int32_t D,
                       int32_t Dv, const uint16_t* q, const uint16_t* kv, const int32_t* idx,
                       int32_t k, double sm_scale, const int32_t* rows, int32_t n_rows,
                       double* out, double* lse, int threads) {
  mla_ctx c = {bt, H, D, Dv, q, kv, idx, k, sm_scale, rows, out, lse, num_pages};
  run_items((int64_t)n_rows * H, threads, mla_item, &c);
}

/* Dense MLA: the same attention over every visible position. */
void oracle_dense_mla(const oracle_batch* bt, int64_t num_pages, int32_t H, int32_t D, int32_t Dv,
                      const uint16_t* q, const uint16_t* kv, double sm_scale, const int32_t* rows,
                      int32_t n_rows, double* out, double* lse, int threads) {
  mla_ctx c = {bt, H, D, Dv, q, kv, NULL, 0, sm_scale, rows, out, lse, num_pages};
  run_items((int64_t)n_rows * H, threads, mla_item, &c);
}

/* ---- expanded multi-head attention (masked MHA) ---------------------------
 * "MTP and sparse attention: NSA and DSA", caveat on short-sequence prefill
 * and the per-pair accounting beside the DSA table: dense prefill runs the
 * expanded multi-head form, 2*H*(128 + 64) + 2*H*128 FLOPs per pair (scores
 * over 128 up-projected key dims plus the 64 shared rope dims, values of 128
 * up-projected dims per head), and the V3.2 report emulates DSA's selection
 * in that form with a mask ("masked MHA mode").  Per row t and head h, over
 * the positions S_t the row attends (idx[t] when given, else every visible
 * position; positions on a page outside the pool are left out):
 *   kn(s,d) = sum_c w_uk(h,d,c) c(s,c),   vn(s,d) = sum_c w_uv(h,d,c) c(s,c)
 *   z(s) = sm_scale * (sum_d qn(t,h,d) kn(s,d) + sum_r qr(t,h,r) kv(s,512+r))
 *   o(t,h,d) = sum_s softmax(z)(s) vn(s,d),  lse = m + ln sum_s exp(z(s) - m)
 * with c(s,.) the first 512 dims of the cached latent row, d < 128, r < 64.
 * Layouts: qn [T][H][128], qr [T][H][64], w_uk and w_uv [H][128][512], all
 * bf16; kv [pages*64][576] bf16.
 */
typedef struct {
  const oracle_batch* bt;
  int32_t H;
  const uint16_t *qn, *qr, *w_uk, *w_uv, *kv;
  const int32_t* idx;
  int32_t k;
  double sm_scale;
  const int32_t* rows;
  int32_t n_rows;
  double* out;
  double* lse;
  int64_t num_pages;
} mha_ctx;

enum { MHA_DN = 128, MHA_DR = 64, MHA_C = 512, MHA_KV = 576 };

/* One item = (request b, head h): the up-projected keys and values of the
 * request's positions are formed once, then every requested row of b
 * attends over its positions. */
static void mha_item(void* p, int64_t item) {
  mha_ctx* c = (mha_ctx*)p;
  int32_t b = (int32_t)(item / c->H);
  int32_t h = (int32_t)(item % c->H);
  /* the positions any requested row of b can see */
  int64_t vmax = 0;
  for (int32_t i = 0; i < c->n_rows; ++i)
    if (oracle_row_request(c->bt, c->rows[i]) == b) {
      int64_t v = oracle_row_visible(c->bt, c->rows[i]);
      if (v > vmax) vmax = v;
    }
  if (vmax == 0) {
    for (int32_t i = 0; i < c->n_rows; ++i)
      if (oracle_row_request(c->bt, c->rows[i]) == b) {
        double* o = c->out + ((int64_t)i * c->H + h) * MHA_DN;
        for (int d = 0; d < MHA_DN; ++d) o[d] = 0.0;
        c->lse[(int64_t)i * c->H + h] = -INFINITY;
      }
    return;
  }
  double* wk = (double*)malloc(sizeof(double) * MHA_DN * MHA_C);
  double* wv = (double*)malloc(sizeof(double) * MHA_DN * MHA_C);
  for (int64_t x = 0; x < (int64_t)MHA_DN * MHA_C; ++x) {
    wk[x] = oracle_bf16_decode(c->w_uk[(int64_t)h * MHA_DN * MHA_C + x]);
    wv[x] = oracle_bf16_decode(c->w_uv[(int64_t)h * MHA_DN * MHA_C + x]);
  }
  /* kn, vn, rope of positions 0 .. vmax-1 (unused for a page outside the pool) */
  double* kn = (double*)calloc((size_t)vmax * MHA_DN, sizeof(double));
  double* vn = (double*)calloc((size_t)vmax * MHA_DN, sizeof(double));
  double* rp = (double*)calloc((size_t)vmax * MHA_DR, sizeof(double));
  double lat[MHA_C];
  for (int64_t s = 0; s < vmax; ++s) {
    if (!oracle_page_valid(c->bt, b, s, c->num_pages)) continue;
    const uint16_t* row = c->kv + oracle_slot(c->bt, b, s) * MHA_KV;
    for (int x = 0; x < MHA_C; ++x) lat[x] = oracle_bf16_decode(row[x]);
    for (int d = 0; d < MHA_DN; ++d) {
      double a = 0.0, v = 0.0;
      for (int x = 0; x < MHA_C; ++x) {
        a += wk[d * MHA_C + x] * lat[x];
        v += wv[d * MHA_C + x] * lat[x];
      }
      kn[s * MHA_DN + d] = a;
      vn[s * MHA_DN + d] = v;
    }
    for (int r = 0; r < MHA_DR; ++r) rp[s * MHA_DR + r] = oracle_bf16_decode(row[MHA_C + r]);
  }
  int64_t* S = (int64_t*)malloc(sizeof(int64_t) * (size_t)(vmax > c->k ? vmax : c->k));
  double* z = (double*)malloc(sizeof(double) * (size_t)(vmax > c->k ? vmax : c->k));
  for (int32_t i = 0; i < c->n_rows; ++i) {
    int32_t t = c->rows[i];
    if (oracle_row_request(c->bt, t) != b) continue;
    int64_t v = oracle_row_visible(c->bt, t);
    double* o = c->out + ((int64_t)i * c->H + h) * MHA_DN;
    for (int d = 0; d < MHA_DN; ++d) o[d] = 0.0;
    /* the position list S */
    int64_t n = 0;
    if (c->idx) {
      for (int32_t j = 0; j < c->k; ++j) {
        int32_t s = c->idx[(int64_t)i * c->k + j];
        if (s >= 0 && s < v && oracle_page_valid(c->bt, b, s, c->num_pages)) S[n++] = s;
      }
    } else {
      for (int64_t s = 0; s < v; ++s)
        if (oracle_page_valid(c->bt, b, s, c->num_pages)) S[n++] = s;
    }
    if (n == 0) {
      c->lse[(int64_t)i * c->H + h] = -INFINITY;
      continue;
    }
    double qn[MHA_DN], qr[MHA_DR];
    for (int d = 0; d < MHA_DN; ++d)
      qn[d] = oracle_bf16_decode(c->qn[((int64_t)t * c->H + h) * MHA_DN + d]);
    for (int r = 0; r < MHA_DR; ++r)
      qr[r] = oracle_bf16_decode(c->qr[((int64_t)t * c->H + h) * MHA_DR + r]);
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int d = 0; d < MHA_DN; ++d) dot += qn[d] * kn[S[j] * MHA_DN + d];
      for (int r = 0; r < MHA_DR; ++r) dot += qr[r] * rp[S[j] * MHA_DR + r];
      z[j] = c->sm_scale * dot;
      if (z[j] > m) m = z[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
      z[j] = exp(z[j] - m);
      sum += z[j];
    }
    for (int64_t j = 0; j < n; ++j)
      for (int d = 0; d < MHA_DN; ++d) o[d] += z[j] / sum * vn[S[j] * MHA_DN + d];
    c->lse[(int64_t)i * c->H + h] = m + log(sum);
  }
  free(z);
  free(S);
  free(rp);
  free(vn);
  free(kn);
  free(wv);
  free(wk);
}

void oracle_masked_mha(const oracle_batch* bt, int64_t num_pages, int32_t H, const uint16_t* qn,
                       const uint16_t* qr, const uint16_t* w_uk, const uint16_t* w_uv,
                       const uint16_t* kv, const int32_t* idx, int32_t k, double sm_scale,
                       const int32_t* rows, int32_t n_rows, double* out, double* lse,
                       int threads) {
  mha_ctx c = {bt, H, qn, qr, w_uk, w_uv, kv, idx, k, sm_scale, rows, n_rows, out, lse, num_pages};
  run_items((int64_t)bt->B * H, threads, mha_item, &c);
}

/* ---- cache append ---------------------------------------------------------
 * "MTP and sparse attention: NSA and DSA", new demands on inference engines:
 * the indexer keys are a second paged cache beside the latent, stored as
 * FP8 with a 4-byte scale per key (cache accounting listing: 128 + 4 bytes
 * per token).  "[SGLang] NSA", forward_decode: the new tokens' latent rows
 * go into the paged pool before the attention.  Readings taken where the
 * pages stop: one scale per key = its largest magnitude / 448 in fp32 (1 for
 * an all-zero key), codes = e4m3fn(k / scale) rounded to nearest with ties
 * to the even code and saturated at +-448; the quotient is formed in fp32
 * (the precision the stored scale has); row j of a request with n rows and L
 * cached tokens is the token at position L - n + j. */

/* OCP e4m3fn code of x: the nearest of the 127 finite magnitudes (codes
 * 0x00 .. 0x7E, found by trying each), ties to the even code, which is the
 * even mantissa; magnitudes beyond 448 take 448; the sign is kept (-0.0 ->
 * 0x80). */
uint8_t oracle_e4m3_encode(float x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  if (isinf(x)) return (uint8_t)(sign | 0x7E);
  const double a = fabs((double)x);
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 0x7F; ++c) {
    const double d = fabs(a - oracle_e4m3_decode((uint8_t)c));
    if (d < bd || (d == bd && (c & 1) == 0)) {
      bd = d;
      best = c;
    }
  }
  return (uint8_t)(sign | best);
}

/* Writes the n_rows new tokens into the caches: k_new bf16 [T, D_idx],
 * kv_new bf16 [T, D_kv]; k8 [num_pages * page_size, D_idx], ks [...],
 * kv [..., D_kv].  Rows whose page id lies outside [0, num_pages), or whose
 * position is negative, write nothing. */
void oracle_cache_append(const oracle_batch* bt, int32_t num_pages, int32_t D_idx, int32_t D_kv,
                         const uint16_t* k_new, const uint16_t* kv_new, uint8_t* k8, float* ks,
                         uint16_t* kv) {
  for (int32_t b = 0; b < bt->B; ++b) {
    const int64_t n = bt->cu_q[b + 1] - bt->cu_q[b];
    for (int64_t j = 0; j < n; ++j) {
      const int64_t t = bt->cu_q[b] + j;
      const int64_t pos = (int64_t)bt->seqlens_k[b] - n + j;
      if (pos < 0 || pos >= (int64_t)bt->max_pages * bt->page_size) continue;
      const int64_t page = bt->page_table[(int64_t)b * bt->max_pages + pos / bt->page_size];
      if (page < 0 || page >= num_pages) continue;
      const int64_t slot = page * bt->page_size + pos % bt->page_size;
      float amax = 0.0f;
      for (int d = 0; d < D_idx; ++d) {
        const float x = (float)oracle_bf16_decode(k_new[t * D_idx + d]);
        if (fabsf(x) > amax) amax = fabsf(x);
      }
      const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
      for (int d = 0; d < D_idx; ++d) {
        const float x = (float)oracle_bf16_decode(k_new[t * D_idx + d]);
        const float qv = x / scale;
        k8[slot * D_idx + d] = oracle_e4m3_encode(qv);
      }
      ks[slot] = scale;
      for (int d = 0; d < D_kv; ++d) kv[slot * D_kv + d] = kv_new[t * D_kv + d];
    }
  }
}

/* ---- index transform -------------------------------------------------------
 * "[SGLang] NSA": the top-k's positions are turned into the page-table
 * indices the paged sparse kernel reads, or into offsets of a ragged KV
 * buffer.  idx int32 [n_rows, k] holds logical positions (-1 padding) of the
 * rows `rows`; out receives, per entry: the position itself (space 0), its
 * slot page_table[b][s / page_size] * page_size + s % page_size, -1 for a
 * page id outside [0, num_pages) (space 1), or kv_offsets[b] + s (space 2). */
void oracle_transform_index(const oracle_batch* bt, int32_t num_pages, int32_t space,
                            const int32_t* kv_offsets, const int32_t* idx, const int32_t* rows,
                            int32_t n_rows, int32_t k, int32_t* out) {
  for (int32_t i = 0; i < n_rows; ++i) {
    const int32_t b = oracle_row_request(bt, rows[i]);
    for (int32_t j = 0; j < k; ++j) {
      const int32_t s = idx[(int64_t)i * k + j];
      int32_t r = -1;
      if (s >= 0 && b >= 0) {
        if (space == 0) {
          r = s;
        } else if (space == 1) {
          const int64_t page = bt->page_table[(int64_t)b * bt->max_pages + s / bt->page_size];
          r = (page >= 0 && page < num_pages) ? (int32_t)(page * bt->page_size + s % bt->page_size)
                                              : -1;
        } else {
          r = kv_offsets[b] + s;
        }
      }
      out[(int64_t)i * k + j] = r;
    }
  }
}

/* ---- multi-layer schedule -------------------------------------------------
 * "Multi-layer Indexer: Overlapping Selection and Attention in DeepSeek
 * Sparse Attention", abstract: IndexCache keeps an indexer on a fraction 1/r
 * of the layers (here layers l with l % r == 0) and the other layers reuse
 * the latest selection; MLI lets each layer attend the previous indexer
 * layer's selection so that its own indexer runs concurrently with its
 * attention.  For each layer: produces[l] = the number of the selection it
 * makes (its rank among the indexer layers) or -1, and attends[l] = the
 * number of the selection its attention reads.  Walks the layers in order,
 * keeping the latest selection made and the one before it. */
void oracle_layer_schedule(int32_t n_layers, int32_t r, int32_t mli, int32_t* produces,
                           int32_t* attends) {
  int32_t made = 0;       /* selections made so far */
  int32_t latest = -1;    /* the newest selection, before this layer's own */
  for (int32_t l = 0; l < n_layers; ++l) {
    const int keeps = (l % r) == 0;
    produces[l] = keeps ? made : -1;
    if (keeps) {
      /* MLI: attend the selection before this layer's own, when there is one */
      attends[l] = (mli && latest >= 0) ? latest : made;
      latest = made;
      ++made;
    } else {
      attends[l] = latest;
    }
  }
}
