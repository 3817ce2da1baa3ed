/*
 * Seeded synthetic inputs for the DSA decode path.
 *
 * This module only makes input bytes: random draws, FP8 (OCP e4m3fn) and
 * bf16 encoding of the drawn values, page permutations and heavy-token
 * positions.  It holds none of the method's arithmetic (no index score,
 * no selection, no attention).  Both the GPU path and the CPU oracle read
 * the bytes written here; neither is linked into this file.
 *
 * Random numbers come from a counter-based generator: element n of stream
 * s under seed S is mix64(key(S, s) + golden * (n + 1)), where mix64 is
 * the SplitMix64 output function (Steele, Lea, Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014).  Every element is a pure
 * function of (seed, stream, index), so the result does not depend on the
 * thread count.  Normals use the Box-Muller transform on two uniforms.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define GOLDEN 0x9e3779b97f4a7c15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64(mix64(seed + GOLDEN) ^ (stream * 0xd1b54a32d192ed03ULL));
}

static inline uint64_t draw(uint64_t key, uint64_t n) { return mix64(key + GOLDEN * (n + 1)); }

/* uniform in [0, 1) with 53 random bits */
static inline double u01(uint64_t key, uint64_t n) { return (double)(draw(key, n) >> 11) * 0x1.0p-53; }

/* uniform in (0, 1] */
static inline double u01_open0(uint64_t key, uint64_t n) {
  return (double)((draw(key, n) >> 11) + 1) * 0x1.0p-53;
}

/* standard normal number n of the stream: Box-Muller on the uniform pair
 * (2*(n/2), 2*(n/2)+1); even n takes the cosine branch, odd n the sine. */
static inline double normal(uint64_t key, uint64_t n) {
  uint64_t p = n >> 1;
  double r = sqrt(-2.0 * log(u01_open0(key, 2 * p)));
  double th = 6.283185307179586476925286766559 * u01(key, 2 * p + 1);
  return (n & 1) ? r * sin(th) : r * cos(th);
}

static inline void normal_pair(uint64_t key, uint64_t p, double* a, double* b) {
  double r = sqrt(-2.0 * log(u01_open0(key, 2 * p)));
  double th = 6.283185307179586476925286766559 * u01(key, 2 * p + 1);
  *a = r * cos(th);
  *b = r * sin(th);
}

/* ---- encoders ---------------------------------------------------------- */

/* OCP 8-bit e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities; 0x7f / 0xff are NaN; largest finite 448.  Round to nearest,
 * ties to even; magnitudes beyond 448 saturate to 448. */
uint8_t synth_e4m3_encode(double x) {
  uint8_t sign = (x < 0 || (x == 0 && signbit(x))) ? 0x80 : 0;
  double a = fabs(x);
  if (!(a == a)) return 0x7f;
  if (a >= 448.0) return sign | 0x7e;
  if (a < 0x1.0p-6) {
    /* subnormal step 2^-9; code m*2^-9 for m in 0..8 (m = 8 is 2^-6, code 8) */
    double m = rint(a * 512.0);
    return sign | (uint8_t)m;
  }
  int e2;
  double f = frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
  int e = e2 - 1;           /* a = (2f) * 2^e, 2f in [1, 2) */
  double m = rint((2.0 * f - 1.0) * 8.0);
  if (m >= 8.0) {
    m = 0.0;
    e += 1;
  }
  int be = e + 7;
  if (be > 15 || (be == 15 && m >= 7.0)) return sign | 0x7e;
  return sign | (uint8_t)((be << 3) | (int)m);
}

/* bf16 from float: round to nearest, ties to even (finite inputs). */
static inline uint16_t bf16_from_float(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint16_t synth_bf16_encode(double x) { return bf16_from_float((float)x); }

/* ---- thread helper ------------------------------------------------------ */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} job_t;

static void* job_run(void* p) {
  job_t* j = (job_t*)p;
  if (j->lo < j->hi) j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static int pick_threads(int threads) {
  if (threads > 0) return threads > 256 ? 256 : threads;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return (int)n;
}

static void parallel_for(int64_t n, int threads, range_fn fn, void* ctx) {
  int nt = pick_threads(threads);
  if (n < 4096 || nt == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t th[256];
  job_t jobs[256];
  int64_t per = (n + nt - 1) / nt;
  for (int i = 0; i < nt; ++i) {
    jobs[i].fn = fn;
    jobs[i].ctx = ctx;
    jobs[i].lo = i * per < n ? i * per : n;
    jobs[i].hi = (i + 1) * per < n ? (i + 1) * per : n;
    pthread_create(&th[i], NULL, job_run, &jobs[i]);
  }
  for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
}

/* ---- public primitives -------------------------------------------------- */

void synth_uniform(uint64_t seed, uint64_t stream, int64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = u01(key, (uint64_t)i);
}

void synth_normal(uint64_t seed, uint64_t stream, int64_t n, double* out) {
  uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = normal(key, (uint64_t)i);
}

/* uniformly random permutation of 0..n-1 (Fisher-Yates driven by the stream) */
void synth_permutation(uint64_t seed, uint64_t stream, int32_t n, int32_t* out) {
  uint64_t key = stream_key(seed, stream);
  for (int32_t i = 0; i < n; ++i) out[i] = i;
  for (int32_t i = n - 1; i > 0; --i) {
    uint64_t r = draw(key, (uint64_t)i);
    int32_t j = (int32_t)(r % (uint64_t)(i + 1));
    int32_t t = out[i];
    out[i] = out[j];
    out[j] = t;
  }
}

/* `count` distinct positions drawn uniformly from [0, n), written in the
 * order drawn (rejection of repeats).  Returns 0, or -1 if count > n. */
int synth_distinct(uint64_t seed, uint64_t stream, int32_t n, int32_t count, int32_t* out) {
  if (count > n || count < 0) return -1;
  uint64_t key = stream_key(seed, stream);
  uint8_t* seen = (uint8_t*)calloc((size_t)n, 1);
  if (!seen) return -1;
  uint64_t c = 0;
  for (int32_t k = 0; k < count;) {
    int32_t p = (int32_t)(draw(key, c++) % (uint64_t)n);
    if (!seen[p]) {
      seen[p] = 1;
      out[k++] = p;
    }
  }
  free(seen);
  return 0;
}

/* bf16 tensor of n elements, element i = bf16(float(scale * normal_i)). */
typedef struct {
  uint64_t key;
  double scale;
  uint16_t* out;
} bf16_ctx;

static void bf16_range(void* p, int64_t lo, int64_t hi) {
  bf16_ctx* c = (bf16_ctx*)p;
  int64_t i = lo;
  if (i & 1) {
    c->out[i] = bf16_from_float((float)(c->scale * normal(c->key, (uint64_t)i)));
    ++i;
  }
  for (; i + 1 < hi; i += 2) {
    double a, b;
    normal_pair(c->key, (uint64_t)(i >> 1), &a, &b);
    c->out[i] = bf16_from_float((float)(c->scale * a));
    c->out[i + 1] = bf16_from_float((float)(c->scale * b));
  }
  if (i < hi) c->out[i] = bf16_from_float((float)(c->scale * normal(c->key, (uint64_t)i)));
}

void synth_bf16_normal(uint64_t seed, uint64_t stream, int64_t n, double scale, uint16_t* out,
                       int threads) {
  bf16_ctx c = {stream_key(seed, stream), scale, out};
  parallel_for(n, threads, bf16_range, &c);
}

/* Indexer queries: T tokens of H*D values ~ N(0,1) (element n = t*H*D + i of
 * the stream).  Each token is quantised with one fp32 scale = amax / 448
 * (scale 1 for an all-zero token).  head_sum[t*D + d] receives the
 * pre-quantisation sum over heads of the token's values at dim d. */
typedef struct {
  uint64_t key;
  int H, D;
  uint8_t* q8;
  float* q_scale;
  double* head_sum;
} q_ctx;

static void q_range(void* p, int64_t lo, int64_t hi) {
  q_ctx* c = (q_ctx*)p;
  int64_t per = (int64_t)c->H * c->D;
  double* buf = (double*)malloc(sizeof(double) * (size_t)per);
  for (int64_t t = lo; t < hi; ++t) {
    double amax = 0.0;
    for (int64_t i = 0; i < per; ++i) {
      buf[i] = normal(c->key, (uint64_t)(t * per + i));
      double a = fabs(buf[i]);
      if (a > amax) amax = a;
    }
    float s = amax > 0 ? (float)(amax / 448.0) : 1.0f;
    c->q_scale[t] = s;
    for (int64_t i = 0; i < per; ++i) c->q8[t * per + i] = synth_e4m3_encode(buf[i] / (double)s);
    if (c->head_sum) {
      for (int d = 0; d < c->D; ++d) {
        double acc = 0.0;
        for (int h = 0; h < c->H; ++h) acc += buf[(int64_t)h * c->D + d];
        c->head_sum[t * c->D + d] = acc;
      }
    }
  }
  free(buf);
}

void synth_indexer_q(uint64_t seed, uint64_t stream, int32_t T, int32_t H, int32_t D, uint8_t* q8,
                     float* q_scale, double* head_sum, int threads) {
  q_ctx c = {stream_key(seed, stream), H, D, q8, q_scale, head_sum};
  int64_t n = T;
  /* parallel_for only splits ranges of >= 4096 items; tokens are heavy, so
   * split by hand when there are fewer. */
  if (n < 4096) {
    int nt = pick_threads(threads);
    if (nt > n) nt = (int)(n > 0 ? n : 1);
    pthread_t th[256];
    job_t jobs[256];
    int64_t per = (n + nt - 1) / nt;
    for (int i = 0; i < nt; ++i) {
      jobs[i].fn = q_range;
      jobs[i].ctx = &c;
      jobs[i].lo = i * per < n ? i * per : n;
      jobs[i].hi = (i + 1) * per < n ? (i + 1) * per : n;
      pthread_create(&th[i], NULL, job_run, &jobs[i]);
    }
    for (int i = 0; i < nt; ++i) pthread_join(th[i], NULL);
  } else {
    parallel_for(n, threads, q_range, &c);
  }
}

/* Indexer keys of a batch, written at their physical cache slots.
 *
 * Request b has L[b] tokens; token s of request b is logical key
 * g = key_off[b] + s.  Its pre-quantisation value at dim d is
 *   normal(base stream, g*D + d)
 *   + heavy_gain * dir[b*D + d]            if heavy[g] != 0
 *   + noise_scale * normal(noise stream, g*D + d)   if noise_scale != 0
 * and it is quantised with one fp32 scale = amax / 448 into
 * k8[slot*D ...], k_scale[slot], slot = page_table[b*max_pages + s/P]*P + s%P.
 */
typedef struct {
  uint64_t key_base, key_noise;
  double noise_scale, heavy_gain;
  int32_t B, D, P, max_pages;
  const int32_t* L;
  const int64_t* key_off;
  const int32_t* page_table;
  const double* dir;
  const uint8_t* heavy;
  uint8_t* k8;
  float* k_scale;
  int64_t total;
} k_ctx;

static void k_range(void* p, int64_t lo, int64_t hi) {
  k_ctx* c = (k_ctx*)p;
  double* buf = (double*)malloc(sizeof(double) * (size_t)c->D);
  int32_t b = 0;
  for (int64_t g = lo; g < hi; ++g) {
    while (b + 1 < c->B && c->key_off[b + 1] <= g) ++b;
    int64_t s = g - c->key_off[b];
    double amax = 0.0;
    /* D is even, so the key's normals are whole Box-Muller pairs */
    for (int d = 0; d < c->D; d += 2)
      normal_pair(c->key_base, (uint64_t)(g * c->D + d) >> 1, &buf[d], &buf[d + 1]);
    if (c->heavy && c->heavy[g])
      for (int d = 0; d < c->D; ++d) buf[d] += c->heavy_gain * c->dir[(int64_t)b * c->D + d];
    if (c->noise_scale != 0.0) {
      for (int d = 0; d < c->D; d += 2) {
        double e0, e1;
        normal_pair(c->key_noise, (uint64_t)(g * c->D + d) >> 1, &e0, &e1);
        buf[d] += c->noise_scale * e0;
        buf[d + 1] += c->noise_scale * e1;
      }
    }
    for (int d = 0; d < c->D; ++d)
      if (fabs(buf[d]) > amax) amax = fabs(buf[d]);
    float sc = amax > 0 ? (float)(amax / 448.0) : 1.0f;
    int64_t page = c->page_table[(int64_t)b * c->max_pages + s / c->P];
    int64_t slot = page * c->P + s % c->P;
    c->k_scale[slot] = sc;
    for (int d = 0; d < c->D; ++d) c->k8[slot * c->D + d] = synth_e4m3_encode(buf[d] / (double)sc);
  }
  free(buf);
}

void synth_indexer_keys(uint64_t seed, uint64_t stream_base, uint64_t stream_noise, double noise_scale,
                        int32_t B, int32_t D, int32_t P, const int32_t* L, const int64_t* key_off,
                        const int32_t* page_table, int32_t max_pages, const double* dir,
                        const uint8_t* heavy, double heavy_gain, uint8_t* k8, float* k_scale,
                        int threads) {
  k_ctx c;
  c.key_base = stream_key(seed, stream_base);
  c.key_noise = stream_key(seed, stream_noise);
  c.noise_scale = noise_scale;
  c.heavy_gain = heavy_gain;
  c.B = B;
  c.D = D;
  c.P = P;
  c.max_pages = max_pages;
  c.L = L;
  c.key_off = key_off;
  c.page_table = page_table;
  c.dir = dir;
  c.heavy = heavy;
  c.k8 = k8;
  c.k_scale = k_scale;
  c.total = key_off[B - 1] + L[B - 1];
  parallel_for(c.total, threads, k_range, &c);
}
