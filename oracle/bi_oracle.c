/*
 * bi_oracle.c -- plain, slow, fp64 CPU reference for batch-invariant
 * RMSNorm, dense matmul and causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * What it follows.  "Defeating Nondeterminism in LLM Inference" as summarised
 * on mobiles-han.blogspot.com (section on the approach, the three-row table of
 * RMSNorm / MatMul / Attention) names the three operations and demands that one
 * input always yields the same bits, whatever the batch.  The page defines none
 * of the operations, so each function below writes out the textbook
 * definition, evaluated in fp64 with one plain sequential order:
 *   - RMSNorm:   r = 1/sqrt(mean_c(x_c^2) + eps),  y_c = x_c * r * g_c
 *   - matmul:    C[i][j] = sum_k A[i][k] * W[k][j]           (W is [K][N])
 *   - attention: causal softmax(scale * q.k) . V over absolute positions, the
 *                kv head of q head h being h / (n_q / n_kv)
 * The GPU reaches these results only up to rounding, through one fixed fp32 /
 * bf16 order; the oracle is exact up to fp64 rounding.
 *
 * The split-and-fold routine evaluates the same attention a second way:
 * partial softmax sums over fixed-size key blocks at absolute multiples of the
 * block size (the "fixed-size splits" of the attention row of that table),
 * folded left in ascending block order.  Algebraically it equals the direct
 * definition, which makes it a check on the fold formula, not a second
 * reference.
 *
 * Inputs are bf16 bit patterns (uint16), decoded exactly to fp64 by the
 * oracle's own codec below.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define BIO_ABI 1

int bio_abi_version(void) { return BIO_ABI; }

/* bf16 is the top 16 bits of an IEEE binary32; widening is exact. */
static double bf16_to_f64(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

void bio_bf16_decode(const uint16_t* src, double* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_to_f64(src[i]);
}

/* The nearest bf16 to an fp64 value, rounded once (ties to even): 8
 * significant bits within binary32's exponent range, steps of 2^-133 below
 * 2^-126 (gradual underflow), infinity past the largest finite value.  A NaN
 * becomes the quiet NaN with its sign.  This is the rounding a bf16 tensor
 * applies to an exact result; going through fp32 first would round twice. */
static uint16_t f64_to_bf16(double x) {
  const uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return sign | 0x7FC0u;
  const double ax = fabs(x);
  if (isinf(ax)) return sign | 0x7F80u;
  if (ax == 0.0) return sign;
  int e;
  frexp(ax, &e); /* ax = f 2^e with 0.5 <= f < 1 */
  int q = e - 8; /* weight of the 8th significant bit */
  if (q < -133) q = -133;
  const double r = ldexp(nearbyint(ldexp(ax, -q)), q); /* scaling is exact */
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80u;
  const float f = (float)r; /* exact: at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(sign | (uint16_t)(u >> 16));
}

void bio_bf16_encode(const double* src, uint16_t* dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) dst[i] = f64_to_bf16(src[i]);
}

/* ------------------------------------------------------------------------- */
/* A tiny static work splitter over [0, n): thread t takes a contiguous range. */

typedef void (*range_fn)(void* ctx, int64_t lo, int64_t hi);
typedef struct {
  range_fn fn;
  void* ctx;
  int64_t lo, hi;
} range_job;

static void* range_trampoline(void* p) {
  range_job* j = (range_job*)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static void parallel_for(int64_t n, int nthreads, range_fn fn, void* ctx) {
  if (n <= 0) return;
  if (nthreads < 1) nthreads = 1;
  if ((int64_t)nthreads > n) nthreads = (int)n;
  if (nthreads == 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  range_job* jobs = (range_job*)malloc(sizeof(range_job) * (size_t)nthreads);
  int started = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].lo = n * t / nthreads;
    jobs[t].hi = n * (t + 1) / nthreads;
    if (t == 0) continue; /* the caller's thread runs range 0 */
    if (pthread_create(&th[t], NULL, range_trampoline, &jobs[t]) != 0) {
      fn(ctx, jobs[t].lo, jobs[t].hi); /* could not spawn: run inline */
      jobs[t].fn = NULL;
    } else {
      ++started;
    }
  }
  fn(ctx, jobs[0].lo, jobs[0].hi);
  for (int t = 1; t < nthreads; ++t)
    if (jobs[t].fn) pthread_join(th[t], NULL);
  (void)started;
  free(th);
  free(jobs);
}

/* ------------------------------------------------------------------------- */
/* RMSNorm.  x: bf16 [rows][hidden]; gamma: bf16 [hidden]; y: f64 [rows][hidden];
 * rstd: f64 [rows] or NULL.  eps is added inside the square root.            */

typedef struct {
  const uint16_t* x;
  const uint16_t* gamma;
  int64_t hidden;
  double eps;
  double* y;
  double* rstd;
} rms_ctx;

static void rms_range(void* p, int64_t lo, int64_t hi) {
  rms_ctx* c = (rms_ctx*)p;
  const int64_t H = c->hidden;
  for (int64_t r = lo; r < hi; ++r) {
    const uint16_t* xr = c->x + r * H;
    double ss = 0.0;
    for (int64_t i = 0; i < H; ++i) {
      double v = bf16_to_f64(xr[i]);
      ss += v * v;
    }
    double rs = 1.0 / sqrt(ss / (double)H + c->eps);
    if (c->rstd) c->rstd[r] = rs;
    double* yr = c->y + r * H;
    for (int64_t i = 0; i < H; ++i)
      yr[i] = bf16_to_f64(xr[i]) * rs * bf16_to_f64(c->gamma[i]);
  }
}

void bio_rmsnorm_f64(const uint16_t* x, const uint16_t* gamma, int64_t rows, int64_t hidden,
                     double eps, double* y, double* rstd, int nthreads) {
  rms_ctx c = {x, gamma, hidden, eps, y, rstd};
  parallel_for(rows, nthreads, rms_range, &c);
}

/* ------------------------------------------------------------------------- */
/* Matmul.  a: bf16 [m][k] row-major; w: bf16 [k][n] row-major; c: f64
 * [nrows][n].  Output row t is row rows[t] of A*W (rows == NULL: row t).
 * Every C[i][j] is accumulated sequentially in ascending k.                  */

typedef struct {
  const uint16_t* a;
  const double* w; /* decoded once: [k][n] */
  int64_t n, k;
  const int64_t* rows;
  double* c;
} mm_ctx;

static void mm_range(void* p, int64_t lo, int64_t hi) {
  mm_ctx* c = (mm_ctx*)p;
  const int64_t N = c->n, K = c->k;
  for (int64_t t = lo; t < hi; ++t) {
    int64_t i = c->rows ? c->rows[t] : t;
    const uint16_t* ar = c->a + i * K;
    double* cr = c->c + t * N;
    for (int64_t j = 0; j < N; ++j) cr[j] = 0.0;
    /* i-k-j loop order: each C[i][j] still sums its terms in ascending k. */
    for (int64_t kk = 0; kk < K; ++kk) {
      double av = bf16_to_f64(ar[kk]);
      const double* wr = c->w + kk * N;
      for (int64_t j = 0; j < N; ++j) cr[j] += av * wr[j];
    }
  }
}

int bio_matmul_f64(const uint16_t* a, const uint16_t* w, int64_t m, int64_t n, int64_t k,
                   const int64_t* rows, int64_t nrows, double* c, int nthreads) {
  (void)m;
  double* wd = (double*)malloc(sizeof(double) * (size_t)(k * n > 0 ? k * n : 1));
  if (!wd) return 1;
  bio_bf16_decode(w, wd, k * n);
  mm_ctx ctx = {a, wd, n, k, rows, c};
  parallel_for(nrows, nthreads, mm_range, &ctx);
  free(wd);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Causal grouped-query attention over LOGICAL (unpaged) keys and values.
 *   q:  bf16 [T][n_q][d]          one row per query token
 *   k, v: bf16 [total_kv][n_kv][d] all sequences' keys/values back to back;
 *        sequence b owns rows kv_off[b] .. kv_off[b+1]-1, row j = position j
 *   tok_seq[t], tok_pos[t]: the sequence and absolute position of query t
 *   out: f64 [T][n_q][d]; lse: f64 [T][n_q] (natural log) or NULL
 * Query at position p attends to positions 0..p of its own sequence.         */

typedef struct {
  const uint16_t *q, *k, *v;
  const int64_t* kv_off;
  const int32_t *tok_seq, *tok_pos;
  int nq, nkv, d;
  double scale;
  int split; /* 0: direct definition; >0: split-and-fold with this block size */
  double *out, *lse;
} att_ctx;

static double dot_q_k(const att_ctx* c, int64_t t, int h, int64_t krow, int g) {
  const uint16_t* qr = c->q + (t * c->nq + h) * (int64_t)c->d;
  const uint16_t* kr = c->k + (krow * c->nkv + g) * (int64_t)c->d;
  double s = 0.0;
  for (int i = 0; i < c->d; ++i) s += bf16_to_f64(qr[i]) * bf16_to_f64(kr[i]);
  return c->scale * s;
}

static void att_range(void* p, int64_t lo, int64_t hi) {
  att_ctx* c = (att_ctx*)p;
  const int d = c->d;
  const int group = c->nq / c->nkv;
  double* z = NULL;
  int64_t zcap = 0;
  double* acc = (double*)malloc(sizeof(double) * (size_t)d);
  double* oacc = (double*)malloc(sizeof(double) * (size_t)d);
  for (int64_t item = lo; item < hi; ++item) {
    const int64_t t = item / c->nq;
    const int h = (int)(item % c->nq);
    const int g = h / group;
    const int b = c->tok_seq[t];
    const int64_t pos = c->tok_pos[t];
    const int64_t base = c->kv_off[b];
    const int64_t nkeys = pos + 1;
    if (nkeys > zcap) {
      free(z);
      zcap = nkeys;
      z = (double*)malloc(sizeof(double) * (size_t)zcap);
    }
    for (int64_t j = 0; j < nkeys; ++j) z[j] = dot_q_k(c, t, h, base + j, g);
    double* o = c->out + (t * c->nq + h) * (int64_t)d;
    double m_fin, l_fin;
    if (c->split <= 0) {
      /* Direct definition: softmax with the maximum subtracted. */
      double m = -INFINITY;
      for (int64_t j = 0; j < nkeys; ++j)
        if (z[j] > m) m = z[j];
      double l = 0.0;
      for (int i = 0; i < d; ++i) acc[i] = 0.0;
      for (int64_t j = 0; j < nkeys; ++j) {
        double e = exp(z[j] - m);
        l += e;
        const uint16_t* vr = c->v + ((base + j) * c->nkv + g) * (int64_t)d;
        for (int i = 0; i < d; ++i) acc[i] += e * bf16_to_f64(vr[i]);
      }
      for (int i = 0; i < d; ++i) o[i] = acc[i] / l;
      m_fin = m;
      l_fin = l;
    } else {
      /* Partials over blocks [S*s, S*s+S) clipped to 0..pos, folded left:
       *   m' = max(m, m_s); l <- l e^{m-m'} + l_s e^{m_s-m'};
       *   o  <- o e^{m-m'} + o_s e^{m_s-m'}; finally out = o / l.          */
      const int64_t S = c->split;
      double m = -INFINITY, l = 0.0;
      for (int i = 0; i < d; ++i) oacc[i] = 0.0;
      for (int64_t s0 = 0; s0 < nkeys; s0 += S) {
        int64_t s1 = s0 + S < nkeys ? s0 + S : nkeys;
        double ms = -INFINITY;
        for (int64_t j = s0; j < s1; ++j)
          if (z[j] > ms) ms = z[j];
        double ls = 0.0;
        for (int i = 0; i < d; ++i) acc[i] = 0.0;
        for (int64_t j = s0; j < s1; ++j) {
          double e = exp(z[j] - ms);
          ls += e;
          const uint16_t* vr = c->v + ((base + j) * c->nkv + g) * (int64_t)d;
          for (int i = 0; i < d; ++i) acc[i] += e * bf16_to_f64(vr[i]);
        }
        if (s0 == 0) {
          m = ms;
          l = ls;
          for (int i = 0; i < d; ++i) oacc[i] = acc[i];
        } else {
          double mn = m > ms ? m : ms;
          double a = exp(m - mn), bb = exp(ms - mn);
          l = l * a + ls * bb;
          for (int i = 0; i < d; ++i) oacc[i] = oacc[i] * a + acc[i] * bb;
          m = mn;
        }
      }
      for (int i = 0; i < d; ++i) o[i] = oacc[i] / l;
      m_fin = m;
      l_fin = l;
    }
    if (c->lse) c->lse[t * c->nq + h] = m_fin + log(l_fin);
  }
  free(z);
  free(acc);
  free(oacc);
}

int bio_attention_f64(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      const int64_t* kv_off, const int32_t* tok_seq, const int32_t* tok_pos,
                      int64_t ntok, int nq, int nkv, int d, double scale, int split, double* out,
                      double* lse, int nthreads) {
  if (nq <= 0 || nkv <= 0 || d <= 0 || nq % nkv != 0) return 1;
  att_ctx c = {q, k, v, kv_off, tok_seq, tok_pos, nq, nkv, d, scale, split, out, lse};
  parallel_for(ntok * nq, nthreads, att_range, &c);
  return 0;
}
