/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the weight-streaming
 * skinny matmul C[m,n] = A[m,k] . W[k,n] and the steps around it (Q8_0-,
 * Q4_0- and Q2_0-style block dequant, per-row top-k, the window-row cast, the
 * gate).
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the bench's
 * CPU-baseline leg call this code; the library's product path never does, and
 * this file shares no source, header, table or helper with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread oracle.c -o liboracle.so
 * (no fast-math: every fp64 operation below is the IEEE operation written).
 *
 * Conventions (the readings are listed with their reasons in the design notes):
 *   - 16-bit floating inputs are passed as raw bit patterns (uint16), IEEE
 *     binary16 ("f16") or bfloat16 ("bf16").
 *   - A is [m][k] row-major with row stride lda (elements).
 *   - W is stored [n][k], k-contiguous: stored row j holds the logical column
 *     j of W[k,n].  So C[i][j] = sum_kk A[i][kk] * W[j][kk].
 *   - C is produced in fp64, [m][n] row-major with row stride ldc.
 *
 * Sources for what is computed:
 *   - the product itself: the nx_batchscale_kat page states the problem as
 *     C[m,n] = A[m,k] . W[k,n] with fp32 (here: exact-as-possible fp64)
 *     accumulation; the Strata PR #109 page ("What") requires every row of a
 *     batched call to equal the single-row call, which an order-free fp64
 *     reference is the natural yardstick for.
 *   - dequant: the opus r35 track A page (section 1, router dequant reuse)
 *     dequantises block-quantised weights to f16 with a `dq_f16` kernel but
 *     defines no format; the format fixed here is Q8_0-style: blocks of 32
 *     consecutive k, int8 codes q and one f16 scale d per block, w = d * q,
 *     rounded once to f16 (round to nearest, ties to even).
 *   - top-k: the Strata PR #109 page ("What", router bullet) takes a per-row
 *     top-10 of the router logits; ordered by value descending, equal values
 *     (IEEE ==, so -0 == +0) by lower index first.
 *   - the window-row cast and the scalar gate: the Strata PR #109 page
 *     ("What", the bf16 cast and shared-expert gate bullets) casts the
 *     window's fp32 rows to bf16 and gates the shared expert with a
 *     multi-row GEMV followed by a sigmoid; the cast rounds to nearest, ties
 *     to even, and the sigmoid is the logistic function 1 / (1 + e^-x).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_Q8_0 = 4, ORACLE_Q4_0 = 5, ORACLE_Q2_0 = 6 };

/* ---------------------------------------------------------------------------
 * Scalar conversions, written from the format definitions.
 * ------------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 = subnormal (fraction * 2^-24), exponent 31 = inf/NaN. */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32 (8 exponent bits, bias 127,
 * 7 fraction bits). */
double oracle_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -133); /* f * 2^-7 * 2^-126 */
  } else if (e == 255) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(128 + f), e - 134); /* (1 + f/128) * 2^(e-127) */
  }
  return sign ? -v : v;
}

/* Round a finite double to the nearest binary16, ties to even; magnitudes
 * that round to 2^16 or beyond become infinity.  Written from the definition:
 * find the spacing of f16 values around |x|, count |x| in units of that
 * spacing, round that count to an integer (ties to even), and encode. */
uint16_t oracle_f64_to_f16_rne(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (isnan(x)) return 0x7e00;
  if (isinf(x)) return sign | 0x7c00;
  if (ax == 0.0) return sign;

  int e2;               /* ax = fr * 2^e2, fr in [0.5, 1) */
  (void)frexp(ax, &e2);
  int E = e2 - 1;       /* ax in [2^E, 2^(E+1)) */
  int quantum_exp;      /* spacing of f16 values at ax is 2^quantum_exp */
  if (E < -14) {
    quantum_exp = -24;  /* subnormal range: fixed spacing 2^-24 */
  } else {
    quantum_exp = E - 10;
  }
  double units = ldexp(ax, -quantum_exp); /* exact: scaling by a power of two */
  double lo = floor(units);
  double frac = units - lo;               /* exact: the fraction bits of units */
  double r;
  if (frac > 0.5) {
    r = lo + 1.0;
  } else if (frac < 0.5) {
    r = lo;
  } else {
    r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0; /* tie: to even */
  }

  if (E < -14) {
    /* r in [0, 1024]; r == 1024 is 2^-14, the smallest normal, whose bit
     * pattern 0x0400 is exactly the integer 1024. */
    return sign | (uint16_t)r;
  }
  /* normal: r in [1024, 2048]; 2048 carries into the next binade */
  int exp_field = E + 15;
  int ri = (int)r;
  if (ri == 2048) {
    ri = 1024;
    exp_field += 1;
  }
  if (exp_field >= 31) return sign | 0x7c00;
  return sign | (uint16_t)((exp_field << 10) | (ri - 1024));
}

/* bfloat16 round to nearest, ties to even, by the same method as the f16
 * encoder above.  bfloat16 keeps binary32's exponent range: normals from
 * 2^-126 with 8 significant bits (spacing 2^(E-7) in [2^E, 2^(E+1))),
 * subnormals with the fixed spacing 2^-133, largest finite (2 - 2^-7) * 2^127;
 * anything that rounds past it is infinity. */
uint16_t oracle_f64_to_bf16_rne(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double ax = fabs(x);
  if (isnan(x)) return 0x7fc0;
  if (isinf(x)) return sign | 0x7f80;
  if (ax == 0.0) return sign;

  int e2;
  (void)frexp(ax, &e2);
  int E = e2 - 1;       /* ax in [2^E, 2^(E+1)) */
  int quantum_exp = (E < -126) ? -133 : E - 7;
  double units = ldexp(ax, -quantum_exp);
  double lo = floor(units);
  double frac = units - lo;
  double r;
  if (frac > 0.5) {
    r = lo + 1.0;
  } else if (frac < 0.5) {
    r = lo;
  } else {
    r = (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0; /* tie: to even */
  }
  if (E < -126) {
    /* r in [0, 128]; 128 is 2^-126, the smallest normal, pattern 0x0080 */
    return sign | (uint16_t)r;
  }
  int exp_field = E + 127;
  int ri = (int)r;   /* in [128, 256]; 256 carries into the next binade */
  if (ri == 256) {
    ri = 128;
    exp_field += 1;
  }
  if (exp_field >= 255) return sign | 0x7f80;
  return sign | (uint16_t)((exp_field << 7) | (ri - 128));
}

/* The window-row cast: out[i] = RNE_bf16(in[i]) for binary32 inputs (each is
 * exact in fp64, so rounding the fp64 value is rounding the fp32 value). */
void oracle_cast_f32_bf16(int64_t count, const float* in, uint16_t* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = oracle_f64_to_bf16_rne((double)in[i]);
}

/* The scalar gate's nonlinearity, elementwise: y[i] = 1 / (1 + e^-x[i]). */
void oracle_sigmoid(int64_t count, const double* x, double* y) {
  for (int64_t i = 0; i < count; ++i) y[i] = 1.0 / (1.0 + exp(-x[i]));
}

/* ---------------------------------------------------------------------------
 * Dequant of the Q8_0-style block format.
 *   qs: int8 [n][k] (k-contiguous), d: f16 bits [n][k/32], out: f16 bits [n][k]
 *   out[j][kk] = RNE_f16( d[j][kk/32] * qs[j][kk] )   (product exact in fp64)
 * Returns 0, or -1 when k is not a multiple of 32.
 * ------------------------------------------------------------------------- */
int oracle_dequant_q8_0(int64_t n, int64_t k, const int8_t* qs, const uint16_t* d,
                        uint16_t* out) {
  if (k % 32 != 0) return -1;
  int64_t nb = k / 32;
  for (int64_t j = 0; j < n; ++j) {
    for (int64_t kk = 0; kk < k; ++kk) {
      double scale = oracle_f16_to_f64(d[j * nb + kk / 32]);
      double w = scale * (double)qs[j * k + kk];
      out[j * k + kk] = oracle_f64_to_f16_rne(w);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Dequant of the Q4_0-style block format (4-bit codes).  The pages name 4-
 * and 2-bit block formats (the Strata PR #109 page, "Measured": IQ3_S and
 * Q2_0 runs) without defining one, so this format is fixed here:
 *   blocks of 32 consecutive k, one f16 scale d per block, unsigned 4-bit
 *   codes q in 0..15 stored two per byte, element kk of a row in byte kk / 2
 *   (the low nibble for even kk, the high nibble for odd kk); the weight is
 *   d * (q - 8), rounded once to f16 (round to nearest, ties to even).
 *   qs: uint8 [n][k/2], d: f16 bits [n][k/32], out: f16 bits [n][k]
 * The product is exact in fp64 (an 11-bit significand times an integer of
 * magnitude at most 8).  Returns 0, or -1 when k is not a multiple of 32.
 * ------------------------------------------------------------------------- */
int oracle_dequant_q4_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                        uint16_t* out) {
  if (k % 32 != 0) return -1;
  int64_t nb = k / 32;
  for (int64_t j = 0; j < n; ++j) {
    for (int64_t kk = 0; kk < k; ++kk) {
      uint8_t byte = qs[j * (k / 2) + kk / 2];
      int q = (kk % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
      double scale = oracle_f16_to_f64(d[j * nb + kk / 32]);
      double w = scale * (double)(q - 8);
      out[j * k + kk] = oracle_f64_to_f16_rne(w);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Dequant of the Q2_0-style block format (2-bit codes).  The Strata PR #109
 * page names a 2-bit block format ("Measured": Q2_0 runs) without defining
 * it, so this format is fixed here as the 2-bit counterpart of the Q4_0-style
 * one above:
 *   blocks of 32 consecutive k, one f16 scale d per block, unsigned 2-bit
 *   codes q in 0..3 stored four per byte, element kk of a row in byte kk / 4
 *   at bits 2 * (kk % 4) and 2 * (kk % 4) + 1 (the first element of a byte in
 *   its lowest two bits); the weight is d * (q - 2), rounded once to f16
 *   (round to nearest, ties to even).
 *   qs: uint8 [n][k/4], d: f16 bits [n][k/32], out: f16 bits [n][k]
 * The product is exact in fp64 (q - 2 is -2, -1, 0 or 1); the rounding only
 * matters where 2 * |d| passes the largest f16.  Returns 0, or -1 when k is
 * not a multiple of 32.
 * ------------------------------------------------------------------------- */
int oracle_dequant_q2_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                        uint16_t* out) {
  if (k % 32 != 0) return -1;
  int64_t nb = k / 32;
  for (int64_t j = 0; j < n; ++j) {
    for (int64_t kk = 0; kk < k; ++kk) {
      uint8_t byte = qs[j * (k / 4) + kk / 4];
      int q = (byte >> (2 * (kk % 4))) & 0x3;
      double scale = oracle_f16_to_f64(d[j * nb + kk / 32]);
      double w = scale * (double)(q - 2);
      out[j * k + kk] = oracle_f64_to_f16_rne(w);
    }
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * The matmul.  Inputs are decoded to fp64 once, then every C[i][j] is one
 * sequential fp64 sum over kk = 0..k-1.  Threads split the (i, j) pairs into
 * contiguous column blocks per row; no dot product is ever split.
 * When `absolute` is non-zero the oracle instead returns sum |A| * |W|, which
 * the tests use to bound fp32 rounding error.
 * ------------------------------------------------------------------------- */
typedef struct {
  int64_t m, n, k;
  const double* a;  /* [m][k] */
  const double* w;  /* [n][k] */
  double* c;
  int64_t ldc;
  int absolute;
  int64_t first, last; /* range of flattened (i, j-block) work items */
  int64_t jblock;
} mm_job;

static void* mm_worker(void* arg) {
  mm_job* jb = (mm_job*)arg;
  int64_t nblk = (jb->n + jb->jblock - 1) / jb->jblock;
  for (int64_t item = jb->first; item < jb->last; ++item) {
    int64_t i = item / nblk;
    int64_t j0 = (item % nblk) * jb->jblock;
    int64_t j1 = j0 + jb->jblock < jb->n ? j0 + jb->jblock : jb->n;
    const double* arow = jb->a + i * jb->k;
    for (int64_t j = j0; j < j1; ++j) {
      const double* wrow = jb->w + j * jb->k;
      double s = 0.0;
      if (jb->absolute) {
        for (int64_t kk = 0; kk < jb->k; ++kk) s += fabs(arow[kk]) * fabs(wrow[kk]);
      } else {
        for (int64_t kk = 0; kk < jb->k; ++kk) s += arow[kk] * wrow[kk];
      }
      jb->c[i * jb->ldc + j] = s;
    }
  }
  return NULL;
}

static double decode16(int kind, uint16_t v) {
  return kind == ORACLE_BF16 ? oracle_bf16_to_f64(v) : oracle_f16_to_f64(v);
}

/* A: bits [m][lda] (f16 or bf16, a_kind).  W: for F16/BF16 bits [n][k]; for
 * Q8_0 int8 codes [n][k], for Q4_0 packed codes uint8 [n][k/2], for Q2_0
 * packed codes uint8 [n][k/4], each with
 * w_scales f16 bits [n][k/32].  C: fp64 [m][ldc].
 * threads <= 0 means 1.  Returns 0, -1 on a bad argument, -2 on no memory. */
int oracle_mm(int64_t m, int64_t n, int64_t k, int a_kind, const uint16_t* A, int64_t lda,
              int w_kind, const void* W, const uint16_t* w_scales, double* C, int64_t ldc,
              int threads, int absolute) {
  if (m < 0 || n < 0 || k < 0 || lda < k || ldc < n) return -1;
  if (a_kind != ORACLE_F16 && a_kind != ORACLE_BF16) return -1;
  const int blockq = w_kind == ORACLE_Q8_0 || w_kind == ORACLE_Q4_0 || w_kind == ORACLE_Q2_0;
  if (w_kind != ORACLE_F16 && w_kind != ORACLE_BF16 && !blockq) return -1;
  if (blockq && (k % 32 != 0 || w_scales == NULL)) return -1;
  if (m == 0 || n == 0) return 0;

  double* a = (double*)malloc(sizeof(double) * (size_t)(m * k + 1));
  double* w = (double*)malloc(sizeof(double) * (size_t)(n * k + 1));
  uint16_t* deq = NULL;
  if (!a || !w) {
    free(a);
    free(w);
    return -2;
  }
  for (int64_t i = 0; i < m; ++i)
    for (int64_t kk = 0; kk < k; ++kk) a[i * k + kk] = decode16(a_kind, A[i * lda + kk]);

  if (blockq) {
    deq = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * k + 1));
    if (!deq) {
      free(a);
      free(w);
      return -2;
    }
    if (w_kind == ORACLE_Q8_0)
      oracle_dequant_q8_0(n, k, (const int8_t*)W, w_scales, deq);
    else if (w_kind == ORACLE_Q4_0)
      oracle_dequant_q4_0(n, k, (const uint8_t*)W, w_scales, deq);
    else
      oracle_dequant_q2_0(n, k, (const uint8_t*)W, w_scales, deq);
    for (int64_t idx = 0; idx < n * k; ++idx) w[idx] = oracle_f16_to_f64(deq[idx]);
    free(deq);
  } else {
    const uint16_t* wb = (const uint16_t*)W;
    for (int64_t idx = 0; idx < n * k; ++idx) w[idx] = decode16(w_kind, wb[idx]);
  }

  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  int64_t jblock = 64;
  int64_t nblk = (n + jblock - 1) / jblock;
  int64_t items = m * nblk;
  if (threads > items) threads = (int)items;

  mm_job jobs[256];
  pthread_t tids[256];
  int spawned[256];
  int64_t per = (items + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    mm_job* jb = &jobs[t];
    jb->m = m; jb->n = n; jb->k = k; jb->a = a; jb->w = w; jb->c = C; jb->ldc = ldc;
    jb->absolute = absolute; jb->jblock = jblock;
    jb->first = t * per;
    jb->last = (t + 1) * per < items ? (t + 1) * per : items;
    spawned[t] = 0;
  }
  /* threads 1.. run on their own pthreads; job 0 (and any job whose spawn
   * failed) runs on the calling thread */
  for (int t = 1; t < threads; ++t)
    if (jobs[t].first < jobs[t].last)
      spawned[t] = pthread_create(&tids[t], NULL, mm_worker, &jobs[t]) == 0;
  for (int t = 0; t < threads; ++t)
    if (!spawned[t] && jobs[t].first < jobs[t].last) mm_worker(&jobs[t]);
  for (int t = 1; t < threads; ++t)
    if (spawned[t]) pthread_join(tids[t], NULL);
  free(a);
  free(w);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Top-k of each row of a logit matrix: sort the row's (value, index) pairs by
 * value descending, equal values by index ascending, keep the first topk.
 * Logits are fp64 here; callers pass fp32 logits widened exactly.
 * ------------------------------------------------------------------------- */
typedef struct {
  double v;
  int32_t i;
} vi_pair;

static int by_value_desc_index_asc(const void* pa, const void* pb) {
  const vi_pair* a = (const vi_pair*)pa;
  const vi_pair* b = (const vi_pair*)pb;
  if (a->v > b->v) return -1;
  if (a->v < b->v) return 1;
  return (a->i < b->i) ? -1 : (a->i > b->i);  /* equal values (incl. -0 == +0) */
}

int oracle_topk(int64_t m, int64_t n, const double* logits, int64_t ldl, int32_t topk,
                int32_t* idx, double* val) {
  if (m < 0 || n < 1 || topk < 1 || topk > n || ldl < n) return -1;
  vi_pair* row = (vi_pair*)malloc(sizeof(vi_pair) * (size_t)n);
  if (!row) return -2;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      row[j].v = logits[i * ldl + j];
      row[j].i = (int32_t)j;
    }
    qsort(row, (size_t)n, sizeof(vi_pair), by_value_desc_index_asc);
    for (int32_t t = 0; t < topk; ++t) {
      idx[i * topk + t] = row[t].i;
      val[i * topk + t] = row[t].v;
    }
  }
  free(row);
  return 0;
}
