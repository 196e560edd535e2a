/*
 * bnn_oracle.c -- plain, slow CPU oracle for packed binary (+1/-1) products.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the test oracle, not the product: only
 * the test-suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it.  It shares no code, header, table or constant with the HIP library
 * and includes nothing from it.
 *
 * Sources (cited by page title and section):
 *   [BME]  "Binary Math Effectiveness -- why / how / when" (Binary-Neural-
 *          Networks lab docs), section 1 "The core identity": the encoding
 *          table (bit 0 means +1, bit 1 means -1), the definition of the dot
 *          product of two +-1 vectors, and the edge-case table (pad bits
 *          encode +1 and only the logical length n counts; n = 0 gives 0; a
 *          channel scale alpha = 0 gives 0; non-+-1 inputs are projected to
 *          -1 when <= 0 and to +1 when > 0).
 *   [BME 2.1] same page, section 2.1 "Arithmetic": a row of K values takes
 *          ceil(K/64) 64-bit words.
 *
 * How it computes: every product is taken from its DEFINITION.  Packed rows
 * are unpacked to +-1 integers (reading only the K logical bits), and each
 * output is the plain sum over k of x[k]*w[k].  The XOR/popcount identity of
 * [BME 1] is deliberately NOT used here, so that the tests can check the
 * identity (and the GPU path, which uses it) against this definition.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *   - bit order inside a word: element k is bit (k % 64) of word (k / 64),
 *     least significant bit first; words are stored little-endian.
 *   - projection of +0, -0 and NaN: -1 (they are not > 0); positive
 *     subnormals: +1 (no flush to zero; compile without fast-math).
 *   - bf16 values are widened to fp32 exactly (bits << 16) before the test.
 *   - the sign->repack output bit is 1 (-1) when the integer dot is <= 0,
 *     packed along N with the same bit order; pad bits are 0 (+1).
 *   - scaled output: one fp32 multiply, (float)dot * alpha[n], rounded to
 *     nearest even.
 *   - threshold repack ("Architecture Decision Record", Decision: "BN after
 *     binary"): a BatchNorm followed by the next layer's projection reduces
 *     to "-1 when dot <= t[n]", inverted on channels with a negative scale.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread
 *        bnn_oracle.c -o libbnn_oracle.so
 */
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* [BME 2.1]: number of 64-bit words holding k logical values. */
int64_t oracle_words(int64_t k) { return k <= 0 ? 0 : (k + 63) / 64; }

/* [BME 1] edge-case table, "non-+-1 inputs": > 0 projects to +1, anything
 * else (<= 0, and NaN, which is not > 0) projects to -1. */
int oracle_sign_f32(float v) { return (v > 0.0f) ? 1 : -1; }

/* bf16 is the upper half of an fp32 bit pattern; widening is exact. */
float oracle_bf16_to_f32(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

int oracle_sign_bf16(uint16_t h) { return oracle_sign_f32(oracle_bf16_to_f32(h)); }

/* [BME 1] encoding table: +1 is stored as bit 0, -1 as bit 1. */
static uint64_t bit_of_sign(int s) { return s < 0 ? 1u : 0u; }

/* Read logical element k of a packed row (no pad bit is ever read). */
static int packed_sign_at(const uint64_t *row, int64_t k) {
  uint64_t bit = (row[k / 64] >> (k % 64)) & 1u;
  return bit ? -1 : 1;
}

/* Pack rows x k fp32 values (row stride ld elements) into rows x words(k)
 * words.  Every bit starts at 0, so pad bits encode +1 ([BME 1] padding). */
void oracle_pack_f32(const float *src, int64_t rows, int64_t k, int64_t ld, uint64_t *dst) {
  int64_t kw = oracle_words(k);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t w = 0; w < kw; ++w) dst[r * kw + w] = 0;
    for (int64_t i = 0; i < k; ++i) {
      int s = oracle_sign_f32(src[r * ld + i]);
      dst[r * kw + i / 64] |= bit_of_sign(s) << (i % 64);
    }
  }
}

/* Same as oracle_pack_f32 for bf16 input given as raw 16-bit patterns. */
void oracle_pack_bf16(const uint16_t *src, int64_t rows, int64_t k, int64_t ld, uint64_t *dst) {
  int64_t kw = oracle_words(k);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t w = 0; w < kw; ++w) dst[r * kw + w] = 0;
    for (int64_t i = 0; i < k; ++i) {
      int s = oracle_sign_bf16(src[r * ld + i]);
      dst[r * kw + i / 64] |= bit_of_sign(s) << (i % 64);
    }
  }
}

/* Unpack rows x words(k) packed words to rows x k int8 values in {+1, -1}.
 * Only the k logical bits of each row are read ([BME 1]: logical n). */
void oracle_unpack(const uint64_t *p, int64_t rows, int64_t k, int8_t *out) {
  int64_t kw = oracle_words(k);
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t i = 0; i < k; ++i) out[r * k + i] = (int8_t)packed_sign_at(p + r * kw, i);
}

/* Definition of the dot product of two +-1 vectors of length k: the sum of
 * the elementwise products.  k = 0 gives the empty sum 0 ([BME 1], n = 0). */
static int64_t dot_pm1(const int8_t *a, const int8_t *b, int64_t k) {
  int64_t s = 0;
  for (int64_t i = 0; i < k; ++i) s += (int64_t)a[i] * (int64_t)b[i];
  return s;
}

/* ------------------------------------------------------------------------ */
/* Row-parallel driver: rows of X are split over threads; integer sums make
 * the result independent of the split. */

enum { OUT_I32 = 0, OUT_SCALED = 1, OUT_REPACK = 2, OUT_REPACK_THR = 3 };

typedef struct {
  const uint64_t *xp;
  const int8_t *wu; /* W unpacked once: N x K */
  const float *alpha;
  const int32_t *thr;   /* OUT_REPACK_THR: per-channel threshold */
  const uint8_t *flip;  /* OUT_REPACK_THR: per-channel flip, or NULL */
  void *y;
  int64_t m_begin, m_end, N, K;
  int mode;
} job_t;

static void *gemm_rows(void *arg) {
  job_t *j = (job_t *)arg;
  int64_t kw = oracle_words(j->K);
  int64_t nw = oracle_words(j->N);
  int8_t *xu = (int8_t *)malloc((size_t)(j->K > 0 ? j->K : 1));
  for (int64_t m = j->m_begin; m < j->m_end; ++m) {
    oracle_unpack(j->xp + m * kw, 1, j->K, xu);
    if (j->mode == OUT_REPACK) {
      uint64_t *yp = (uint64_t *)j->y + m * nw;
      for (int64_t w = 0; w < nw; ++w) yp[w] = 0;
      for (int64_t n = 0; n < j->N; ++n) {
        int64_t d = dot_pm1(xu, j->wu + n * j->K, j->K);
        /* [BME 1] projection applied to the integer output: <= 0 -> -1. */
        int s = (d > 0) ? 1 : -1;
        yp[n / 64] |= bit_of_sign(s) << (n % 64);
      }
    } else if (j->mode == OUT_REPACK_THR) {
      /* "Architecture Decision Record", Decision, "BN after binary": the next
       * layer's input bit is the projection of a per-channel affine function
       * of the dot, which reduces to "-1 when d <= t[n]", inverted when f[n]
       * is set. */
      uint64_t *yp = (uint64_t *)j->y + m * nw;
      for (int64_t w = 0; w < nw; ++w) yp[w] = 0;
      for (int64_t n = 0; n < j->N; ++n) {
        int64_t d = dot_pm1(xu, j->wu + n * j->K, j->K);
        int minus = d <= (int64_t)j->thr[n];
        if (j->flip && j->flip[n]) minus = !minus;
        yp[n / 64] |= (uint64_t)minus << (n % 64);
      }
    } else {
      for (int64_t n = 0; n < j->N; ++n) {
        int64_t d = dot_pm1(xu, j->wu + n * j->K, j->K);
        if (j->mode == OUT_I32) {
          ((int32_t *)j->y)[m * j->N + n] = (int32_t)d;
        } else {
          /* [BME 1] channel scale: one fp32 product of the exact integer. */
          float fd = (float)d;
          float r = fd * j->alpha[n];
          ((float *)j->y)[m * j->N + n] = r;
        }
      }
    }
  }
  free(xu);
  return NULL;
}

static int resolve_threads(int nthreads, int64_t M) {
  if (nthreads <= 0) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = c > 0 ? (int)c : 1;
  }
  if (nthreads > 256) nthreads = 256;
  if (M < nthreads) nthreads = (int)(M > 0 ? M : 1);
  return nthreads;
}

static void run(const uint64_t *xp, const uint64_t *wp, const float *alpha, const int32_t *thr,
                const uint8_t *flip, void *y, int64_t M, int64_t N, int64_t K, int mode,
                int nthreads) {
  if (M <= 0 || N <= 0) return;
  int64_t kk = K > 0 ? K : 0;
  int8_t *wu = (int8_t *)malloc((size_t)(N * kk > 0 ? N * kk : 1));
  oracle_unpack(wp, N, kk, wu);
  int nt = resolve_threads(nthreads, M);
  pthread_t th[256];
  job_t jobs[256];
  for (int t = 0; t < nt; ++t) {
    jobs[t].xp = xp;
    jobs[t].wu = wu;
    jobs[t].alpha = alpha;
    jobs[t].thr = thr;
    jobs[t].flip = flip;
    jobs[t].y = y;
    jobs[t].m_begin = M * t / nt;
    jobs[t].m_end = M * (t + 1) / nt;
    jobs[t].N = N;
    jobs[t].K = kk;
    jobs[t].mode = mode;
  }
  for (int t = 1; t < nt; ++t) pthread_create(&th[t], NULL, gemm_rows, &jobs[t]);
  gemm_rows(&jobs[0]);
  for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
  free(wu);
}

/* Y[m][n] = <x_m, w_n> over the K logical elements; X is M x words(K),
 * W is N x words(K) (rows are output channels), Y is M x N row-major. */
void oracle_gemm_i32(const uint64_t *xp, const uint64_t *wp, int64_t M, int64_t N, int64_t K,
                     int32_t *y, int nthreads) {
  run(xp, wp, NULL, NULL, NULL, y, M, N, K, OUT_I32, nthreads);
}

/* Y[m][n] = (float)<x_m, w_n> * alpha[n]  ([BME 1], channel scale). */
void oracle_gemm_scaled(const uint64_t *xp, const uint64_t *wp, const float *alpha, int64_t M,
                        int64_t N, int64_t K, float *y, int nthreads) {
  run(xp, wp, alpha, NULL, NULL, y, M, N, K, OUT_SCALED, nthreads);
}

/* Packed M x words(N): bit n of row m is the projected sign of <x_m, w_n>. */
void oracle_sign_repack(const uint64_t *xp, const uint64_t *wp, int64_t M, int64_t N, int64_t K,
                        uint64_t *yp, int nthreads) {
  run(xp, wp, NULL, NULL, NULL, yp, M, N, K, OUT_REPACK, nthreads);
}

/* Packed M x words(N): bit n of row m is 1 when <x_m, w_n> <= thr[n], inverted
 * where flip[n] is non-zero (flip may be NULL).  A BatchNorm between binary
 * layers ("BN after binary", Architecture Decision Record) folds into
 * (thr, flip); thr = 0 with no flips is oracle_sign_repack. */
void oracle_sign_repack_thr(const uint64_t *xp, const uint64_t *wp, const int32_t *thr,
                            const uint8_t *flip, int64_t M, int64_t N, int64_t K, uint64_t *yp,
                            int nthreads) {
  run(xp, wp, NULL, thr, flip, yp, M, N, K, OUT_REPACK_THR, nthreads);
}

/* out[i] = <x_{mi[i]}, w_{ni[i]}> for a list of (m, n) pairs: the sampled
 * form of oracle_gemm_i32, used where the full product is too large. */
void oracle_dot_pairs(const uint64_t *xp, const uint64_t *wp, int64_t K, const int64_t *mi,
                      const int64_t *ni, int64_t count, int32_t *out) {
  int64_t kw = oracle_words(K);
  int64_t kk = K > 0 ? K : 0;
  int8_t *a = (int8_t *)malloc((size_t)(kk > 0 ? kk : 1));
  int8_t *b = (int8_t *)malloc((size_t)(kk > 0 ? kk : 1));
  for (int64_t i = 0; i < count; ++i) {
    oracle_unpack(xp + mi[i] * kw, 1, kk, a);
    oracle_unpack(wp + ni[i] * kw, 1, kk, b);
    out[i] = (int32_t)dot_pm1(a, b, kk);
  }
  free(a);
  free(b);
}

/* ------------------------------------------------------------------------ */
/* Real-valued activations times packed sign weights: the inference form of a
 * layer whose weights alone are binarised (binary_nn README, "Binary
 * Regression" and "Triton Kernel Benchmark": the eval-only packed-sign path
 * of BinaryLinear, whose outputs differ from the dense product by rounding
 * only).
 *
 *   s[m][n] = sum over k < K of x[m][k] * w_n[k],   w_n[k] in {+1, -1}
 *
 * with w_n[k] read from the packed row ([BME 1] encoding; pad bits never
 * read), x given as bf16 bit patterns (row stride ldx elements) widened
 * exactly, and the sum taken in k order in double.  For the inputs the tests
 * use the double sum is exact; in general its error is below K * 2^-53 *
 * sum |x|, far below fp32 rounding.  Rows are split over threads. */

typedef struct {
  const uint16_t *x;
  int64_t ldx;
  const int8_t *wu;
  double *s;
  int64_t m_begin, m_end, N, K;
} signw_job_t;

static void *signw_rows(void *arg) {
  const signw_job_t *j = (const signw_job_t *)arg;
  for (int64_t m = j->m_begin; m < j->m_end; ++m) {
    for (int64_t n = 0; n < j->N; ++n) {
      const int8_t *w = j->wu + n * j->K;
      double acc = 0.0;
      for (int64_t k = 0; k < j->K; ++k)
        acc += (double)oracle_bf16_to_f32(j->x[m * j->ldx + k]) * (double)w[k];
      j->s[m * j->N + n] = acc;
    }
  }
  return NULL;
}

void oracle_dot_signw_bf16(const uint16_t *x, int64_t ldx, const uint64_t *wp, int64_t M,
                           int64_t N, int64_t K, double *s, int nthreads) {
  if (M <= 0 || N <= 0) return;
  int64_t kk = K > 0 ? K : 0;
  int8_t *wu = (int8_t *)malloc((size_t)(N * kk > 0 ? N * kk : 1));
  oracle_unpack(wp, N, kk, wu);
  int nt = resolve_threads(nthreads, M);
  pthread_t th[256];
  signw_job_t jobs[256];
  for (int t = 0; t < nt; ++t) {
    jobs[t].x = x;
    jobs[t].ldx = ldx;
    jobs[t].wu = wu;
    jobs[t].s = s;
    jobs[t].m_begin = M * t / nt;
    jobs[t].m_end = M * (t + 1) / nt;
    jobs[t].N = N;
    jobs[t].K = kk;
  }
  for (int t = 1; t < nt; ++t) pthread_create(&th[t], NULL, signw_rows, &jobs[t]);
  signw_rows(&jobs[0]);
  for (int t = 1; t < nt; ++t) pthread_join(th[t], NULL);
  free(wu);
}
