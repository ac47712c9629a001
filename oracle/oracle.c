/*
 * oracle.c -- plain, slow, obviously correct CPU reference for C = A*B.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke entry point and
 * the benchmark's cpu_baseline leg may load this library. The GPU product
 * path never calls it, links it, or shares code with it.
 *
 * What it computes (persistent-kernel forum thread, question: the GEMM a
 * persistent kernel tiles; tile scheduling only changes which worker
 * computes which output tile, never the value -- KernelWiki "Persistent
 * Kernels with Cluster Launch Control", "Choosing between static and CLC
 * scheduling": neither scheduler adds work):
 *
 *     C[i][j] = sum_{k=0}^{K-1} dec(A[i][k]) * dec(B[k][j])
 *
 * evaluated in IEEE double, k ascending, for every (i, j). A is M x K
 * row-major, B is K x N row-major, C is M x N row-major (the pages fix no
 * layout; this is the plain reading of "C = A*B" on row-major arrays).
 * dec() decodes the stored bit patterns exactly, written here from the
 * format definitions: IEEE 754 binary16, bfloat16 (the top half of IEEE
 * binary32) and OCP 8-bit E4M3 ("fn": no infinities, one NaN mantissa).
 *
 * Rows are split over host threads; each row's sums are still taken in
 * k order, so threading does not change a single bit of the result.
 *
 * Parity status: every function here is pinned by the CPU test suite
 * (exhaustive decoder tables against torch's casts, encoders against
 * numpy/torch casts, exact rational GEMM on tiny shapes, closed forms).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 0, ORACLE_BF16 = 1, ORACLE_E4M3FN = 2 };

/* ---- decoders: bit pattern -> exact double ------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_decode_f16(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 0x1f, m = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24); /* subnormal: m * 2^(1-15-10) */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/2^10) * 2^(e-15) */
  return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double oracle_decode_bf16(uint16_t h) {
  int s = h >> 15, e = (h >> 7) & 0xff, m = h & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)m, -133); /* m * 2^(1-127-7) */
  else if (e == 255)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(128 + m), e - 134); /* (1 + m/2^7) * 2^(e-127) */
  return s ? -v : v;
}

/* OCP E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent
 * 15 is an ordinary binade except S.1111.111, which is NaN; no infinity. */
double oracle_decode_e4m3fn(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 0xf, m = b & 7;
  double v;
  if (e == 15 && m == 7)
    v = NAN;
  else if (e == 0)
    v = ldexp((double)m, -9); /* m * 2^(1-7-3) */
  else
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  return s ? -v : v;
}

static double decode_one(const void* bits, int64_t idx, int dtype) {
  switch (dtype) {
    case ORACLE_F16: return oracle_decode_f16(((const uint16_t*)bits)[idx]);
    case ORACLE_BF16: return oracle_decode_bf16(((const uint16_t*)bits)[idx]);
    default: return oracle_decode_e4m3fn(((const uint8_t*)bits)[idx]);
  }
}

int oracle_decode_array(const void* bits, int64_t n, int dtype, double* out) {
  if (dtype < 0 || dtype > 2 || n < 0) return 1;
  for (int64_t i = 0; i < n; ++i) out[i] = decode_one(bits, i, dtype);
  return 0;
}

/* ---- encoders: double -> nearest representable, ties to even ------------ */

/* Round a non-negative double y (already an exact scaling of the input by a
 * power of two, y < 2^52) to the nearest integer, ties to even. */
static double round_half_even(double y) {
  double r = floor(y), f = y - r;
  if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  return r;
}

/* Generic IEEE-style binary format with `eb` exponent bits, `mb` fraction
 * bits, bias 2^(eb-1)-1, subnormals and infinities; round to nearest even. */
static uint32_t encode_ieee(double x, int eb, int mb) {
  const int bias = (1 << (eb - 1)) - 1, emax_field = (1 << eb) - 1;
  const uint32_t sign = signbit(x) ? (1u << (eb + mb)) : 0u;
  if (isnan(x)) return (uint32_t)emax_field << mb | (1u << (mb - 1)); /* quiet NaN */
  double a = fabs(x);
  if (isinf(a)) return sign | (uint32_t)emax_field << mb;
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E);            /* a = f * 2^E, f in [0.5, 1): unbiased exponent E-1 */
  int e = E - 1;
  if (e < 1 - bias) e = 1 - bias; /* subnormal binade shares the minimum exponent */
  double q = round_half_even(ldexp(a, mb - e)); /* significand in units of 2^(e-mb) */
  if (q >= ldexp(1.0, mb + 1)) { q = ldexp(q, -1); e += 1; } /* rounding carried out of the binade */
  int field;
  uint32_t frac;
  if (q < ldexp(1.0, mb)) { /* subnormal (only possible at the minimum exponent) */
    field = 0;
    frac = (uint32_t)q;
  } else {
    field = e + bias;
    frac = (uint32_t)(q - ldexp(1.0, mb));
  }
  if (field >= emax_field) return sign | (uint32_t)emax_field << mb; /* overflow -> inf */
  return sign | (uint32_t)field << mb | frac;
}

uint16_t oracle_encode_f16_rne(double x) { return (uint16_t)encode_ieee(x, 5, 10); }
uint16_t oracle_encode_bf16_rne(double x) { return (uint16_t)encode_ieee(x, 8, 7); }

/* out_dtype: ORACLE_F16 or ORACLE_BF16 */
int oracle_round_array(const double* x, int64_t n, int out_dtype, uint16_t* out) {
  if (out_dtype != ORACLE_F16 && out_dtype != ORACLE_BF16) return 1;
  for (int64_t i = 0; i < n; ++i)
    out[i] = out_dtype == ORACLE_F16 ? oracle_encode_f16_rne(x[i]) : oracle_encode_bf16_rne(x[i]);
  return 0;
}

/* ---- the GEMM ----------------------------------------------------------- */

typedef struct {
  const void* A;
  const double* Bd; /* B decoded, K x N row-major */
  int64_t N, K;
  int dtype;
  const int64_t* rows; /* which rows of A/C to compute */
  int64_t r0, r1;      /* this worker's slice of `rows` */
  double* C;           /* output: one row of N per entry of `rows` */
} gemm_job;

static void* gemm_worker(void* p) {
  gemm_job* j = (gemm_job*)p;
  for (int64_t r = j->r0; r < j->r1; ++r) {
    int64_t i = j->rows[r];
    double* c = j->C + r * j->N;
    for (int64_t n = 0; n < j->N; ++n) c[n] = 0.0;
    for (int64_t k = 0; k < j->K; ++k) {
      double a = decode_one(j->A, i * j->K + k, j->dtype);
      const double* b = j->Bd + k * j->N;
      for (int64_t n = 0; n < j->N; ++n) c[n] += a * b[n];
    }
  }
  return NULL;
}

/* C[r][:] = row rows[r] of A*B, for r in [0, nrows). Returns 0 on success. */
int oracle_gemm_rows(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype,
                     const int64_t* rows, int64_t nrows, double* C, int nthreads) {
  if (M < 0 || N < 0 || K < 0 || nrows < 0 || dtype < 0 || dtype > 2) return 1;
  for (int64_t r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= M) return 1;
  if (nrows == 0 || N == 0) return 0;
  double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
  if (!Bd) return 2;
  oracle_decode_array(B, K * N, dtype, Bd);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nrows) nthreads = (int)nrows;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
  gemm_job* jobs = (gemm_job*)malloc(sizeof(gemm_job) * nthreads);
  char* spawned = (char*)calloc((size_t)nthreads, 1);
  int rc = (th && jobs && spawned) ? 0 : 2;
  for (int t = 0; rc == 0 && t < nthreads; ++t) {
    gemm_job j = {A, Bd, N, K, dtype, rows, nrows * t / nthreads, nrows * (t + 1) / nthreads, C};
    jobs[t] = j;
    if (pthread_create(&th[t], NULL, gemm_worker, &jobs[t]) == 0)
      spawned[t] = 1;
    else
      gemm_worker(&jobs[t]); /* could not spawn a thread: do this slice inline */
  }
  for (int t = 0; rc == 0 && t < nthreads; ++t)
    if (spawned[t]) pthread_join(th[t], NULL);
  free(spawned);
  free(th);
  free(jobs);
  free(Bd);
  return rc;
}

/* Full product: C (M x N) = A (M x K) * B (K x N). */
int oracle_gemm(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype, double* C,
                int nthreads) {
  if (M < 0) return 1;
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)(M > 0 ? M : 1));
  if (!rows) return 2;
  for (int64_t i = 0; i < M; ++i) rows[i] = i;
  int rc = oracle_gemm_rows(A, B, M, N, K, dtype, rows, M, C, nthreads);
  free(rows);
  return rc;
}

/* ---- the parity measure ------------------------------------------------- */

/* Normwise relative error ||C - C_ref||_F / ||C_ref||_F of n output bit
 * patterns (out_dtype F16 or BF16) against the double reference. If the
 * reference is all zero, returns 0 when every output is +-0 and +inf
 * otherwise. NaN outputs give NaN. */
double oracle_normwise_error(const uint16_t* c_bits, int out_dtype, const double* ref, int64_t n) {
  double num = 0.0, den = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    double c = out_dtype == ORACLE_F16 ? oracle_decode_f16(c_bits[i]) : oracle_decode_bf16(c_bits[i]);
    double d = c - ref[i];
    num += d * d;
    den += ref[i] * ref[i];
  }
  if (den == 0.0) return num == 0.0 ? 0.0 : INFINITY;
  return sqrt(num) / sqrt(den);
}
