/* Sanitizer driver for the CPU oracle (test infrastructure).
 *
 * Built with gcc -fsanitize=address,undefined -fno-sanitize-recover=all
 * together with oracle/oracle.c and run as a plain executable (no Python in
 * the process), it exercises every entry point of the oracle -- every
 * decoder pattern, the encoders across the whole double range, full and
 * row-sampled GEMMs on odd shapes with several thread counts, the
 * normwise error -- so that an out-of-bounds access, a use of
 * uninitialised memory through the threads, or undefined behaviour
 * (shifts, overflow) aborts the run. It prints "ok" and exits 0 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_decode_f16(uint16_t h);
double oracle_decode_bf16(uint16_t h);
double oracle_decode_e4m3fn(uint8_t b);
int oracle_decode_array(const void* bits, int64_t n, int dtype, double* out);
uint16_t oracle_encode_f16_rne(double x);
uint16_t oracle_encode_bf16_rne(double x);
int oracle_round_array(const double* x, int64_t n, int out_dtype, uint16_t* out);
int oracle_gemm_rows(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype, const int64_t* rows,
                     int64_t nrows, double* C, int nthreads);
int oracle_gemm(const void* A, const void* B, int64_t M, int64_t N, int64_t K, int dtype, double* C, int nthreads);
double oracle_normwise_error(const uint16_t* c_bits, int out_dtype, const double* ref, int64_t n);

static uint32_t rng = 12345u;
static uint32_t next(void) {
  rng = rng * 1664525u + 1013904223u;
  return rng >> 8;
}

static int check_gemm(int dtype, int64_t M, int64_t N, int64_t K, int threads) {
  const int es = dtype == 2 ? 1 : 2;
  uint8_t* A = malloc((size_t)(M * K * es) + 1);
  uint8_t* B = malloc((size_t)(K * N * es) + 1);
  double* C = malloc(sizeof(double) * (size_t)(M * N) + 8);
  double* R = malloc(sizeof(double) * (size_t)(N) * 3 + 8);
  uint16_t* bits = malloc(sizeof(uint16_t) * (size_t)(M * N) + 2);
  if (!A || !B || !C || !R || !bits) return 1;
  /* finite small values: fp16 0x3C00-ish patterns, bf16 0x3F80-ish, e4m3 0x30-ish */
  for (int64_t i = 0; i < M * K; ++i) {
    if (es == 2) ((uint16_t*)A)[i] = (uint16_t)((dtype == 0 ? 0x3800 : 0x3F00) + (next() & 0x3FF) - 0x200);
    else A[i] = (uint8_t)(0x28 + (next() & 0x1F));
  }
  for (int64_t i = 0; i < K * N; ++i) {
    if (es == 2) ((uint16_t*)B)[i] = (uint16_t)((dtype == 0 ? 0xB800 : 0xBF00) + (next() & 0x3FF) - 0x200);
    else B[i] = (uint8_t)(0xA8 + (next() & 0x1F));
  }
  if (oracle_gemm(A, B, M, N, K, dtype, C, threads)) return 2;
  if (M > 0 && N > 0) {
    int64_t rows[3] = {M - 1, 0, M / 2};
    if (oracle_gemm_rows(A, B, M, N, K, dtype, rows, 3, R, threads)) return 3;
    for (int r = 0; r < 3; ++r)
      for (int64_t j = 0; j < N; ++j)
        if (R[r * N + j] != C[rows[r] * N + j]) return 4;
  }
  if (oracle_round_array(C, M * N, dtype == 0 ? 0 : 1, bits)) return 5;
  (void)oracle_normwise_error(bits, dtype == 0 ? 0 : 1, C, M * N);
  free(A);
  free(B);
  free(C);
  free(R);
  free(bits);
  return 0;
}

int main(void) {
  /* every decoder pattern */
  double sink = 0.0;
  for (uint32_t h = 0; h < 65536; ++h) {
    const double a = oracle_decode_f16((uint16_t)h), b = oracle_decode_bf16((uint16_t)h);
    if (isfinite(a)) sink += a * 0.0;
    if (isfinite(b)) sink += b * 0.0;
  }
  for (uint32_t h = 0; h < 256; ++h) {
    const double c = oracle_decode_e4m3fn((uint8_t)h);
    if (isfinite(c)) sink += c * 0.0;
  }
  /* encoders across the double range, including infinities, NaN, subnormals and ties */
  const double specials[] = {0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 1e300, -1e300, 1e-300, 5.96e-8, 2.98e-8,
                             INFINITY, -INFINITY, NAN, 3.0e38, 3.4e38, 1.0e-45, 0.1, 1.0 / 3.0};
  for (size_t i = 0; i < sizeof(specials) / sizeof(specials[0]); ++i) {
    sink += (double)oracle_encode_f16_rne(specials[i]) * 0.0;
    sink += (double)oracle_encode_bf16_rne(specials[i]) * 0.0;
  }
  for (int i = 0; i < 200000; ++i) {
    const double x = ldexp((double)(int32_t)(next() << 8) / 2147483648.0, (int)(next() % 600) - 300);
    sink += (double)oracle_encode_f16_rne(x) * 0.0 + (double)oracle_encode_bf16_rne(x) * 0.0;
  }
  /* decode_array / round_array on every dtype */
  uint16_t pat[512];
  double val[512];
  for (int i = 0; i < 512; ++i) pat[i] = (uint16_t)next();
  for (int dt = 0; dt < 3; ++dt)
    if (oracle_decode_array(pat, 512, dt, val)) return 10;
  /* GEMMs: odd shapes, empty sizes, several thread counts */
  const int64_t shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {17, 9, 33}, {64, 1, 130}, {1, 70, 3}, {0, 4, 5}, {4, 0, 5}, {4, 6, 0}};
  for (int dt = 0; dt < 3; ++dt)
    for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
      for (int th = 1; th <= 9; th += 4) {
        const int rc = check_gemm(dt, shapes[s][0], shapes[s][1], shapes[s][2], th);
        if (rc) {
          fprintf(stderr, "gemm check %d failed (dtype %d shape %zu threads %d)\n", rc, dt, s, th);
          return 20 + rc;
        }
      }
  printf("ok %g\n", sink);
  return 0;
}
