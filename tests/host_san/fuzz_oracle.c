/* Randomized round trips through the oracle's C functions, for a build of
 * oracle/qg_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Buffers have exactly the sizes the oracle documents, so an access past
 * them is a sanitizer error.  Checks along the way: every binary16 survives
 * f16 -> f64 -> f16; quantize -> pack -> unpack returns the same codes,
 * scales and zero points; dequant rows equal (u - offset) * s; the sweep of a
 * one-hot X returns the dequantized column, and a column subset returns the
 * same values as the full sweep.
 * Usage: fuzz_oracle SEED ITERATIONS.  Prints "ok <cases>" and exits 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_f64_to_f16(double x);
double oracle_f16_to_f64(uint16_t h);
int64_t oracle_packed_bytes(int fmt, int64_t N, int64_t K);
int oracle_quantize(const float* W, int64_t ldw, int64_t N, int64_t K, int fmt, int8_t* codes,
                    uint16_t* scales, uint8_t* zeros);
int oracle_pack(const int8_t* codes, const uint16_t* scales, const uint8_t* zeros, int64_t N, int64_t K,
                int fmt, uint8_t* packed);
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int fmt, int8_t* codes, uint16_t* scales,
                  uint8_t* zeros);
int oracle_dequant(const uint8_t* packed, int64_t N, int64_t K, int fmt, int64_t row0, int64_t nrows,
                   double* out);
int oracle_sweep_f64(const uint8_t* packed, int64_t N, int64_t K, int fmt, const uint16_t* X, int64_t ldx,
                     int M, double* Y, int64_t ldy, const int64_t* cols, int64_t ncols, int nthreads);

static long g_iter;
#define EXPECT(c)                                                                          \
  do {                                                                                     \
    if (!(c)) {                                                                            \
      fprintf(stderr, "fuzz check failed: %s (line %d, iteration %ld)\n", #c, __LINE__, g_iter); \
      exit(4);                                                                             \
    }                                                                                      \
  } while (0)

static uint64_t g_s;
static uint64_t next(void) { /* splitmix64 */
  uint64_t z = (g_s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static int64_t rnd(int64_t lo, int64_t hi) { return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1)); }
static double unif(void) { return (double)(next() >> 11) * 0x1p-53; }

static const int kFmts[4] = {4, 5, 0x104, 0x204};

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) abort();
  return p;
}

static void one_case(void) {
  const int fmt = kFmts[rnd(0, 3)];
  const int gs = fmt == 0x104 ? 64 : 32;
  const int zp = fmt == 0x204;
  const int64_t N = rnd(1, 70), K = gs * rnd(1, 10), ldw = K + rnd(0, 3), G = K / gs;
  float* W = xmalloc((size_t)((N - 1) * ldw + K) * sizeof(float));
  /* weights over several magnitudes, whole zero groups, one-sided groups */
  const double mag = pow(2.0, (double)rnd(-20, 4));
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      double v = (unif() * 2 - 1) * mag;
      if (rnd(0, 9) == 0) v = 0;
      if (zp && (k / 32) % 3 == 1) v = fabs(v);
      W[n * ldw + k] = (float)v;
    }
  if (rnd(0, 3) == 0)
    for (int64_t k = 0; k < gs; k++) W[k] = 0.0f; /* row 0, group 0 all zero */
  int8_t* codes = xmalloc((size_t)(N * K));
  uint16_t* scales = xmalloc((size_t)(N * G) * 2);
  uint8_t* zeros = zp ? xmalloc((size_t)(N * G)) : NULL;
  EXPECT(oracle_quantize(W, ldw, N, K, fmt, codes, scales, zeros) == 0);
  const int64_t pb = oracle_packed_bytes(fmt, N, K);
  EXPECT(pb > 0 && oracle_packed_bytes(fmt, N, K + 16) == 0);
  uint8_t* packed = xmalloc((size_t)pb);
  EXPECT(oracle_pack(codes, scales, zeros, N, K, fmt, packed) == 0);
  int8_t* c2 = xmalloc((size_t)(N * K));
  uint16_t* s2 = xmalloc((size_t)(N * G) * 2);
  uint8_t* z2 = zp ? xmalloc((size_t)(N * G)) : NULL;
  EXPECT(oracle_unpack(packed, N, K, fmt, c2, s2, z2) == 0);
  EXPECT(memcmp(codes, c2, (size_t)(N * K)) == 0);
  EXPECT(memcmp(scales, s2, (size_t)(N * G) * 2) == 0);
  if (zp) EXPECT(memcmp(zeros, z2, (size_t)(N * G)) == 0);
  /* dequant of a row range */
  const int64_t r0 = rnd(0, N - 1), nr = rnd(1, N - r0);
  double* wh = xmalloc((size_t)(nr * K) * sizeof(double));
  EXPECT(oracle_dequant(packed, N, K, fmt, r0, nr, wh) == 0);
  for (int64_t t = 0; t < nr; t++)
    for (int64_t k = 0; k < K; k++) {
      const int64_t n = r0 + t, g = k / gs;
      const double s = oracle_f16_to_f64(scales[n * G + g]);
      const double q = zp ? (double)codes[n * K + k] - zeros[n * G + g] : (double)codes[n * K + k];
      EXPECT(wh[t * K + k] == q * s);
    }
  EXPECT(oracle_dequant(packed, N, K, fmt, r0, N - r0 + 1, wh) != 0);
  /* one-hot X rows: row m selects k = km[m]; Y[m, n] must be w_hat[n, km[m]] */
  const int M = (int)rnd(1, 5);
  const int64_t ldx = K + rnd(0, 2);
  uint16_t* X = xmalloc((size_t)((M - 1) * ldx + K) * 2);
  memset(X, 0, (size_t)((M - 1) * ldx + K) * 2);
  int64_t km[5];
  for (int m = 0; m < M; m++) {
    km[m] = rnd(0, K - 1);
    X[m * ldx + km[m]] = 0x3C00; /* 1.0 */
  }
  const int64_t ldy = N + rnd(0, 2);
  double* Y = xmalloc((size_t)((M - 1) * ldy + N) * sizeof(double));
  EXPECT(oracle_sweep_f64(packed, N, K, fmt, X, ldx, M, Y, ldy, NULL, 0, (int)rnd(1, 4)) == 0);
  double* all = xmalloc((size_t)(N * K) * sizeof(double));
  EXPECT(oracle_dequant(packed, N, K, fmt, 0, N, all) == 0);
  for (int m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) EXPECT(Y[m * ldy + n] == all[n * K + km[m]]);
  /* random X: a column subset equals the same columns of the full sweep */
  for (int m = 0; m < M; m++)
    for (int64_t k = 0; k < K; k++) X[m * ldx + k] = oracle_f64_to_f16(unif() * 4 - 2);
  EXPECT(oracle_sweep_f64(packed, N, K, fmt, X, ldx, M, Y, ldy, NULL, 0, (int)rnd(1, 4)) == 0);
  const int64_t nc = rnd(1, N);
  int64_t* cols = xmalloc((size_t)nc * sizeof(int64_t));
  for (int64_t i = 0; i < nc; i++) cols[i] = rnd(0, N - 1);
  const int64_t ldy2 = nc + rnd(0, 2);
  double* Ys = xmalloc((size_t)((M - 1) * ldy2 + nc) * sizeof(double));
  EXPECT(oracle_sweep_f64(packed, N, K, fmt, X, ldx, M, Ys, ldy2, cols, nc, (int)rnd(1, 4)) == 0);
  for (int m = 0; m < M; m++)
    for (int64_t i = 0; i < nc; i++) EXPECT(Ys[m * ldy2 + i] == Y[m * ldy + cols[i]]);
  cols[0] = N;
  EXPECT(oracle_sweep_f64(packed, N, K, fmt, X, ldx, M, Ys, ldy2, cols, nc, 1) != 0);
  free(W), free(codes), free(scales), free(zeros), free(packed), free(c2), free(s2), free(z2);
  free(wh), free(X), free(Y), free(all), free(cols), free(Ys);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: fuzz_oracle SEED ITERATIONS\n");
    return 2;
  }
  g_s = strtoull(argv[1], NULL, 10);
  const long iters = strtol(argv[2], NULL, 10);
  for (uint32_t h = 0; h < 65536; h++) {
    const double v = oracle_f16_to_f64((uint16_t)h);
    if (!isnan(v)) EXPECT(oracle_f64_to_f16(v) == h);
  }
  for (g_iter = 0; g_iter < iters; g_iter++) one_case();
  printf("ok %ld\n", iters);
  return 0;
}
