/*
 * CPU ORACLE for the fused quantized weight sweep -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no source with the GPU library and is written
 * to be read against its definition, not to be fast:
 *
 *   Quantizer (Quasar/q27 wiki, engine-internals list, "Weights" item: 4-bit
 *   symmetric groupwise weights with fp16 scales, dequantized inside the GEMV;
 *   group size 32 and the 5-bit variant per the sweep's specification):
 *     per row n and group g of 32 consecutive k:
 *       amax = max |W[n,k]|                       (fp32, exact)
 *       s    = fp16_RNE((double)amax / Qmax)      Qmax = 7 (4-bit), 15 (5-bit)
 *       q    = 0 if s == 0, else clamp(RNE((double)W / (double)s), -Qmax, Qmax)
 *       u    = q + 2^(bits-1)                     (stored offset-binary code)
 *   Dequant:  w_hat = (double)q * (double)s       (exact in fp64)
 *   Sweep:    Y[m,n] = sum_{k ascending} (double)X[m,k] * w_hat[n,k]   (fp64)
 *
 * Tiled group-32 layout ("QG32 tiled v1", our own: the pages do not publish q4s/q5f):
 *   16 rows x 128 k per tile; tile (rb, kt) at byte (rb*NKT + kt)*TB with
 *   NKT = ceil(K/128), TB = 1152 (4-bit) or 1408 (5-bit).  For element (n, k):
 *   r = n mod 16, j = (k mod 128)/32, c = (k mod 32)/8, e = k mod 8.
 *     low 4 bits of u : LE word at byte 16*(r+16c) + 4j, bit 4*(e>>1) + 16*(e&1)
 *     bit 4 of u      : LE word at byte 1152 + 4*(r+16c),
 *                       bit (4 + 16*(e&1) + 4*(e>>1) + j) mod 32   (5-bit only)
 *     scale s(n, 4kt+j): binary16 at byte 1024 + 8r + 2j
 *   Rows n >= N and groups g >= K/32 are padding: u = 2^(bits-1), s = +0.
 *
 * Non-finite inputs (NaN/Inf in W) or a scale that rounds to fp16 infinity
 * make the quantizer return 3 (the codes are then unspecified).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- IEEE binary16 <-> binary64, written from the format ---------- */

/* binary64 -> binary16, round to nearest, ties to even. */
uint16_t oracle_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000u : 0u;
  if (isnan(x)) return (uint16_t)(sign | 0x7e00u);
  double a = fabs(x);
  if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
  if (a == 0.0) return sign;
  int E;
  frexp(a, &E);          /* a = f * 2^E, f in [0.5, 1) */
  int e = E - 1;         /* a in [2^e, 2^(e+1)) */
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  int ulp_exp = (e < -14) ? -24 : e - 10;
  double r = nearbyint(ldexp(a, -ulp_exp)); /* exact scaling, then RNE */
  if (e < -14) {
    /* subnormal range: value = r * 2^-24, r <= 1024 (1024 = smallest normal) */
    return (uint16_t)(sign | (uint16_t)r);
  }
  long ri = (long)r;     /* in [1024, 2048] */
  if (ri == 2048) {
    ri = 1024;
    e += 1;
  }
  if (e > 15) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)(((e + 15) << 10) | (ri - 1024)));
}

double oracle_f16_to_f64(uint16_t h) {
  int ex = (h >> 10) & 0x1f;
  int man = h & 0x3ff;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + man), ex - 25);
  return (h & 0x8000u) ? -v : v;
}

/* ----------------------------- layout helpers ---------------------------- */

static int64_t nkt_of(int64_t K) { return (K + 127) / 128; }
static int64_t nrb_of(int64_t N) { return (N + 15) / 16; }
static int64_t tile_bytes(int bits) { return bits == 4 ? 1152 : 1408; }

int64_t oracle_packed_bytes(int bits, int64_t N, int64_t K) {
  if ((bits != 4 && bits != 5) || N <= 0 || K <= 0 || K % 32) return 0;
  return nrb_of(N) * nkt_of(K) * tile_bytes(bits);
}

static uint32_t rd32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}
static void wr32(uint8_t* p, uint32_t v) {
  p[0] = (uint8_t)v;
  p[1] = (uint8_t)(v >> 8);
  p[2] = (uint8_t)(v >> 16);
  p[3] = (uint8_t)(v >> 24);
}

typedef struct {
  int64_t code_word;  /* byte offset of the word holding the low nibble */
  int code_bit;
  int64_t hi_word;    /* byte offset of the word holding bit 4 */
  int hi_bit;
  int64_t scale;      /* byte offset of the group's fp16 scale */
} loc_t;

static loc_t locate(int64_t n, int64_t k, int64_t NKT, int bits) {
  loc_t L;
  int64_t rb = n / 16, kt = k / 128;
  int r = (int)(n % 16), j = (int)((k % 128) / 32), c = (int)((k % 32) / 8), e = (int)(k % 8);
  int64_t base = (rb * NKT + kt) * tile_bytes(bits);
  L.code_word = base + 16 * (r + 16 * c) + 4 * j;
  L.code_bit = 4 * (e >> 1) + 16 * (e & 1);
  L.hi_word = base + 1152 + 4 * (r + 16 * c);
  L.hi_bit = (4 + 16 * (e & 1) + 4 * (e >> 1) + j) % 32;
  L.scale = base + 1024 + 8 * r + 2 * j;
  return L;
}

/* ------------------------------- quantizer ------------------------------- */

/*
 * codes[n*K + k] = q (int8), scales[n*(K/32) + g] = binary16 bits of s.
 * Returns 0, or 3 for non-finite input / scale overflow.
 */
int oracle_quantize(const float* W, int64_t ldw, int64_t N, int64_t K, int bits,
                    int8_t* codes, uint16_t* scales) {
  const int qmax = (1 << (bits - 1)) - 1;
  const int64_t G = K / 32;
  int status = 0;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const float* w = W + n * ldw + 32 * g;
      float amax = 0.0f;
      for (int t = 0; t < 32; t++) {
        if (!isfinite(w[t])) status = 3;
        float a = fabsf(w[t]);
        if (a > amax) amax = a;
      }
      uint16_t sb = oracle_f64_to_f16((double)amax / (double)qmax);
      if ((sb & 0x7c00u) == 0x7c00u) status = 3;
      scales[n * G + g] = sb;
      double s = oracle_f16_to_f64(sb);
      for (int t = 0; t < 32; t++) {
        int q = 0;
        if (s != 0.0 && isfinite(w[t]) && isfinite(s)) {
          double v = nearbyint((double)w[t] / s);
          if (v > qmax) v = qmax;
          if (v < -qmax) v = -qmax;
          q = (int)v;
        }
        codes[n * K + 32 * g + t] = (int8_t)q;
      }
    }
  }
  return status;
}

/* --------------------------------- pack ---------------------------------- */

/* Writes every byte of the padded tile grid (padding included). */
int oracle_pack(const int8_t* codes, const uint16_t* scales, int64_t N, int64_t K, int bits,
                uint8_t* packed) {
  const int64_t NKT = nkt_of(K), NRB = nrb_of(N), G = K / 32;
  const int bias = 1 << (bits - 1);
  memset(packed, 0, (size_t)(NRB * NKT * tile_bytes(bits)));
  for (int64_t n = 0; n < NRB * 16; n++) {
    for (int64_t k = 0; k < NKT * 128; k++) {
      int valid = (n < N) && (k < K);
      int u = valid ? codes[n * K + k] + bias : bias;
      loc_t L = locate(n, k, NKT, bits);
      uint32_t w = rd32(packed + L.code_word);
      w |= (uint32_t)(u & 15) << L.code_bit;
      wr32(packed + L.code_word, w);
      if (bits == 5) {
        uint32_t h = rd32(packed + L.hi_word);
        h |= (uint32_t)((u >> 4) & 1) << L.hi_bit;
        wr32(packed + L.hi_word, h);
      }
      if (k % 32 == 0) {
        uint16_t sb = valid ? scales[n * G + k / 32] : 0;
        packed[L.scale] = (uint8_t)sb;
        packed[L.scale + 1] = (uint8_t)(sb >> 8);
      }
    }
  }
  return 0;
}

/* ------------------------------ scalar decode ---------------------------- */

static int decode_u(const uint8_t* packed, int64_t n, int64_t k, int64_t NKT, int bits) {
  loc_t L = locate(n, k, NKT, bits);
  int u = (int)((rd32(packed + L.code_word) >> L.code_bit) & 15u);
  if (bits == 5) u |= (int)(((rd32(packed + L.hi_word) >> L.hi_bit) & 1u) << 4);
  return u;
}

static uint16_t decode_scale(const uint8_t* packed, int64_t n, int64_t g, int64_t NKT, int bits) {
  loc_t L = locate(n, 32 * g, NKT, bits);
  return (uint16_t)(packed[L.scale] | (packed[L.scale + 1] << 8));
}

/* Reads q and s back from the bytes, bit by bit. */
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int bits, int8_t* codes,
                  uint16_t* scales) {
  const int64_t NKT = nkt_of(K), G = K / 32;
  const int bias = 1 << (bits - 1);
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++)
      codes[n * K + k] = (int8_t)(decode_u(packed, n, k, NKT, bits) - bias);
    for (int64_t g = 0; g < G; g++) scales[n * G + g] = decode_scale(packed, n, g, NKT, bits);
  }
  return 0;
}

/* w_hat rows [row0, row0+nrows) as fp64 (exact q * s), decoded from bytes. */
int oracle_dequant(const uint8_t* packed, int64_t N, int64_t K, int bits, int64_t row0,
                   int64_t nrows, double* out) {
  const int64_t NKT = nkt_of(K);
  const int bias = 1 << (bits - 1);
  if (row0 < 0 || row0 + nrows > N) return 1;
  for (int64_t t = 0; t < nrows; t++) {
    int64_t n = row0 + t;
    for (int64_t k = 0; k < K; k++) {
      double s = oracle_f16_to_f64(decode_scale(packed, n, k / 32, NKT, bits));
      out[t * K + k] = (double)(decode_u(packed, n, k, NKT, bits) - bias) * s;
    }
  }
  return 0;
}

/* --------------------------------- sweep --------------------------------- */

typedef struct {
  const uint8_t* packed;
  int64_t N, K;
  int bits;
  const uint16_t* X;
  int64_t ldx;
  int M;
  double* Y;
  int64_t ldy;
  const int64_t* cols;
  int64_t ncols;
  int64_t c0, c1;
  int status;
} sweep_job_t;

static void* sweep_worker(void* arg) {
  sweep_job_t* J = (sweep_job_t*)arg;
  double* wrow = (double*)malloc(sizeof(double) * (size_t)J->K);
  double* xrow = (double*)malloc(sizeof(double) * (size_t)J->K);
  if (!wrow || !xrow) {
    J->status = 2;
    free(wrow);
    free(xrow);
    return NULL;
  }
  for (int64_t ci = J->c0; ci < J->c1; ci++) {
    int64_t n = J->cols ? J->cols[ci] : ci;
    oracle_dequant(J->packed, J->N, J->K, J->bits, n, 1, wrow);
    for (int m = 0; m < J->M; m++) {
      for (int64_t k = 0; k < J->K; k++) xrow[k] = oracle_f16_to_f64(J->X[m * J->ldx + k]);
      double acc = 0.0;
      for (int64_t k = 0; k < J->K; k++) acc += xrow[k] * wrow[k];
      /* Y column index: position in the requested column list */
      J->Y[(int64_t)m * J->ldy + ci] = acc;
    }
  }
  free(wrow);
  free(xrow);
  return NULL;
}

/*
 * Y[m*ldy + i] = sum_k X[m,k] * w_hat[cols[i], k] for i < ncols (all N
 * columns in order when cols == NULL, ncols = N).  X is binary16 bits.
 * Work is split over `nthreads` POSIX threads by columns.
 */
int oracle_sweep_f64(const uint8_t* packed, int64_t N, int64_t K, int bits, const uint16_t* X,
                     int64_t ldx, int M, double* Y, int64_t ldy, const int64_t* cols,
                     int64_t ncols, int nthreads) {
  if (!cols) ncols = N;
  for (int64_t i = 0; cols && i < ncols; i++)
    if (cols[i] < 0 || cols[i] >= N) return 1;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (ncols < nthreads) nthreads = ncols > 0 ? (int)ncols : 1;
  sweep_job_t jobs[256];
  pthread_t th[256];
  for (int t = 0; t < nthreads; t++) {
    sweep_job_t* J = &jobs[t];
    J->packed = packed;
    J->N = N;
    J->K = K;
    J->bits = bits;
    J->X = X;
    J->ldx = ldx;
    J->M = M;
    J->Y = Y;
    J->ldy = ldy;
    J->cols = cols;
    J->ncols = ncols;
    J->c0 = ncols * t / nthreads;
    J->c1 = ncols * (t + 1) / nthreads;
    J->status = 0;
  }
  int started = 0;
  for (int t = 1; t < nthreads; t++) {
    if (pthread_create(&th[t], NULL, sweep_worker, &jobs[t]) != 0) break;
    started = t;
  }
  sweep_worker(&jobs[0]);
  for (int t = 1; t <= started; t++) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; t++) sweep_worker(&jobs[t]);
  for (int t = 0; t < nthreads; t++)
    if (jobs[t].status) return jobs[t].status;
  return 0;
}

/* ------------------------- array conveniences ---------------------------- */

void oracle_f64_to_f16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f64_to_f16(x[i]);
}

void oracle_f16_to_f64_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; i++) out[i] = oracle_f16_to_f64(h[i]);
}
