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
 * Format variants (a format code in place of `bits`; the same tile grid and
 * code words, only the group size and the per-group parameters differ):
 *   0x104  4-bit symmetric, group 64 (the Quasar/q27 wiki's Q4_G64 accounting:
 *          half a byte per weight plus one fp16 scale per 64 weights).  Qmax 7,
 *          u = q + 8; tile 1088 bytes; the scale of row r and group h =
 *          (k mod 128)/64 is binary16 at byte 1024 + 4r + 2h.  K % 64 == 0.
 *   0x204  4-bit asymmetric, group 32, with an integer zero point per group
 *          (the INT4 W4A16 group-32 asymmetric weights of the qwen38 model
 *          notes, AWQ-INT4 path).  Per row n and group g:
 *            lo = min(0, min W), hi = max(0, max W)            (fp32, exact)
 *            s  = fp16_RNE(((double)hi - (double)lo) / 15)
 *            z  = 0 if s == 0, else clamp(RNE(-(double)lo / s), 0, 15)
 *            u  = z if s == 0, else clamp(RNE((double)W / s) + z, 0, 15)
 *          w_hat = (u - z) * s (zero is exact); u is stored as is (low 4 bits
 *          as above), s at 1024 + 8r + 2j, and z of group j of row r in bits
 *          4j .. 4j+3 of the little-endian 16-bit word at byte 1152 + 2r;
 *          tile 1184 bytes.  Padding: u = 0, z = 0, s = +0.
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

typedef struct {
  int cbits;   /* code bits: 4 or 5 */
  int gs;      /* weights per scale group: 32 or 64 */
  int zp;      /* 1: asymmetric with a zero point per group */
  int64_t tb;  /* bytes per 16 x 128 tile */
} fmt_t;

/* 0 for an unknown format code. */
static int fmt_of(int fmt, fmt_t* f) {
  switch (fmt) {
    case 4: *f = (fmt_t){4, 32, 0, 1152}; return 1;
    case 5: *f = (fmt_t){5, 32, 0, 1408}; return 1;
    case 0x104: *f = (fmt_t){4, 64, 0, 1088}; return 1;
    case 0x204: *f = (fmt_t){4, 32, 1, 1184}; return 1;
  }
  return 0;
}

static int64_t nkt_of(int64_t K) { return (K + 127) / 128; }
static int64_t nrb_of(int64_t N) { return (N + 15) / 16; }

int64_t oracle_packed_bytes(int fmt, int64_t N, int64_t K) {
  fmt_t f;
  if (!fmt_of(fmt, &f) || N <= 0 || K <= 0 || K % f.gs) return 0;
  return nrb_of(N) * nkt_of(K) * f.tb;
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
  int64_t hi_word;    /* byte offset of the word holding bit 4 (5-bit) */
  int hi_bit;
  int64_t scale;      /* byte offset of the group's fp16 scale */
  int64_t zero;       /* byte offset of the 16-bit word holding the zero point */
  int zero_bit;
} loc_t;

static loc_t locate(int64_t n, int64_t k, int64_t NKT, const fmt_t* f) {
  loc_t L;
  int64_t rb = n / 16, kt = k / 128;
  int r = (int)(n % 16), j = (int)((k % 128) / 32), c = (int)((k % 32) / 8), e = (int)(k % 8);
  int64_t base = (rb * NKT + kt) * f->tb;
  L.code_word = base + 16 * (r + 16 * c) + 4 * j;
  L.code_bit = 4 * (e >> 1) + 16 * (e & 1);
  L.hi_word = base + 1152 + 4 * (r + 16 * c);
  L.hi_bit = (4 + 16 * (e & 1) + 4 * (e >> 1) + j) % 32;
  if (f->gs == 64)
    L.scale = base + 1024 + 4 * r + 2 * (j / 2);
  else
    L.scale = base + 1024 + 8 * r + 2 * j;
  L.zero = base + 1152 + 2 * r;
  L.zero_bit = 4 * j;
  return L;
}

/* ------------------------------- quantizer ------------------------------- */

/*
 * scales[n*(K/gs) + g] = binary16 bits of s.  Symmetric formats:
 * codes[n*K + k] = q (int8, -Qmax..Qmax).  Zero-point format: codes = u
 * (0..15) and zeros[n*(K/32) + g] = z.  Returns 0, 1 for a bad format or K,
 * or 3 for non-finite input / scale overflow.
 */
int oracle_quantize(const float* W, int64_t ldw, int64_t N, int64_t K, int fmt,
                    int8_t* codes, uint16_t* scales, uint8_t* zeros) {
  fmt_t f;
  if (!fmt_of(fmt, &f) || K % f.gs || (f.zp && !zeros)) return 1;
  const int gs = f.gs;
  const int qmax = (1 << (f.cbits - 1)) - 1;
  const int64_t G = K / gs;
  int status = 0;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t g = 0; g < G; g++) {
      const float* w = W + n * ldw + gs * g;
      for (int t = 0; t < gs; t++)
        if (!isfinite(w[t])) status = 3;
      if (!f.zp) {
        float amax = 0.0f;
        for (int t = 0; t < gs; t++) {
          float a = fabsf(w[t]);
          if (a > amax) amax = a;
        }
        uint16_t sb = oracle_f64_to_f16((double)amax / (double)qmax);
        if ((sb & 0x7c00u) == 0x7c00u) status = 3;
        scales[n * G + g] = sb;
        double s = oracle_f16_to_f64(sb);
        for (int t = 0; t < gs; t++) {
          int q = 0;
          if (s != 0.0 && isfinite(w[t]) && isfinite(s)) {
            double v = nearbyint((double)w[t] / s);
            if (v > qmax) v = qmax;
            if (v < -qmax) v = -qmax;
            q = (int)v;
          }
          codes[n * K + gs * g + t] = (int8_t)q;
        }
      } else {
        float lo = 0.0f, hi = 0.0f;
        for (int t = 0; t < gs; t++) {
          if (w[t] < lo) lo = w[t];
          if (w[t] > hi) hi = w[t];
        }
        uint16_t sb = oracle_f64_to_f16(((double)hi - (double)lo) / 15.0);
        if ((sb & 0x7c00u) == 0x7c00u) status = 3;
        scales[n * G + g] = sb;
        double s = oracle_f16_to_f64(sb);
        int z = 0;
        int ok = s != 0.0 && isfinite(s);
        if (ok) {
          double zz = nearbyint(-(double)lo / s);
          if (zz < 0) zz = 0;
          if (zz > 15) zz = 15;
          z = (int)zz;
        }
        zeros[n * G + g] = (uint8_t)z;
        for (int t = 0; t < gs; t++) {
          int u = z;
          if (ok && isfinite(w[t])) {
            double v = nearbyint((double)w[t] / s) + z;
            if (v < 0) v = 0;
            if (v > 15) v = 15;
            u = (int)v;
          }
          codes[n * K + gs * g + t] = (int8_t)u;
        }
      }
    }
  }
  return status;
}

/* --------------------------------- pack ---------------------------------- */

/* Writes every byte of the padded tile grid (padding included). */
int oracle_pack(const int8_t* codes, const uint16_t* scales, const uint8_t* zeros, int64_t N,
                int64_t K, int fmt, uint8_t* packed) {
  fmt_t f;
  if (!fmt_of(fmt, &f) || K % f.gs || (f.zp && !zeros)) return 1;
  const int64_t NKT = nkt_of(K), NRB = nrb_of(N), G = K / f.gs;
  const int bias = f.zp ? 0 : 1 << (f.cbits - 1);
  memset(packed, 0, (size_t)(NRB * NKT * f.tb));
  for (int64_t n = 0; n < NRB * 16; n++) {
    for (int64_t k = 0; k < NKT * 128; k++) {
      int valid = (n < N) && (k < K);
      int u = valid ? codes[n * K + k] + bias : bias;
      loc_t L = locate(n, k, NKT, &f);
      uint32_t w = rd32(packed + L.code_word);
      w |= (uint32_t)(u & 15) << L.code_bit;
      wr32(packed + L.code_word, w);
      if (f.cbits == 5) {
        uint32_t h = rd32(packed + L.hi_word);
        h |= (uint32_t)((u >> 4) & 1) << L.hi_bit;
        wr32(packed + L.hi_word, h);
      }
      if (k % f.gs == 0) {
        uint16_t sb = valid ? scales[n * G + k / f.gs] : 0;
        packed[L.scale] = (uint8_t)sb;
        packed[L.scale + 1] = (uint8_t)(sb >> 8);
        if (f.zp) {
          int z = valid ? zeros[n * G + k / f.gs] & 15 : 0;
          uint32_t zw = (uint32_t)packed[L.zero] | ((uint32_t)packed[L.zero + 1] << 8);
          zw |= (uint32_t)z << L.zero_bit;
          packed[L.zero] = (uint8_t)zw;
          packed[L.zero + 1] = (uint8_t)(zw >> 8);
        }
      }
    }
  }
  return 0;
}

/* ------------------------------ scalar decode ---------------------------- */

static int decode_u(const uint8_t* packed, int64_t n, int64_t k, int64_t NKT, const fmt_t* f) {
  loc_t L = locate(n, k, NKT, f);
  int u = (int)((rd32(packed + L.code_word) >> L.code_bit) & 15u);
  if (f->cbits == 5) u |= (int)(((rd32(packed + L.hi_word) >> L.hi_bit) & 1u) << 4);
  return u;
}

static uint16_t decode_scale(const uint8_t* packed, int64_t n, int64_t k, int64_t NKT, const fmt_t* f) {
  loc_t L = locate(n, k, NKT, f);
  return (uint16_t)(packed[L.scale] | (packed[L.scale + 1] << 8));
}

/* The value subtracted from u: the bias 2^(bits-1), or the group's zero point. */
static int decode_offset(const uint8_t* packed, int64_t n, int64_t k, int64_t NKT, const fmt_t* f) {
  if (!f->zp) return 1 << (f->cbits - 1);
  loc_t L = locate(n, k, NKT, f);
  uint32_t zw = (uint32_t)packed[L.zero] | ((uint32_t)packed[L.zero + 1] << 8);
  return (int)((zw >> L.zero_bit) & 15u);
}

/* Reads the codes (q, or u for the zero-point format), scales and zero points
 * back from the bytes, bit by bit. */
int oracle_unpack(const uint8_t* packed, int64_t N, int64_t K, int fmt, int8_t* codes,
                  uint16_t* scales, uint8_t* zeros) {
  fmt_t f;
  if (!fmt_of(fmt, &f) || K % f.gs || (f.zp && !zeros)) return 1;
  const int64_t NKT = nkt_of(K), G = K / f.gs;
  for (int64_t n = 0; n < N; n++) {
    for (int64_t k = 0; k < K; k++) {
      int u = decode_u(packed, n, k, NKT, &f);
      codes[n * K + k] = (int8_t)(f.zp ? u : u - decode_offset(packed, n, k, NKT, &f));
    }
    for (int64_t g = 0; g < G; g++) {
      scales[n * G + g] = decode_scale(packed, n, g * f.gs, NKT, &f);
      if (f.zp) zeros[n * G + g] = (uint8_t)decode_offset(packed, n, g * f.gs, NKT, &f);
    }
  }
  return 0;
}

/* w_hat rows [row0, row0+nrows) as fp64 (exact (u - offset) * s), decoded
 * from bytes. */
int oracle_dequant(const uint8_t* packed, int64_t N, int64_t K, int fmt, int64_t row0,
                   int64_t nrows, double* out) {
  fmt_t f;
  if (!fmt_of(fmt, &f) || K % f.gs) return 1;
  const int64_t NKT = nkt_of(K);
  if (row0 < 0 || row0 + nrows > N) return 1;
  for (int64_t t = 0; t < nrows; t++) {
    int64_t n = row0 + t;
    for (int64_t k = 0; k < K; k++) {
      double s = oracle_f16_to_f64(decode_scale(packed, n, k, NKT, &f));
      int q = decode_u(packed, n, k, NKT, &f) - decode_offset(packed, n, k, NKT, &f);
      out[t * K + k] = (double)q * s;
    }
  }
  return 0;
}

/* --------------------------------- sweep --------------------------------- */

typedef struct {
  const uint8_t* packed;
  int64_t N, K;
  int fmt;
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
    if (oracle_dequant(J->packed, J->N, J->K, J->fmt, n, 1, wrow)) {
      J->status = 1;
      break;
    }
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
int oracle_sweep_f64(const uint8_t* packed, int64_t N, int64_t K, int fmt, const uint16_t* X,
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
    J->fmt = fmt;
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
