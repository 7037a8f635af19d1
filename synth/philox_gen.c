/*
 * Seeded synthetic inputs for the quantized weight sweep: host implementation.
 *
 * This file is an INPUT GENERATOR.  It holds none of the method's arithmetic
 * (no scales, codes, packing or products); it only draws the random weights
 * and activations that both the CPU oracle and the GPU library consume.
 * synth/synth_gpu.hip implements the very same definition for bulk generation
 * on the device; tests check the two agree bit for bit.
 *
 * Definition (shared with the device implementation):
 *
 *   Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 *   Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds of
 *     (hi0,lo0) = 0xD2511F53 * c0,  (hi1,lo1) = 0xCD9E8D57 * c2   (32x32->64)
 *     c = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)
 *   with the key bumped by (0x9E3779B9, 0xBB67AE85) between rounds.
 *
 *   Stream layout: key = (seed mod 2^32, seed >> 32); counter =
 *   (b mod 2^32, b >> 32, stream, 0) for block number b.
 *
 *   Normal variate number i of a stream: the Irwin-Hall sum of twelve
 *   uniforms, taken from blocks 3i, 3i+1, 3i+2 (words in order):
 *     isum = sum_{t<12} word_t + 6 - 6*2^32        (exact int64)
 *     z    = isum / 2^32                            (exact in fp64; mean 0,
 *                                                   variance 1, support +-6)
 *   A weight with standard deviation sigma is  (float)((double)isum * c)
 *   with c = sigma * 2^-32 in fp64 (one fp64 rounding, then one RNE to fp32).
 *
 *   Outlier mask of element i: word 0 of block i of the mask stream is below
 *   `thresh` (thresh = floor(p * 2^32)).  A masked weight becomes
 *   (float)((double)w * mult), exact in fp64 then one RNE to fp32.
 *
 * Everything above is integer arithmetic plus single correctly rounded IEEE
 * operations, so the host and device produce identical bits.
 */
#include <stdint.h>
#include <stddef.h>
#include <pthread.h>

static void philox4x32_10(const uint32_t ctr_in[4], uint32_t k0, uint32_t k1,
                          uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  for (int r = 0; r < 10; r++) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
    uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

/* Raw Philox block, exported for known-answer tests. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2],
                         uint32_t out[4]) {
  philox4x32_10(ctr, key[0], key[1], out);
}

static void block(uint64_t seed, uint32_t stream, uint64_t b, uint32_t out[4]) {
  uint32_t ctr[4] = {(uint32_t)b, (uint32_t)(b >> 32), stream, 0u};
  philox4x32_10(ctr, (uint32_t)seed, (uint32_t)(seed >> 32), out);
}

static int64_t irwin_hall12(uint64_t seed, uint32_t stream, uint64_t i) {
  uint32_t w[4];
  int64_t s = 0;
  for (int t = 0; t < 3; t++) {
    block(seed, stream, 3 * i + (uint64_t)t, w);
    s += (int64_t)w[0] + (int64_t)w[1] + (int64_t)w[2] + (int64_t)w[3];
  }
  return s + 6 - 6 * ((int64_t)1 << 32);
}

/* z_i = isum_i / 2^32 for i in [first, first+count), exact fp64. */
void synth_std_normal_f64(uint64_t seed, uint32_t stream, uint64_t first,
                          int64_t count, double* out) {
  const double inv = 1.0 / 4294967296.0;
  for (int64_t t = 0; t < count; t++)
    out[t] = (double)irwin_hall12(seed, stream, first + (uint64_t)t) * inv;
}

/* Mask words: 1 where element i of the mask stream is an outlier. */
void synth_outlier_mask(uint64_t seed, uint32_t stream, uint64_t first,
                        int64_t count, uint32_t thresh, uint8_t* out) {
  uint32_t w[4];
  for (int64_t t = 0; t < count; t++) {
    block(seed, stream, first + (uint64_t)t, w);
    out[t] = (uint8_t)(w[0] < thresh);
  }
}

typedef struct {
  uint64_t seed;
  int64_t K;
  int64_t row0, row1;
  double c;
  uint32_t wstream, mstream, thresh;
  double mult;
  float* out;
  int64_t ldo;
  int64_t out_row0;
} wjob_t;

static void* weights_worker(void* p) {
  wjob_t* j = (wjob_t*)p;
  uint32_t w[4];
  for (int64_t n = j->row0; n < j->row1; n++) {
    float* o = j->out + (n - j->out_row0) * j->ldo;
    for (int64_t k = 0; k < j->K; k++) {
      uint64_t i = (uint64_t)n * (uint64_t)j->K + (uint64_t)k;
      float v = (float)((double)irwin_hall12(j->seed, j->wstream, i) * j->c);
      if (j->thresh) {
        block(j->seed, j->mstream, i, w);
        if (w[0] < j->thresh) v = (float)((double)v * j->mult);
      }
      o[k] = v;
    }
  }
  return NULL;
}

/*
 * Rows [row0, row0+nrows) of the N x K weight matrix of `seed` (element index
 * i = n*K + k), written to out[(n-row0)*ldo + k].  thresh = 0 disables
 * outliers.  Work is split over `nthreads` POSIX threads by rows.
 */
int synth_weights_f32(uint64_t seed, int64_t K, int64_t row0, int64_t nrows,
                      double sigma, uint32_t wstream, uint32_t mstream,
                      uint32_t thresh, double mult, float* out, int64_t ldo,
                      int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nrows < nthreads) nthreads = nrows > 0 ? (int)nrows : 1;
  pthread_t th[256];
  wjob_t jobs[256];
  const double c = sigma / 4294967296.0;
  for (int t = 0; t < nthreads; t++) {
    wjob_t* j = &jobs[t];
    j->seed = seed;
    j->K = K;
    j->row0 = row0 + nrows * t / nthreads;
    j->row1 = row0 + nrows * (t + 1) / nthreads;
    j->c = c;
    j->wstream = wstream;
    j->mstream = mstream;
    j->thresh = thresh;
    j->mult = mult;
    j->out = out;
    j->ldo = ldo;
    j->out_row0 = row0;
  }
  int started = 0;
  for (int t = 1; t < nthreads; t++) {
    if (pthread_create(&th[t], NULL, weights_worker, &jobs[t]) != 0) break;
    started = t;
  }
  weights_worker(&jobs[0]);
  for (int t = 1; t <= started; t++) pthread_join(th[t], NULL);
  for (int t = started + 1; t < nthreads; t++) weights_worker(&jobs[t]);
  return 0;
}
