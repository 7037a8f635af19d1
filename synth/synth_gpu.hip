// Seeded synthetic weights on the device: an INPUT GENERATOR, not part of the
// quantized sweep.  Same definition as the host generator in philox_gen.c
// (Philox4x32-10 of Salmon et al., SC'11; Irwin-Hall sum of twelve uniforms;
// one fp64 rounding then one RNE to fp32; Bernoulli outlier mask on its own
// stream).  Only integer arithmetic and single correctly rounded IEEE
// operations are used, so its output matches the host generator bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1, uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; r++) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0;
    const uint32_t n2 = hi0 ^ c3 ^ k1;
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

__global__ void __launch_bounds__(256) weights_kernel(uint64_t seed, int64_t K, int64_t row0,
                                                      int64_t nrows, double c, uint32_t wstream,
                                                      uint32_t mstream, uint32_t thresh,
                                                      double mult, float* out, int64_t ldo) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int64_t total = nrows * K;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / K, k = t - r * K;
    const uint64_t i = (uint64_t)(row0 + r) * (uint64_t)K + (uint64_t)k;
    int64_t s = 0;
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 3; q++) {
      const uint64_t b = 3 * i + (uint64_t)q;
      philox((uint32_t)b, (uint32_t)(b >> 32), wstream, 0u, k0, k1, w);
      s += (int64_t)w[0] + (int64_t)w[1] + (int64_t)w[2] + (int64_t)w[3];
    }
    s += 6 - 6 * ((int64_t)1 << 32);
    float v = (float)((double)s * c);
    if (thresh) {
      philox((uint32_t)i, (uint32_t)(i >> 32), mstream, 0u, k0, k1, w);
      if (w[0] < thresh) v = (float)((double)v * mult);
    }
    out[r * ldo + k] = v;
  }
}

}  // namespace

extern "C" int synth_weights_f32_gpu(uint64_t seed, int64_t K, int64_t row0, int64_t nrows,
                                     double sigma, uint32_t wstream, uint32_t mstream,
                                     uint32_t thresh, double mult, float* out, int64_t ldo,
                                     void* stream) {
  if (K <= 0 || nrows <= 0 || ldo < K || out == nullptr) return 1;
  const double c = sigma / 4294967296.0;
  const int64_t total = nrows * K;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(weights_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     seed, K, row0, nrows, c, wstream, mstream, thresh, mult, out, ldo);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
