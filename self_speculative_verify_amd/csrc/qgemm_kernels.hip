// gfx950 kernels of the quantized weight sweep: pack, verify acceptance, workspace fill,
// and the launch helpers of every sweep kernel.
//
// The method (Quasar/q27 wiki): decode streams every quantized linear weight
// once per step ("decode physics" paragraph) and one weight read serves all
// draft positions of all slots (intro bullets on the fused verify sweep and
// the width-12 verify GEMM).  The weights are symmetric group-wise codes with
// fp16 scales, dequantized inside the product ("Weights" item of the
// engine-internals list).  Here: group 32, 4 or 5 bits, a tiled layout whose
// 1152/1408-byte tiles are read with one 16-byte load per lane.
//
// Exactness: codes are unpacked to exact fp16 integers (IEEE binary16 with
// exponent field 25 has unit spacing on [1024, 2048), so OR-ing a code into
// the mantissa of 1024.0 and subtracting 1024 + bias gives q exactly); every
// product q * x is exact in fp32 and each group's partial sum is scaled by
// its own fp32 scale.  Rounding a dequantized q*s to fp16 would not be exact.
#include <mutex>

#include "qgemm.h"
#include "sweep_device.h"

namespace qg {

// Scratch of the allocation-free sweep: one static array, which every GPU
// the library runs on holds (at its own address) until the process ends.  In
// host code `scratch` names a host-side stand-in, not device memory: only the
// address fetched per device below is ever passed to a kernel or a copy.
static __device__ __align__(256) uint8_t scratch[QGEMM_NOALLOC_SCRATCH_BYTES];

// The current device's copy of the scratch array (and its size): its
// address is fetched once per device, with that device current, and kept.
hipError_t scratch_base(uint8_t** base, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *base = (uint8_t*)addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

// --------------------------------------------------------------------------
// pack
// --------------------------------------------------------------------------

// binary64 -> binary16 bits, round to nearest even, from the bit fields.
__device__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t b = __double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7ff);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7ff) return sign | (man ? 0x7e00u : 0x7c00u);
  if (ex == 0) return sign;                       // zero or fp64 subnormal: rounds to 0
  int e = ex - 1023;                              // |x| in [2^e, 2^(e+1))
  if (e > 15) return sign | 0x7c00u;
  if (e < -25) return sign;
  const uint64_t sig = man | (1ull << 52);        // |x| = sig * 2^(e-52)
  const int ue = (e < -14 ? -14 : e) - 10;        // exponent of the target ulp
  const int sh = 52 + ue - e;                     // 42 .. 53
  uint64_t r = sig >> sh;
  const uint64_t rem = sig & ((1ull << sh) - 1);
  const uint64_t half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (r & 1))) r++;
  if (e < -14) return sign | (uint16_t)r;         // subnormal (r == 1024: min normal)
  if (r == 2048) {
    r = 1024;
    e++;
  }
  if (e > 15) return sign | 0x7c00u;
  return sign | (uint16_t)(((e + 15) << 10) | (int)(r - 1024));
}

// One thread per (row n of the padded grid, k tile): quantizes the tile's
// groups of that row and writes its 4 x 16 code bytes, its scales and (5-bit)
// 4 x 4 high-bit bytes or (zero-point format) its 16-bit zero-point word.  No
// two threads write the same byte.
//   symmetric (Q4, Q5, G64): s = fp16(amax / Qmax), u = clamp(rint(w / s)) + bias
//   zero point (ZP): lo = min(0, min w), hi = max(0, max w),
//     s = fp16((hi - lo) / 15), z = clamp(rint(-lo / s), 0, 15),
//     u = clamp(rint(w / s) + z, 0, 15)
template <int F>
__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ W, int64_t ldw, int N,
                                                   int K, int nkt, int64_t total,
                                                   uint8_t* __restrict__ packed,
                                                   unsigned* __restrict__ flag) {
  constexpr int BITS = F == kFmtQ5 ? 5 : 4;
  constexpr bool kZP = F == kFmtZP;
  constexpr int GS = fmt_group(F), NG = kTileK / GS;  // groups of a row in a tile
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int n = (int)(idx / nkt), kt = (int)(idx % nkt);
  const int r = n & 15;
  const int qmax = (1 << (BITS - 1)) - 1, bias = kZP ? 0 : 1 << (BITS - 1);
  const int G = K / GS;
  uint8_t* tile = packed + ((int64_t)(n >> 4) * nkt + kt) * tile_bytes(F);
  uint32_t code[4][4];
  uint32_t hi[4] = {0, 0, 0, 0};
  uint16_t sc[NG];
  uint32_t zw = 0;
  bool bad = false;
#pragma unroll
  for (int h = 0; h < NG; h++) {
    const int g = NG * kt + h;
    int u[GS];
    uint16_t sb = 0;
    if (n < N && g < G) {
      const float* w = W + (int64_t)n * ldw + (int64_t)g * GS;
      float v[GS];
#pragma unroll
      for (int t = 0; t < GS; t++) {
        v[t] = w[t];
        if (!isfinite(v[t])) bad = true;
      }
      if constexpr (!kZP) {
        float amax = 0.f;
#pragma unroll
        for (int t = 0; t < GS; t++) amax = fmaxf(amax, fabsf(v[t]));
        sb = f64_to_f16_bits((double)amax / (double)qmax);
        if ((sb & 0x7c00u) == 0x7c00u) bad = true;
        const double s = (double)__builtin_bit_cast(_Float16, sb);
#pragma unroll
        for (int t = 0; t < GS; t++) {
          int q = 0;
          if (s != 0.0 && isfinite(v[t]) && isfinite(s)) {
            double qq = rint((double)v[t] / s);
            qq = fmin(fmax(qq, (double)-qmax), (double)qmax);
            q = (int)qq;
          }
          u[t] = q + bias;
        }
      } else {
        float lo = 0.f, hi_ = 0.f;
#pragma unroll
        for (int t = 0; t < GS; t++) {
          lo = v[t] < lo ? v[t] : lo;
          hi_ = v[t] > hi_ ? v[t] : hi_;
        }
        sb = f64_to_f16_bits(((double)hi_ - (double)lo) / 15.0);
        if ((sb & 0x7c00u) == 0x7c00u) bad = true;
        const double s = (double)__builtin_bit_cast(_Float16, sb);
        const bool ok = s != 0.0 && isfinite(s);
        int z = 0;
        if (ok) z = (int)fmin(fmax(rint(-(double)lo / s), 0.0), 15.0);
        zw |= (uint32_t)z << (4 * h);
#pragma unroll
        for (int t = 0; t < GS; t++) {
          int uu = z;
          if (ok && isfinite(v[t])) uu = (int)fmin(fmax(rint((double)v[t] / s) + z, 0.0), 15.0);
          u[t] = uu;
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < GS; t++) u[t] = bias;
    }
    sc[h] = sb;
    // the 32-k groups j of this scale group, as code words
#pragma unroll
    for (int jj = 0; jj < GS / 32; jj++) {
      const int j = h * (GS / 32) + jj;
#pragma unroll
      for (int c = 0; c < 4; c++) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; e++) {
          const int uu = u[32 * jj + 8 * c + e];
          word |= (uint32_t)(uu & 15) << (4 * (e >> 1) + 16 * (e & 1));
          if (BITS == 5) hi[c] |= (uint32_t)((uu >> 4) & 1) << ((4 + 16 * (e & 1) + 4 * (e >> 1) + j) & 31);
        }
        code[c][j] = word;
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    u4_t v = {code[c][0], code[c][1], code[c][2], code[c][3]};
    *(u4_t*)(tile + 16 * (r + 16 * c)) = v;
    if (BITS == 5) *(uint32_t*)(tile + kHiOff + 4 * (r + 16 * c)) = hi[c];
  }
  if constexpr (NG == 4) {
    u2_t s2 = {(uint32_t)sc[0] | ((uint32_t)sc[1] << 16), (uint32_t)sc[2] | ((uint32_t)sc[3] << 16)};
    *(u2_t*)(tile + kScaleOff + 8 * r) = s2;
  } else {
    *(uint32_t*)(tile + kScaleOff + 4 * r) = (uint32_t)sc[0] | ((uint32_t)sc[1] << 16);
  }
  if constexpr (kZP) *(uint16_t*)(tile + kZeroOff + 2 * r) = (uint16_t)zw;
  if (bad) atomicOr(flag, 1u);
}

// Verify head, after the sweep: each row's key (the largest of its copies)
// becomes its argmax column and maximum; each slot accepts its drafts up to
// the first row whose argmax is not the next draft token.  The keys are reset
// for the next call.
__global__ void __launch_bounds__(64) accept_kernel(AcceptArgs a, unsigned long long* keys, const int32_t* drafts,
                                                    int32_t* argmax, float* maxval, int32_t* accepted) {
  __shared__ int32_t am[64];
  const int t = threadIdx.x;
  if (t < a.M) {
    unsigned long long k = 0ull;
    for (int c = 0; c < kKeyCopies; c++) {
      k = umax64(k, keys[c * kKeyRows + t]);
      keys[c * kKeyRows + t] = 0ull;
    }
    am[t] = key_column(k);
    argmax[t] = am[t];
    if (maxval) maxval[t] = key_value(k);
  }
  __syncthreads();
  if (t < a.nslots) {
    const int r0 = a.row0[t], nd = a.ndraft[t];
    int L = 0;
    while (L < nd && am[r0 + L] == drafts[r0 + L]) L++;
    accepted[t] = L;
  }
}

hipError_t launch_accept(const AcceptArgs& a, unsigned long long* keys, const int32_t* drafts, int32_t* argmax,
                         float* maxval, int32_t* accepted, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(64), 0, stream, a, keys, drafts, argmax, maxval, accepted);
  return hipGetLastError();
}

// zero fill for workspaces (no memset node, safe under capture)
__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// --------------------------------------------------------------------------
// launch helpers called by the host dispatcher
// --------------------------------------------------------------------------
hipError_t launch_pack(const float* W, int64_t ldw, int N, int K, int bits, void* packed,
                       unsigned* flag, hipStream_t stream) {
  const int nkt = (K + kTileK - 1) / kTileK;
  const int nrb = (N + kTileRows - 1) / kTileRows;
  const int64_t total = (int64_t)nrb * kTileRows * nkt;
  const int64_t blocks = (total + 255) / 256;
  // bits: a format code
  auto f = bits == kFmtQ5 ? pack_kernel<kFmtQ5> : bits == kFmtG64 ? pack_kernel<kFmtG64>
         : bits == kFmtZP ? pack_kernel<kFmtZP> : pack_kernel<kFmtQ4>;
  hipLaunchKernelGGL(f, dim3((unsigned)blocks), dim3(256), 0, stream, W, ldw, N, K, nkt, total, (uint8_t*)packed,
                     flag);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  int64_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t*)p, words);
  return hipGetLastError();
}

typedef void (*sweep_fn)(SweepArgs);

// stream_*.hip: the stream kernels of one format set each; group_kernels.hip
sweep_fn pick_stream_q4(bool mfma, int cls, int rows);
sweep_fn pick_stream_q5(bool mfma, int cls, int rows);
sweep_fn pick_stream_q4q5(bool mfma, int cls, int rows);
sweep_fn pick_stream_all(bool mfma, int cls, int rows);
sweep_fn pick_group(int cls, bool all);

static sweep_fn pick_stream(bool mfma, int cls, int rows, int fs) {
  switch (fs) {
    case 1: return pick_stream_q4(mfma, cls, rows);
    case 2: return pick_stream_q5(mfma, cls, rows);
    case 3: return pick_stream_q4q5(mfma, cls, rows);
  }
  return pick_stream_all(mfma, cls, rows);
}

// kind: 0 = stream GEMV (cls = rows 1, 2, 4, 8), 1 = stream MFMA (cls 1, 2, 4,
// 8, 16), 2 = group MFMA (cls = padded rows 32, 48, 64).  fs: the formats of
// the launch's jobs (bit 0: 4-bit, 1: 5-bit, 2: group-64, 3: zero-point);
// rows: row blocks per step of a stream kernel.
static sweep_fn pick(int kind, int cls, int fs, int rows) {
  if (kind == 2) return pick_group(cls, (fs & ~3) != 0);
  return pick_stream(kind == 1, cls, rows, fs);
}

int sweep_threads(int kind, int cls) { return kind == 2 ? 64 * group_waves(cls) : 64 * kStreamWavesPerBlock; }

int sweep_blocks_per_cu(int kind, int cls, int fs, int rows) {
  sweep_fn f = pick(kind, cls, fs, rows);
  if (!f) return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)f, sweep_threads(kind, cls), 0) != hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_sweep(int kind, int cls, int fs, int rows, const SweepArgs& args, int grid, hipStream_t stream) {
  sweep_fn f = pick(kind, cls, fs, rows);
  if (!f) return hipErrorInvalidValue;
  hipLaunchKernelGGL(f, dim3(grid), dim3(sweep_threads(kind, cls)), 0, stream, args);
  return hipGetLastError();
}

}  // namespace qg
