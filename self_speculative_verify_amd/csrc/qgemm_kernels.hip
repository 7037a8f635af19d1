// gfx950 kernels of the quantized weight sweep: pack, GEMV sweep, MFMA sweep.
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
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm_internal.h"

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

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

// --------------------------------------------------------------------------
// sweep: shared pieces
// --------------------------------------------------------------------------
// Explicit address spaces keep every weight/activation access a global_load
// (never flat) and every job descriptor read a scalar load.  The host pass of
// the compiler has no such address spaces.
#if defined(__HIP_DEVICE_COMPILE__)
#define QG_GLOBAL __attribute__((address_space(1)))
#define QG_CONST __attribute__((address_space(4)))
#else
#define QG_GLOBAL
#define QG_CONST
#endif

// Split-K partial sums are exchanged through raw buffer accesses with the
// system-coherent cache policy (sc0 sc1: written through to and read from
// memory, as system-scope atomics are), which also vectorize.  kBufWord3 is
// word 3 of a raw (untyped) gfx9 buffer descriptor.
constexpr int kBufWord3 = 0x00020000;
constexpr int kCoherent = 1 | 16;

template <typename T>
__device__ __forceinline__ const QG_GLOBAL T* gload_ptr(const void* p) {
  return (const QG_GLOBAL T*)p;
}

// Eight codes of one group chunk (code word w of group J, high word h) ->
// four fp16 pairs holding the exact q; pair i holds elements (2i, 2i+1).
// Pair i's low nibbles sit at bits (4i, 16+4i) of w.  OR-ing 0x6400 into an
// fp16 sets its exponent field to 25 (value 1024, unit spacing), so
//   pair 0: (w & 0x000F000F) | 0x64006400 = 1024 + u     -> q = t - (1024 + bias)
//   pair 1: (w & 0x00F000F0) | 0x64006400 = 1024 + 16u   -> q = t / 16 - (64 + bias)
// and pairs 2, 3 the same from w >> 8.  Both forms are exact: one packed fp16
// add or fma whose operands and result are exactly representable.  5-bit:
// bit 4 of the pair-i codes of group J sits at bits (4 + 4i + J, 20 + 4i + J)
// mod 32 of h, so rotr(h, J) places pairs 0 and 1 at (4, 20) and (8, 24) --
// bit 4 of u in the first form, of 16u in the second -- and rotr(h, J + 8)
// does the same for pairs 2 and 3.
// v_and_or_b32 (a & m) | o in one instruction.  Written out because with two
// literal operands the compiler splits it into v_and + v_or (a VOP3 encoding
// holds no literal on this target); here the constants live in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(o));
  return r;
}

// Zero-point format: u is stored as is and the subtrahends are per group:
// -(1024 + z) for the first form, -(64 + z) for the second, as fp16 pairs
// built from the zero-point word zz (the row's 16-bit word in both halves):
// 0xE400 | z is -(1024 + z) and 0xD400 | 16 z is -(64 + z), both exact.
template <int F>
__device__ __forceinline__ void unpack8(uint32_t w, uint32_t h, int J, h2_t (&q)[4]) {
  constexpr uint32_t kMagic = 0x64006400u;
  constexpr int kBias = F == kFmtQ5 ? 16 : 8;
  constexpr _Float16 kOff0 = (_Float16)(-1024 - kBias);
  constexpr _Float16 kOff1 = (_Float16)(-64 - kBias);
  h2_t off0 = {kOff0, kOff0}, off1 = {kOff1, kOff1};
  if constexpr (F == kFmtZP) {
    off0 = __builtin_bit_cast(h2_t, and_or(J ? __builtin_amdgcn_alignbit(h, h, 4 * J) : h, 0x000F000Fu, 0xE400E400u));
    off1 = __builtin_bit_cast(h2_t, and_or(J == 1 ? h : __builtin_amdgcn_alignbit(h, h, (4 * J + 28) & 31),
                                           0x00F000F0u, 0xD400D400u));
  }
  const h2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const uint32_t w2 = w >> 8;
  uint32_t t0 = and_or(w, 0x000F000Fu, kMagic), t1 = and_or(w, 0x00F000F0u, kMagic);
  uint32_t t2 = and_or(w2, 0x000F000Fu, kMagic), t3 = and_or(w2, 0x00F000F0u, kMagic);
  if constexpr (F == kFmtQ5) {
    const uint32_t h0 = __builtin_amdgcn_alignbit(h, h, J);
    const uint32_t h2 = __builtin_amdgcn_alignbit(h, h, J + 8);
    t0 = and_or(h0, 0x00100010u, t0);
    t1 = and_or(h0, 0x01000100u, t1);
    t2 = and_or(h2, 0x00100010u, t2);
    t3 = and_or(h2, 0x01000100u, t3);
  }
  q[0] = __builtin_bit_cast(h2_t, t0) + off0;
  q[1] = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, t1), sixteenth, off1);
  q[2] = __builtin_bit_cast(h2_t, t2) + off0;
  q[3] = __builtin_elementwise_fma(__builtin_bit_cast(h2_t, t3), sixteenth, off1);
}

// The per-row word a format keeps beside the codes, as unpack8 takes it: the
// 5-bit high word, or the zero-point word in both halves.
template <int F>
__device__ __forceinline__ uint32_t side_word(uint32_t h) {
  if constexpr (F == kFmtZP) return h | (h << 16);
  return h;
}

__device__ __forceinline__ h8_t cat8(const h2_t (&q)[4]) {
  h8_t o;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    o[2 * i] = q[i].x;
    o[2 * i + 1] = q[i].y;
  }
  return o;
}

// (J is a constant after unrolling, so the rotations take immediates.)
template <int F>
__device__ __forceinline__ h8_t unpack_chunk(uint32_t w, uint32_t hi, int J) {
  h2_t q[4];
  unpack8<F>(w, hi, J, q);
  return cat8(q);
}

// X chunks are written to and read from LDS as the same 16-byte integer
// vector type (then bit-cast), so type-based alias analysis can never move a
// read above the write that produced it.
__device__ __forceinline__ h8_t lds_h8(const uint8_t* p) { return __builtin_bit_cast(h8_t, *(const u4_t*)p); }

// Two fp16 scales from one 32-bit word.  The word is taken by value: a
// bit_cast applied directly to an element of a vector register type was
// compiled to an undefined value (only element 0 survived).
__device__ __forceinline__ h2_t scale_pair(uint32_t word) { return __builtin_bit_cast(h2_t, word); }

// One fp16 scale of a packed pair to fp32 as an instruction of its own, so the
// scale products that follow are two-operand fp32 FMAs; left to itself the
// compiler fuses the conversion into mixed-precision FMAs, which issue more
// slowly on gfx950.
template <int HI>
__device__ __forceinline__ float scale_f32(uint32_t pair) {
  float f;
  if constexpr (HI) asm("v_cvt_f32_f16_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1" : "=v"(f) : "v"(pair));
  else asm("v_cvt_f32_f16_e32 %0, %1" : "=v"(f) : "v"(pair));
  return f;
}

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
// maximum of a 64-bit key over the lanes l ^ mask for mask < span (a power
// of two), bit by bit
template <int kFrom, int kSpan>
__device__ __forceinline__ unsigned long long lanes_max(unsigned long long k) {
#pragma unroll
  for (int m = kFrom; m < kSpan; m <<= 1) k = umax64(k, __shfl_xor(k, m));
  return k;
}
__device__ __forceinline__ void key_max(unsigned long long* p, unsigned long long k) {
  __hip_atomic_fetch_max(p, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ const QG_CONST JobDesc* job_table(const SweepArgs& a) {
  return a.table ? (const QG_CONST JobDesc*)a.table : (const QG_CONST JobDesc*)&a.inl[0];
}

// --------------------------------------------------------------------------
// stream kernels: panels of at most 16 rows (GEMV, or MFMA with one m block)
// --------------------------------------------------------------------------
// Work is a flat sequence of steps (job, row group, k tile); a row group is
// kR consecutive 16-row blocks, and one step reads the kR tiles of its row
// group at one k tile.  The sequence is cut into `nwaves` equal contiguous
// ranges, one per wave, so every wave streams the same number of steps.
// Within one job a row group's steps are consecutive tiles in memory per row
// block (tile index rb * NKT + kt), so the weight pointers simply advance.  A
// wave accumulates one row group at a time; a row group whose steps all lie in
// one range is written to Y directly.  A row group cut by range ends gets one
// partial sum per contributing wave, stored into that wave's slot; the last
// contributor to arrive (per-row-group counter) adds the partials in wave
// order -- k order -- writes Y and resets the counter to zero.  Nothing waits
// on another wave.  The slots and counters are accessed with system-scope
// atomics, which bypass the per-XCD L2 caches (not coherent with each other).
//
// MFMA: v_mfma_f32_16x16x32_f16 with A = X (16 rows x 32 k of one group)
// and B = codes (32 k x 16 rows n): lane l supplies A row l%16 and B column
// n = l%16, both for k chunk l/16 -- exactly the lane's 16 code bytes -- and
// holds D rows 4(l/16) + i of column n.  X row m is placed at A row
// 4(m%4) + m/4, so it comes out in lane group g = m%4, accumulator i = m/4
// (m = g + 4i): a panel of at most 4 kA rows keeps kA = ceil(class / 4)
// accumulators per lane, and the group's scale (one per lane) multiplies only
// those.  A rows whose m >= M read X row M-1 and feed outputs that are never
// stored (MFMA rows are independent).  The placement is the same for every
// class, so a row's arithmetic does not depend on the panel height.
// GEMV: lane l = r + 16c forms, for row n = r and each m, four v_dot2_f32_f16
// over its 8 codes of a group, scaled by the group's scale; the four k chunks
// of a row (lanes r, r+16, r+32, r+48) are summed when the row group is
// written.  X chunks go through a small wave-private LDS buffer.
// Padding groups (beyond K) have codes q = 0 and scale +0, and their X reads
// are clamped into the row, so they add exact zeros: no tile needs a branch.
template <bool kMfma, int kCap, bool kBig>
struct Stream {
  static constexpr int kR = stream_rows(kBig);                        // row blocks per step
  static constexpr int kA = kMfma ? (kCap + 3) / 4 : kCap;           // accumulators per row block
  // Partial-sum slots hold a row group's rows at positions 0 .. class - 1,
  // a lane's accumulators side by side: position kA g + i is row g + 4 i
  // (MFMA), position m row m (GEMV).
  static __device__ __forceinline__ int slot_row(int p) { return kMfma ? p / kA + 4 * (p % kA) : p; }
  static constexpr int kXP = kMfma ? 4 : (kCap * 16 + 63) / 64;      // X loads per lane per step
  // steps in flight per wave: 16 tiles (17-23 KB) per wave either way
  static constexpr int kDepth = kBig ? 2 : 4;

  // one step's loads: codes, scales (group 64: the pair of word s.x), the
  // side word (5-bit high bits or zero points) and the X chunk
  template <int F>
  struct Step {
    u4_t c[kR];
    u2_t s[kR];
    uint32_t h[F == kFmtQ5 || F == kFmtZP ? kR : 1];
    u4_t x[kXP];
  };

  // Position of a step cursor: wp points at tile (rg * kR, kt) of the job and
  // the step's tile r sits roff[r] bytes further (blocks past the job's last
  // read the last one again; their sums are never stored).  Offsets fit 32
  // bits because K <= 2^24 (host check).
  struct Cur {
    const uint8_t* wp;
    uint32_t roff[kR];
    int kt, rg;
  };

  static __device__ __forceinline__ void set_rows(Cur& c, int nrb, uint32_t rstride) {
    const int left = nrb - 1 - c.rg * kR;  // >= 0
#pragma unroll
    for (int r = 0; r < kR; r++) c.roff[r] = (uint32_t)(r < left ? r : left) * rstride;
  }

  // Redirect a finished prefetch cursor to base (its loads are never used).
  static __device__ __forceinline__ void spill_to(Cur& c, const uint8_t* base) {
    if (base == nullptr) return;
    c.wp = base;
#pragma unroll
    for (int r = 0; r < kR; r++) c.roff[r] = 0;
  }

  static __device__ __forceinline__ void advance(Cur& c, int nkt, int nrb, uint32_t rstride, uint32_t tb) {
    c.wp += tb;
    if (++c.kt == nkt) {
      c.kt = 0;
      c.rg++;
      c.wp += (uint64_t)(kR - 1) * rstride;
      set_rows(c, nrb, rstride);
    }
  }

  // Wave w streams the steps whose first unit lies in [start(w), start(w + 1)):
  // q units each, one more for the first rem waves.
  static __device__ __forceinline__ int start_of(int w, int q, int rem) { return w * q + (w < rem ? w : rem); }
  static __device__ __forceinline__ int wave_of(int f, int q, int rem) {
    const int edge = rem * (q + 1);
    return f < edge ? f / (q + 1) : rem + (f - edge) / q;
  }

  // Everything a wave needs to place one row group's sums.
  struct Ctx;
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const Ctx& cx) {
    const int bytes = 2 * cx.G * cx.slot_rows * kR * kTileRows * 4;
    return __builtin_amdgcn_make_buffer_rsrc((void*)cx.slots, (short)0, bytes, kBufWord3);
  }
  struct Ctx {
    const QG_CONST JobDesc* D;
    int* counters;
    float* slots;
    int q, rem, G;         // partition of the flat steps over G waves
    int slot_rows;
    int gw, a, b;
    int lane;
    // split row groups whose partial this wave stored (kind 0 / kind 1)
    int pend_j0, pend_rg0, pend_j1, pend_rg1;
    // verify head: best argmax key of this lane's rows over the columns it
    // finished (accumulator i's row), published at the end of a segment
    unsigned long long best[kA];
  };

  // Write the finished sums of row group rg of job j to Y, or, for a row
  // group cut by this wave's range, store this wave's partial into its slot
  // (kind 0: the range's first row group, kind 1: its last) and note it; the
  // arrival is counted once, at the end of the range (see arrive).
  static __device__ __forceinline__ void flush(float (&acc)[kR][kA], Ctx& cx, int j, int rg) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    const int M = D[j].M, N = D[j].N, nkt = D[j].nkt;
    const int64_t ldy = D[j].ldy;
    QG_GLOBAL float* Y = (QG_GLOBAL float*)D[j].Y;
    if constexpr (!kMfma) {
#pragma unroll
      for (int r = 0; r < kR; r++)
#pragma unroll
        for (int m = 0; m < kCap; m++) {
          float v = acc[r][m];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          acc[r][m] = v;
        }
    }
    const int wt = unit_weight(D[j].fmt);
    const int first = D[j].ubeg + rg * nkt * wt;   // first unit of the row group's first step
    const int last = first + (nkt - 1) * wt;       // ... and of its last step
    const int nn = lane & 15;
    // row m held by this lane in accumulator i (MFMA), or m = i (GEMV, lanes < 16)
    auto row_of = [&](int i) { return kMfma ? (lane >> 4) + 4 * i : i; };
    const bool holder = kMfma || lane < 16;
    if (first >= cx.a && last < cx.b) {
      const bool keys = D[j].keys != nullptr;
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const int n = (rg * kR + r) * kTileRows + nn;
        if (holder && n < N) {
#pragma unroll
          for (int i = 0; i < kA; i++) {
            const int m = row_of(i);
            if (m < M) {
              if (Y) Y[(int64_t)m * ldy + n] = acc[r][i];
              if (keys) cx.best[i] = umax64(cx.best[i], logit_key(acc[r][i], n));
            }
          }
        }
      }
      return;
    }
    // partial: slot of (wave, kind), laid out [column][slot_rows] so that each
    // lane's rows are contiguous; written through to memory (system scope)
    const int srows = cx.slot_rows;
    // kind 0: the row group began before this range (its first row group);
    // kind 1: it begins inside and runs past the range (its last)
    const int kind = cx.a > first ? 0 : 1;
    const uint32_t sbase = (uint32_t)((cx.gw * 2 + kind) * srows * kR * kTileRows) * 4u;
    const __amdgpu_buffer_rsrc_t sr = slot_rsrc(cx);
    if constexpr (kMfma) {
      // this lane's rows go to slot positions kA g .. kA g + kA - 1
      const int p0 = kA * (lane >> 4);
      if (p0 < srows) {
#pragma unroll
        for (int r = 0; r < kR; r++) {
          const uint32_t o = sbase + (uint32_t)(((r * kTileRows + nn) * srows + p0) * 4);
          if constexpr (kA == 4) {
            const f4_t v = {acc[r][0], acc[r][1], acc[r][2], acc[r][3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), sr, o, 0, kCoherent);
          } else if constexpr (kA == 2) {
            const f2_t v = {acc[r][0], acc[r][1]};
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, v), sr, o, 0, kCoherent);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[r][0]), sr, o, 0, kCoherent);
          }
        }
      }
    } else if (lane < 16) {
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const uint32_t o = sbase + (uint32_t)((r * kTileRows + nn) * srows * 4);
        if constexpr (kCap == 1) {
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[r][0]), sr, o, 0, kCoherent);
        } else if constexpr (kCap == 2) {
          const f2_t v = {acc[r][0], acc[r][1]};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2_t, v), sr, o, 0, kCoherent);
        } else {
#pragma unroll
          for (int q = 0; q < kCap; q += 4) {
            const f4_t v = {acc[r][q], acc[r][q + 1], acc[r][q + 2], acc[r][q + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), sr, o + 4u * q, 0, kCoherent);
          }
        }
      }
    }
    if (kind == 0) {
      cx.pend_j0 = j;
      cx.pend_rg0 = rg;
    } else {
      cx.pend_j1 = j;
      cx.pend_rg1 = rg;
    }
  }

  // A split row group's contributors are the waves wf..wl whose ranges hold
  // its first and last steps; its arrival counter is at counters[rg_begin + rg].
  static __device__ __forceinline__ void span(const Ctx& cx, int j, int rg, int& wf, int& wl) {
    const QG_CONST JobDesc* D = cx.D;
    const int wt = unit_weight(D[j].fmt), nkt = D[j].nkt;
    const int first = D[j].ubeg + rg * nkt * wt;
    wf = wave_of(first, cx.q, cx.rem);
    wl = wave_of(first + (nkt - 1) * wt, cx.q, cx.rem);
  }

  // Sums of split row groups.  The last contributor to arrive at a row group
  // (every partial stored and complete) adds all partials in wave order -- k
  // order -- writes Y and resets the arrival counter.  A wave can complete
  // both of its split row groups; all their partial loads are issued before
  // the first add, 4 floats per load.
  // slots hold kCap rows (the class); 4-float chunks per lane, and partials
  // loaded per batch (at least 8 loads in flight)
  static constexpr int kChunksPerLane = (kCap * kR * kTileRows / 4 + 63) / 64;
  static constexpr int kBatch = kChunksPerLane >= 8 ? 1 : 8 / kChunksPerLane;

  static __device__ __forceinline__ void reduce2(const Ctx& cx, bool do0, bool do1) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    const int srows = cx.slot_rows, cols = kR * kTileRows;
    const int slot_bytes = srows * cols * 4;
    const int nchunks = srows * cols / 4;
    const __amdgpu_buffer_rsrc_t sr = slot_rsrc(cx);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
    for (int k = 0; k < 2; k++) {
      if (k == 0 ? !do0 : !do1) continue;
      const int j = k == 0 ? cx.pend_j0 : cx.pend_j1, rg = k == 0 ? cx.pend_rg0 : cx.pend_rg1;
      int wf, wl;
      span(cx, j, rg, wf, wl);
      const int M = D[j].M, N = D[j].N;
      const int64_t ldy = D[j].ldy;
      QG_GLOBAL float* Y = (QG_GLOBAL float*)D[j].Y;
      // The first contributor holds the row group's first step (its kind-1
      // slot); every later one began inside the row group (kind 0).
      auto part = [&](int w, int q) {
        const int kw = w == wf ? 1 : 0;
        return __builtin_bit_cast(
            f4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, 16u * q, (uint32_t)((w * 2 + kw) * slot_bytes), kCoherent));
      };
      f4_t v[kChunksPerLane];
#pragma unroll
      for (int c = 0; c < kChunksPerLane; c++) v[c] = f4_t{0.f, 0.f, 0.f, 0.f};
      for (int w = wf; w <= wl; w += kBatch) {
        f4_t p[kBatch][kChunksPerLane];
#pragma unroll
        for (int t = 0; t < kBatch; t++)
#pragma unroll
          for (int c = 0; c < kChunksPerLane; c++) {
            const int q = lane + 64 * c;
            p[t][c] = (w + t <= wl && q < nchunks) ? part(w + t, q) : f4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
        for (int t = 0; t < kBatch; t++)
#pragma unroll
          for (int c = 0; c < kChunksPerLane; c++)
            if (w + t <= wl) v[c] += p[t][c];
      }
      // verify head: element t of every chunk of this lane is slot position
      // (4 lane + t) mod srows (64 chunks of 4 elements span whole columns)
      unsigned long long kb[4] = {0ull, 0ull, 0ull, 0ull};
      const bool keys = D[j].keys != nullptr;
#pragma unroll
      for (int c = 0; c < kChunksPerLane; c++) {
        const int q = lane + 64 * c;
        if (q >= nchunks) continue;
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const int e = 4 * q + t, col = e / srows, m = slot_row(e - col * srows);
          const int n = rg * cols + col;
          if (m < M && n < N) {
            if (Y) Y[(int64_t)m * ldy + n] = v[c][t];
            if (keys) kb[t] = umax64(kb[t], logit_key(v[c][t], n));
          }
        }
      }
      if (keys) {
        // lanes l and l' hold the same positions when l = l' mod max(srows / 4, 1)
        const int per = srows >= 4 ? srows / 4 : 1;
#pragma unroll
        for (int t = 0; t < 4; t++) {
          unsigned long long k = kb[t];
          for (int msk = per; msk < 64; msk <<= 1) k = umax64(k, __shfl_xor(k, msk));
          const int m = slot_row((4 * lane + t) % srows);
          if (lane < per && m < M && k != 0ull) key_max(D[j].keys + (cx.gw % kKeyCopies) * kKeyRows + m, k);
        }
      }
      if (lane == 0)
        __hip_atomic_store(cx.counters + D[j].rg_begin + rg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }

  // Count this wave's arrivals at its split row groups (kind 0 and kind 1;
  // both atomics issued before either result is used) and reduce those it
  // completes.  Called once, at the end of the range, after every partial
  // store of the wave has completed.
  static __device__ __forceinline__ void arrive(const Ctx& cx) {
    const QG_CONST JobDesc* D = cx.D;
    const bool has0 = cx.pend_j0 >= 0, has1 = cx.pend_j1 >= 0;
    int old0 = 0, old1 = 0;
    if (cx.lane == 0) {
      if (has0)
        old0 = __hip_atomic_fetch_add(cx.counters + D[cx.pend_j0].rg_begin + cx.pend_rg0, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
      if (has1)
        old1 = __hip_atomic_fetch_add(cx.counters + D[cx.pend_j1].rg_begin + cx.pend_rg1, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
    }
    old0 = __builtin_amdgcn_readfirstlane(old0);
    old1 = __builtin_amdgcn_readfirstlane(old1);
    int wf, wl;
    bool last0 = false, last1 = false;
    if (has0) {
      span(cx, cx.pend_j0, cx.pend_rg0, wf, wl);
      last0 = old0 == wl - wf;
    }
    if (has1) {
      span(cx, cx.pend_j1, cx.pend_rg1, wf, wl);
      last1 = old1 == wl - wf;
    }
    if (last0 || last1) reduce2(cx, last0, last1);
  }

  // Issue the loads of the step at cursor c: kR weight tiles (non-temporal:
  // streamed once) and the X chunk.  X reads outside [0, M) x [0, K) are
  // clamped into the matrix (see above); xlane[p] is the lane's byte offset
  // into X for k = 0.
  template <int F>
  static __device__ __forceinline__ void load(Step<F>& t, const Cur& c, const uint16_t* X,
                                              const uint32_t (&xlane)[kXP], int K, int lane) {
#pragma unroll
    for (int r = 0; r < kR; r++) {
      const uint8_t* tp = c.wp + c.roff[r];
      t.c[r] = __builtin_nontemporal_load(gload_ptr<u4_t>(tp + 16 * lane));
      if constexpr (F == kFmtG64) {
        t.s[r].x = __builtin_nontemporal_load(gload_ptr<uint32_t>(tp + kScaleOff + 4 * (lane & 15)));
        t.s[r].y = 0u;
      } else {
        t.s[r] = __builtin_nontemporal_load(gload_ptr<u2_t>(tp + kScaleOff + 8 * (lane & 15)));
      }
      if constexpr (F == kFmtQ5) t.h[r] = __builtin_nontemporal_load(gload_ptr<uint32_t>(tp + kHiOff + 4 * lane));
      if constexpr (F == kFmtZP)
        t.h[r] = __builtin_nontemporal_load(gload_ptr<uint16_t>(tp + kZeroOff + 2 * (lane & 15)));
    }
    const uint8_t* xb = (const uint8_t*)X;
    const int k0 = c.kt * kTileK;
    if constexpr (kMfma) {
      // group j of k tile kt: X[m][k0 + 32j + 8(l/16) ..]
      if (k0 + kTileK <= K) {
        const uint32_t o = xlane[0] + 2u * (uint32_t)k0;
#pragma unroll
        for (int j = 0; j < 4; j++) t.x[j] = *gload_ptr<u4_t>(xb + (o + 64u * j));
      } else {
        const int kl = k0 + 8 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const int k = kl + 32 * j < K - 8 ? k0 + 32 * j : K - 8 - 8 * (lane >> 4);
          t.x[j] = *gload_ptr<u4_t>(xb + (xlane[0] + 2u * (uint32_t)k));
        }
      }
    } else {
      // piece lane + 64p of the chunk: X[row][k0 + 8 col ..]
      const int col = lane & 15;
#pragma unroll
      for (int p = 0; p < kXP; p++) {
        if (k0 + kTileK <= K) {
          t.x[p] = *gload_ptr<u4_t>(xb + (xlane[p] + 2u * (uint32_t)k0));
        } else {
          const int k = k0 + 8 * col < K - 8 ? k0 : K - 8 - 8 * col;
          t.x[p] = *gload_ptr<u4_t>(xb + (xlane[p] + 2u * (uint32_t)k));
        }
      }
    }
  }

  template <int F>
  static __device__ __forceinline__ void compute(float (&acc)[kR][kA], const Step<F>& t, uint8_t* xs,
                                                 int lane) {
    constexpr bool kSide = F == kFmtQ5 || F == kFmtZP;
    if constexpr (kMfma) {
      const f4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const uint32_t side = side_word<F>(t.h[kSide ? r : 0]);
        f4_t p[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const h8_t q = unpack_chunk<F>(t.c[r][j], side, j);
          // group 64: the second half of a group accumulates onto the first
          const f4_t c0 = (F == kFmtG64 && (j & 1)) ? p[j ^ 1] : zero;
          p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, t.x[j]), q, c0, 0, 0, 0);
        }
        const h2_t s01 = scale_pair(t.s[r].x), s23 = scale_pair(t.s[r].y);
        const _Float16 sh[4] = {s01.x, s01.y, s23.x, s23.y};
        if constexpr (F == kFmtG64) {
#pragma unroll
          for (int h = 0; h < 2; h++)
#pragma unroll
            for (int i = 0; i < kA; i++) acc[r][i] = __builtin_fmaf((float)sh[h], p[2 * h + 1][i], acc[r][i]);
        } else {
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < kA; i++) acc[r][i] = __builtin_fmaf((float)sh[j], p[j][i], acc[r][i]);
        }
      }
    } else {
      const int c = lane >> 4;
#pragma unroll
      for (int p = 0; p < kXP; p++) {
        const int piece = lane + 64 * p;
        const int row = piece >> 4, col = piece & 15;
        if (row < kCap) *(u4_t*)(xs + row * kXRowBytes + 16 * col) = t.x[p];
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // LDS writes stay before the reads
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const h2_t s01 = scale_pair(t.s[r].x), s23 = scale_pair(t.s[r].y);
        const _Float16 sh[4] = {s01.x, s01.y, s23.x, s23.y};
        const uint32_t side = side_word<F>(t.h[kSide ? r : 0]);
        float dp[kCap];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          h2_t q[4];
          unpack8<F>(t.c[r][j], side, j, q);
          // group 64: the dot products of both halves, then one scale
          const float sj = (float)sh[F == kFmtG64 ? j >> 1 : j];
          const bool first = F != kFmtG64 || !(j & 1), last = F != kFmtG64 || (j & 1);
#pragma unroll
          for (int m = 0; m < kCap; m++) {
            const h8_t x = lds_h8(xs + m * kXRowBytes + 64 * j + 16 * c);
            const h2_t x0 = {x[0], x[1]}, x1 = {x[2], x[3]}, x2 = {x[4], x[5]}, x3 = {x[6], x[7]};
            float d = __builtin_amdgcn_fdot2(q[0], x0, first ? 0.f : dp[m], false);
            d = __builtin_amdgcn_fdot2(q[1], x1, d, false);
            d = __builtin_amdgcn_fdot2(q[2], x2, d, false);
            d = __builtin_amdgcn_fdot2(q[3], x3, d, false);
            dp[m] = d;
            if (last) acc[r][m] = __builtin_fmaf(sj, d, acc[r][m]);
          }
        }
      }
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the next step's writes stay after these reads
    }
  }

  static __device__ __forceinline__ void zero(float (&acc)[kR][kA]) {
#pragma unroll
    for (int r = 0; r < kR; r++)
#pragma unroll
      for (int i = 0; i < kA; i++) acc[r][i] = 0.f;
  }

  // Steps [s0, s1) of job j (local step index rg * NKT + kt), format F.
  template <int F>
  static __device__ __forceinline__ void segment(Ctx& cx, int j, int s0, int s1, uint8_t* xs) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    constexpr int TB = tile_bytes(F);
    const int nkt = D[j].nkt, nrb = D[j].nrb, M = D[j].M, K = D[j].K;
    const int64_t ldx = D[j].ldx;
    const uint16_t* X = D[j].X;
    const uint32_t rstride = (uint32_t)nkt * TB;
    // lane byte offsets into X (fit 32 bits: host check)
    uint32_t xlane[kXP];
    if constexpr (kMfma) {
      // A row r = l % 16 carries X row (r / 4) + 4 (r % 4)
      const int ar = lane & 15, mr = (ar >> 2) + 4 * (ar & 3);
      const int m = mr < M ? mr : M - 1;
      xlane[0] = 2u * (uint32_t)(m * ldx + 8 * (lane >> 4));
    } else {
#pragma unroll
      for (int p = 0; p < kXP; p++) {
        const int piece = lane + 64 * p;
        const int row = piece >> 4, m = row < M ? row : M - 1;
        xlane[p] = 2u * (uint32_t)(m * ldx + 8 * (piece & 15));
      }
    }
    // consume cursor
    int rg = s0 / nkt;
    int kt = s0 - rg * nkt;
    // prefetch cursor: stops at the segment's last step (later loads re-read it)
    Cur pc;
    pc.rg = rg;
    pc.kt = kt;
    pc.wp = D[j].packed + ((int64_t)rg * kR * nkt + kt) * TB;
    set_rows(pc, nrb, rstride);
    int pleft = s1 - s0 - 1;
    // Past the segment's last step the prefetch keeps issuing its fixed
    // number of loads (so the compiler's wait counts stay exact) but points
    // them at X, which every wave keeps reading and so stays cached, instead
    // of fetching weights again; X smaller than a tile: the last step.
    const uint8_t* xover = 2 * ((int64_t)(M - 1) * ldx + K) >= kTile5 ? (const uint8_t*)X : nullptr;
    Step<F> buf[kDepth];
#pragma unroll
    for (int p = 0; p < kDepth; p++) {
      load<F>(buf[p], pc, X, xlane, K, lane);
      if (pleft > 0) {
        advance(pc, nkt, nrb, rstride, TB);
        pleft--;
      } else {
        spill_to(pc, xover);
      }
    }
    float acc[kR][kA];
    zero(acc);
    const int n = s1 - s0;
    for (int f = 0; f < n; f += kDepth) {
#pragma unroll
      for (int p = 0; p < kDepth; p++) {
        if (f + p < n) {
          compute<F>(acc, buf[p], xs, lane);
          if (kt == nkt - 1 || f + p == n - 1) {
            flush(acc, cx, j, rg);
            zero(acc);
          }
          if (++kt == nkt) {
            kt = 0;
            rg++;
          }
        }
        load<F>(buf[p], pc, X, xlane, K, lane);
        if (pleft > 0) {
          advance(pc, nkt, nrb, rstride, TB);
          pleft--;
        } else {
          spill_to(pc, xover);
        }
      }
    }
    if (D[j].keys) publish(cx, D[j].keys + (cx.gw % kKeyCopies) * kKeyRows, M);
  }

  // The steps of job j whose first unit lies in [u0, u1) (units from the
  // job's first).
  template <int F>
  static __device__ __forceinline__ void segment_in(Ctx& cx, int j, int u0, int u1, uint8_t* xs) {
    constexpr int wt = unit_weight(F);
    const int s0 = (u0 + wt - 1) / wt, s1 = (u1 + wt - 1) / wt;
    if (s0 < s1) segment<F>(cx, j, s0, s1, xs);
  }

  // Verify head: the segment's best key per row, over the 16 lanes holding
  // the row's columns, into the job's keys (one atomic per row and wave).
  static __device__ __forceinline__ void publish(Ctx& cx, unsigned long long* keys, int M) {
    const int lane = cx.lane;
#pragma unroll
    for (int i = 0; i < kA; i++) {
      const unsigned long long k = lanes_max<1, 16>(cx.best[i]);
      const int m = kMfma ? (lane >> 4) + 4 * i : i;
      if ((lane & 15) == 0 && (kMfma || lane == 0) && m < M && k != 0ull) key_max(keys + m, k);
      cx.best[i] = 0ull;
    }
  }

  // Inlined into the kernel on purpose: the job table pointer below is the
  // address of the kernel argument in the constant (kernarg) address space,
  // which a by-reference copy on the stack would not be.
  // kAll: jobs may use every format; else only the 4- and 5-bit group-32
  // ones (a kernel with fewer paths, so fewer registers)
  template <bool kAll>
  static __device__ __forceinline__ void run(const SweepArgs& args, uint8_t* xs) {
    Ctx cx;
    cx.D = job_table(args);
    cx.counters = args.counters;
    cx.slots = args.slots;
    cx.q = args.q;
    cx.rem = args.rem;
    cx.G = args.nwaves;
    cx.slot_rows = args.slot_rows;
    cx.lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane lets the compiler know it
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    cx.gw = (int)blockIdx.x * kStreamWavesPerBlock + wave;
    if (cx.gw >= cx.G) return;
    cx.a = start_of(cx.gw, cx.q, cx.rem);
    cx.b = cx.a + cx.q + (cx.gw < cx.rem ? 1 : 0);
    cx.pend_j0 = cx.pend_j1 = -1;
    cx.pend_rg0 = cx.pend_rg1 = 0;
#pragma unroll
    for (int i = 0; i < kA; i++) cx.best[i] = 0ull;
    // first job of the range: a bucket index into the uend list when the jobs
    // come from a table, else a scan of the (at most 12) inline jobs
    int j = 0;
    if (args.index) {
      const QG_CONST int32_t* ends = (const QG_CONST int32_t*)args.index;
      j = ends[args.njobs + (cx.a >> args.bshift)];
      while (cx.a >= ends[j]) j++;
    } else {
      while (cx.a >= cx.D[j].uend) j++;
    }
    // one segment per job the range touches
    // one segment per job the range touches: the job's steps whose first
    // unit lies in the range
    for (int f = cx.a; f < cx.b; j++) {
      const int ub = cx.D[j].ubeg;
      const int e = cx.D[j].uend < cx.b ? cx.D[j].uend : cx.b;
      const int fmt = cx.D[j].fmt;
      if (fmt == kFmtQ4) segment_in<kFmtQ4>(cx, j, f - ub, e - ub, xs);
      else if (!kAll || fmt == kFmtQ5) segment_in<kFmtQ5>(cx, j, f - ub, e - ub, xs);
      else if (fmt == kFmtG64) segment_in<kFmtG64>(cx, j, f - ub, e - ub, xs);
      else segment_in<kFmtZP>(cx, j, f - ub, e - ub, xs);
      f = e;
    }
    if (cx.pend_j0 >= 0 || cx.pend_j1 >= 0) {
      // every slot store of this wave must be complete before any arrival;
      // both arrivals are counted before either result is waited for
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      arrive(cx);
    }
  }
};

template <bool kMfma, int kCap, bool kAll, bool kBig>
__global__ void __launch_bounds__(64 * kStreamWavesPerBlock) stream_kernel(SweepArgs args) {
  using S = Stream<kMfma, kCap, kBig>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kStreamWavesPerBlock][kMfma ? 16 : kCap * kXRowBytes];
  S::template run<kAll>(args, xs[threadIdx.x >> 6]);
}

// --------------------------------------------------------------------------
// group kernel: panels of 17..64 rows (MFMA, 2..4 m blocks)
// --------------------------------------------------------------------------
// One workgroup of kW waves per unit = (job, kW * kRG row blocks), whole K:
// no K split, so no partial sums cross waves.  The waves walk the k tiles in
// lockstep, one barrier per k tile.  The X chunk of a k tile (kMPad rows x 128
// k) is copied once per workgroup straight from memory into LDS (direct-to-LDS
// loads, no registers), into a ring of kDepth buffers; each wave reads its
// MFMA A fragments for the tile once and applies them to its kRG row blocks,
// so LDS traffic per weight byte falls kRG-fold.  The X copy of tile t is
// issued just before the weight loads of tile t, kDepth tiles ahead, so
// waiting for it never waits on a younger weight load.  Units are handed out
// in job order, one round of the grid at a time in alternating directions;
// the host orders jobs longest K first.
//
// LDS layout of one buffer: 16-byte slot s (X chunk col' of row s / 16,
// col' = s mod 16) holds X[row][8 col .. 8 col + 7] of the k tile with col =
// col' XOR (row mod 16), so the 16 rows an A-fragment read touches fall on
// distinct banks.  Slots past kMPad rows are a landing area for the copies of
// waves with no rows left (every wave issues the same number of copies, which
// keeps the wait counts exact).
// Global memory straight into LDS: 16 (or 4) bytes per lane at dst + 16 *
// lane (dst + 4 * lane); dst is wave-uniform and goes to M0.  Written as
// assembly so the compiler neither tracks nor waits for these copies: the
// group kernel covers them with its own explicit waits (a copy issued before a
// load has completed once that load has).  The compiler's wait counts for its
// own loads are then only ever too strict.  The nop covers the M0-write hazard
// of LDS-direct loads.  M0 is a register the compiler reserves, so the
// sequence saves and restores it.
__device__ __forceinline__ void lds_copy16(const void* src, uint32_t dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(dst)
      : "memory");
}
__device__ __forceinline__ void lds_copy4(const void* src, uint32_t dst) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(dst)
      : "memory");
}

template <int kMPad>
struct Group {
  static constexpr int kW = group_waves(kMPad);
  static constexpr int kMb = kMPad / 16;
  static constexpr int kThreads = 64 * kW;
  static constexpr int kRG = kGroupRows;                             // row blocks per wave
  static_assert(kRG == 2, "one 64-lane scale copy holds the scales of two row blocks");
  static constexpr int kDepth = 4;                                    // code prefetch distance, k tiles
  static constexpr int kBufs = kDepth;                                // ring of k-tile buffers in LDS:
                                                                      // X and scales go kDepth - 1 ahead
  static constexpr int kND = (kMPad * 16 + kThreads - 1) / kThreads;  // X copies per wave and k tile
  static constexpr int kXBytes = kND * kThreads * 16;                 // X area of a buffer
  static constexpr int kBufBytes = kXBytes + kW * 256;                // then 256 scale bytes per wave
  static constexpr int kYRow = kRG * kTileRows;                       // outputs n of a wave
  static_assert(kND * kThreads >= kMPad * 16, "X copies cover the panel");
  static constexpr int kYBytes = kW * kMPad * kYRow * 4;             // output staging (reuses the ring)
  static constexpr int kRingBytes = kBufs * kBufBytes > kYBytes ? kBufs * kBufBytes : kYBytes;
  static constexpr int kLdsBytes = kRingBytes + kMPad * 8;           // then one argmax key per row

  template <int F>
  static constexpr bool kSide = F == kFmtQ5 || F == kFmtZP;   // a side word per row block
  template <int F>
  struct Tiles {
    u4_t c[kRG];
    uint32_t h[kSide<F> ? kRG : 1];
  };
  // vector memory instructions of one k tile per wave: X copies, the scale
  // copy, then the weight loads
  template <int F>
  static constexpr int kLoadsW = kRG * (kSide<F> ? 2 : 1);
  template <int F>
  static constexpr int kLoadsTile = kND + 1 + kLoadsW<F>;

  // Direct-to-LDS copy of this wave's X slots of k tile kt (clamped to the
  // last) into the buffer at LDS address buf.  Slot rows past M repeat row
  // M-1 and k is clamped into the row (padding groups then add exact zeros:
  // their codes are 0).
  static __device__ __forceinline__ void copy_x(const JobDesc& d, int kt, uint32_t buf, int wave, int lane) {
    kt = kt < d.nkt ? kt : d.nkt - 1;
#pragma unroll
    for (int i = 0; i < kND; i++) {
      const int s = 64 * (wave * kND + i) + lane;
      const int row = s >> 4;
      const int col = (s & 15) ^ (row & 15);
      const int m = row < d.M ? row : d.M - 1;
      const int kk = kt * kTileK + 8 * col;
      const int k = kk < d.K - 8 ? kk : d.K - 8;
      lds_copy16(d.X + (int64_t)m * d.ldx + k, buf + 1024u * (uint32_t)(wave * kND + i));
    }
  }

  // The code loads of one tile per row block as raw buffer loads over that
  // tile alone (non-temporal).  A tile past the job's last (the prefetch
  // running ahead of the final tiles) gets a zero-length range: its loads
  // return zeros without touching memory but still count for the waits.
  static constexpr int kNt = 2;  // cache policy: non-temporal
  template <int F>
  static __device__ __forceinline__ void load_w(Tiles<F>& t, const uint8_t* w0, int64_t rstride,
                                                int nrows, int len, int lane) {
#pragma unroll
    for (int r = 0; r < kRG; r++) {
      const uint8_t* tp = w0 + (int64_t)(r < nrows ? r : nrows - 1) * rstride;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)tp, (short)0, len, kBufWord3);
      t.c[r] = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, kNt));
      if constexpr (F == kFmtQ5) t.h[r] = __builtin_amdgcn_raw_buffer_load_b32(rs, kHiOff + 4 * lane, 0, kNt);
      if constexpr (F == kFmtZP) t.h[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, kZeroOff + 2 * (lane & 15), 0, kNt);
    }
  }

  // Copies of k tile kx (clamped to the last) into ring buffer slot, then
  // the code loads of k tile kw into t, in the order the wait counts assume
  // (the scheduling barriers keep it): X, this wave's scales, codes.  The
  // scale copy puts row r's four scales of both row blocks side by side (16
  // bytes per row): lane l copies word l & 1 of row l >> 2, row block
  // (l >> 1) & 1, whose offset from the tile is soff.
  template <int F>
  static __device__ __forceinline__ void copies(const JobDesc& d, int kx, uint32_t buf, const uint8_t* wbase,
                                                uint32_t soff, int wave, int lane) {
    constexpr int TB = tile_bytes(F);
    const uint8_t* tile = wbase + (int64_t)(kx < d.nkt ? kx : d.nkt - 1) * TB;
    copy_x(d, kx, buf, wave, lane);
    lds_copy4(tile + soff, buf + (uint32_t)(kXBytes + 256 * wave));
  }
  template <int F>
  static __device__ __forceinline__ void codes(const JobDesc& d, int kw, Tiles<F>& t, const uint8_t* wbase,
                                               int64_t rstride, int nrows, int lane) {
    constexpr int TB = tile_bytes(F);
    load_w<F>(t, wbase + (int64_t)(kw < d.nkt ? kw : d.nkt - 1) * TB, rstride, nrows, kw < d.nkt ? TB : 0, lane);
  }

  // One unit: row blocks rb0 + kRG * wave + r (r < kRG) of job d, all k tiles.
  template <int F>
  static __device__ void run_unit(const JobDesc& d, int rb0, uint8_t* xs, uint32_t xs_lds, int tid) {
    constexpr int TB = tile_bytes(F);
    // Issue order: codes of tile 0, then per tile t (the prologue for
    // t < kDepth - 1, else the end of tile t - kDepth + 1): copies of tile t,
    // codes of tile t + 1.  The copies of tile kt are therefore complete once
    // at most this many younger loads of this wave are outstanding: the codes
    // of tile kt + 1 and kDepth - 2 whole tiles.
    constexpr int kXWait = kLoadsW<F> + (kDepth - 2) * kLoadsTile<F>;
    static_assert(kXWait < 64, "vmcnt range");
    // s_waitcnt encoding (gfx9): vmcnt low 4 bits, expcnt 7, lgkmcnt 15, vmcnt high 2 bits
    constexpr int kXWaitImm = (kXWait & 15) | (7 << 4) | (15 << 8) | ((kXWait >> 4) << 14);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nkt = d.nkt;
    const int64_t rstride = (int64_t)nkt * TB;
    const int rbw = rb0 + kRG * wave;                  // this wave's first row block
    const int nrows = d.nrb - rbw;                     // valid row blocks (may be <= 0)
    const int rbl = nrows > 0 ? rbw : d.nrb - 1;       // waves past the job re-read its last block
    const int nr = nrows > 0 ? nrows : 1;
    const uint8_t* wbase = d.packed + (int64_t)rbl * rstride;
    const int srb = ((lane >> 1) & 1) < nr ? (lane >> 1) & 1 : nr - 1;
    // group 64: a row's two scales are one word, which both lanes of the
    // pair copy (so words 0 and 1 of a row block are the same)
    const uint32_t soff = (uint32_t)(srb * rstride) +
                          (uint32_t)(F == kFmtG64 ? kScaleOff + 4 * (lane >> 2)
                                                  : kScaleOff + 8 * (lane >> 2) + 4 * (lane & 1));
    Tiles<F> buf[kDepth];
    __builtin_amdgcn_sched_barrier(0);
    codes<F>(d, 0, buf[0], wbase, rstride, nr, lane);
#pragma unroll
    for (int p = 0; p < kDepth - 1; p++) {
      __builtin_amdgcn_sched_barrier(0);
      copies<F>(d, p, xs_lds + (uint32_t)(p * kBufBytes), wbase, soff, wave, lane);
      __builtin_amdgcn_sched_barrier(0);
      codes<F>(d, p + 1, buf[p + 1], wbase, rstride, nr, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    f4_t acc[kRG][kMb];
#pragma unroll
    for (int r = 0; r < kRG; r++)
#pragma unroll
      for (int mb = 0; mb < kMb; mb++) acc[r][mb] = f4_t{0.f, 0.f, 0.f, 0.f};
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    // A fragment of group j, m block mb: row 16 mb + (lane mod 16), chunk
    // 4 j + lane / 16, at its swizzled slot
    const int mr = lane & 15, c = lane >> 4;
    uint32_t aoff[4];
#pragma unroll
    for (int j = 0; j < 4; j++) aoff[j] = (uint32_t)(256 * mr + 16 * ((4 * j + c) ^ mr));
    const uint32_t sread = (uint32_t)(kXBytes + 256 * wave + 16 * mr);
    for (int kt0 = 0; kt0 < nkt; kt0 += kDepth) {
#pragma unroll
      for (int p = 0; p < kDepth; p++) {
        const int kt = kt0 + p;
        if (kt < nkt) {
          // this wave's copies of tile kt have landed; after the barrier every
          // wave's have, and every wave is done with tile kt - 1
          __builtin_amdgcn_s_waitcnt(kXWaitImm);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_s_barrier();
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          const uint8_t* xb = xs + p * kBufBytes;
          // scales of row mr: words 0, 1 of row block 0, then of row block 1
          const u4_t sc = *(const u4_t*)(xb + sread);
          f4_t pr[kRG][kMb];
          // group by group: the A fragments of group j serve all kRG row blocks
#pragma unroll
          for (int j = 0; j < 4; j++) {
            h8_t a[kMb];
#pragma unroll
            for (int mb = 0; mb < kMb; mb++) a[mb] = lds_h8(xb + aoff[j] + 4096 * mb);
            // every MFMA of the group is issued before the first of its
            // results is scaled, so the matrix-core latency overlaps
            // group 64: the odd half of a group accumulates onto the even
            // half's products, which are scaled once, after it
            constexpr bool kG64 = F == kFmtG64;
#pragma unroll
            for (int r = 0; r < kRG; r++) {
              const h8_t q = unpack_chunk<F>(buf[p].c[r][j], side_word<F>(buf[p].h[kSide<F> ? r : 0]), j);
#pragma unroll
              for (int mb = 0; mb < kMb; mb++)
                pr[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], q, (kG64 && (j & 1)) ? pr[r][mb] : zero, 0, 0, 0);
            }
            if (!kG64 || (j & 1)) {
#pragma unroll
              for (int r = 0; r < kRG; r++) {
                // group 32: word j / 2 of the row block holds groups (j & ~1, j | 1);
                // group 64: word 0 holds halves (0, 1)
                const uint32_t sp = sc[2 * r + (kG64 ? 0 : j >> 1)];
                const int hi = kG64 ? j >> 1 : j & 1;
                const float sj = hi ? scale_f32<1>(sp) : scale_f32<0>(sp);
#pragma unroll
                for (int mb = 0; mb < kMb; mb++)
#pragma unroll
                  for (int i = 0; i < 4; i++) acc[r][mb][i] = __builtin_fmaf(sj, pr[r][mb][i], acc[r][mb][i]);
              }
            }
          }
        }
        // copies of tile kt + kDepth - 1 into the buffer of tile kt - 1 (every
        // wave is past it), codes of tile kt + kDepth.  Past the last k tile
        // they (kept for exact wait counts) re-read the last tile into
        // buffers no wave reads again.
        __builtin_amdgcn_sched_barrier(0);
        copies<F>(d, kt + kDepth - 1, xs_lds + (uint32_t)(((p + kDepth - 1) % kBufs) * kBufBytes), wbase, soff,
                  wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        codes<F>(d, kt + kDepth, buf[p], wbase, rstride, nr, lane);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every copy has landed and every wave is done with the ring
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    __syncthreads();
    unsigned long long* best = (unsigned long long*)(xs + kRingBytes);
    if (nrows > 0) store_y(d, acc, rbw, xs + kMPad * kYRow * 4 * wave, best, lane);
    // the ring is free for the next unit's copies; the unit's argmax keys are
    // complete and go to the job's keys
    __syncthreads();
    if (d.keys && tid < d.M) {
      const unsigned long long k = best[tid];
      if (k != 0ull) key_max(d.keys + (blockIdx.x % kKeyCopies) * kKeyRows + tid, k);
      best[tid] = 0ull;
    }
  }

  // The wave's outputs (rows m < kMPad, n = 16 rbw .. 16 rbw + 31) go through
  // its slice of the LDS ring, row-major with 16-byte chunks swizzled by
  // m mod 8, and leave as whole 128-byte row segments: lane L of store t
  // writes row 8 t + L / 8, outputs 4 (L mod 8) .. + 3.
  static __device__ __forceinline__ void store_y(const JobDesc& d, const f4_t (&acc)[kRG][kMb], int rbw,
                                                 uint8_t* st, unsigned long long* best, int lane) {
    const int mr = lane & 15, c = lane >> 4;
#pragma unroll
    for (int r = 0; r < kRG; r++)
#pragma unroll
      for (int mb = 0; mb < kMb; mb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = 16 * mb + 4 * c + i, n = 16 * r + mr;
          *(float*)(st + 128 * m + 16 * ((n >> 2) ^ (m & 7)) + 4 * (n & 3)) = acc[r][mb][i];
        }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    QG_GLOBAL float* Y = (QG_GLOBAL float*)d.Y;
    const int n0 = kTileRows * rbw + 4 * (lane & 7);
#pragma unroll
    for (int t = 0; t < kMPad / 8; t++) {
      const int m = 8 * t + (lane >> 3);
      const f4_t v = *(const f4_t*)(st + 128 * m + 16 * ((lane & 7) ^ (m & 7)));
      if (m < d.M && Y) {
        QG_GLOBAL float* y = Y + (int64_t)m * d.ldy + n0;
        if (n0 + 3 < d.N) {
          *(QG_GLOBAL f4_t*)y = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; e++)
            if (n0 + e < d.N) y[e] = v[e];
        }
      }
      if (d.keys) {
        // verify head: the best of the row's 32 outputs (8 lanes), into the
        // workgroup's key of row m
        unsigned long long k = 0ull;
#pragma unroll
        for (int e = 0; e < 4; e++)
          if (n0 + e < d.N) k = umax64(k, logit_key(v[e], n0 + e));
        k = lanes_max<1, 8>(k);
        if ((lane & 7) == 0 && m < d.M && k != 0ull)
          __hip_atomic_fetch_max(best + m, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  }
};

template <int kMPad, bool kAll>
__global__ void __launch_bounds__(64 * group_waves(kMPad)) __attribute__((amdgpu_waves_per_eu(kMPad >= 64 ? 2 : 3)))
group_kernel(SweepArgs args) {
  using S = Group<kMPad>;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[S::kLdsBytes];
  const uint32_t xs_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)xs;
  const QG_CONST JobDesc* D = job_table(args);
  const int tid = threadIdx.x;
  // argmax keys of the verify head start at 0 (the first unit's barriers
  // order this before any use)
  if (tid < kMPad) ((unsigned long long*)(xs + S::kRingBytes))[tid] = 0ull;
  int j = 0;
  // round i of the grid takes units [i G, (i + 1) G) in alternating
  // directions, so the longest-first order evens out across workgroups
  const int G = (int)gridDim.x, b = (int)blockIdx.x;
  for (int i = 0;; i++) {
    const int u = i * G + ((i & 1) ? G - 1 - b : b);
    if (u >= args.total) break;
    while (u >= D[j].grp_end) j++;
    const JobDesc d = D[j];
    const int rb0 = (u - d.grp_begin) * S::kW * kGroupRows;
    if (d.fmt == kFmtQ4) S::template run_unit<kFmtQ4>(d, rb0, xs, xs_lds, tid);
    else if (!kAll || d.fmt == kFmtQ5) S::template run_unit<kFmtQ5>(d, rb0, xs, xs_lds, tid);
    else if (d.fmt == kFmtG64) S::template run_unit<kFmtG64>(d, rb0, xs, xs_lds, tid);
    else S::template run_unit<kFmtZP>(d, rb0, xs, xs_lds, tid);
  }
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

// kind: 0 = stream GEMV (cls = rows 1, 2, 4, 8), 1 = stream MFMA (cls 1, 2, 4, 8, 16),
//       2 = group MFMA (cls = padded rows 32, 48, 64); all: some job uses a
//       format other than the 4- and 5-bit group-32 ones
template <bool kAll, bool kBig>
static sweep_fn pick_set(int kind, int cls) {
  if (kind == 0) {
    switch (cls) {
      case 1: return stream_kernel<false, 1, kAll, false>;
      case 2: return stream_kernel<false, 2, kAll, false>;
      case 4: return stream_kernel<false, 4, kAll, false>;
      case 8: return stream_kernel<false, 8, kAll, false>;
    }
  } else if (kind == 1) {
    switch (cls) {
      case 1: return stream_kernel<true, 1, kAll, kBig>;
      case 2: return stream_kernel<true, 2, kAll, kBig>;
      case 4: return stream_kernel<true, 4, kAll, kBig>;
      case 8: return stream_kernel<true, 8, kAll, kBig>;
      case 16: return stream_kernel<true, 16, kAll, kBig>;
    }
  } else {
    switch (cls) {
      case 32: return group_kernel<32, kAll>;
      case 48: return group_kernel<48, kAll>;
      case 64: return group_kernel<64, kAll>;
    }
  }
  return nullptr;
}
// big: the MFMA stream kernel with eight-block steps (GEMV and group kernels
// have one step shape)
static sweep_fn pick(int kind, int cls, bool all, bool big) {
  if (big) return all ? pick_set<true, true>(kind, cls) : pick_set<false, true>(kind, cls);
  return all ? pick_set<true, false>(kind, cls) : pick_set<false, false>(kind, cls);
}

int sweep_threads(int kind, int cls) { return kind == 2 ? 64 * group_waves(cls) : 64 * kStreamWavesPerBlock; }

int sweep_blocks_per_cu(int kind, int cls, bool all) {
  sweep_fn f = pick(kind, cls, all, false);
  if (!f) return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)f, sweep_threads(kind, cls), 0) != hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_sweep(int kind, int cls, bool all, bool big, const SweepArgs& args, int grid, hipStream_t stream) {
  if (big && kind != 1) return hipErrorInvalidValue;
  sweep_fn f = pick(kind, cls, all, big);
  if (!f) return hipErrorInvalidValue;
  hipLaunchKernelGGL(f, dim3(grid), dim3(sweep_threads(kind, cls)), 0, stream, args);
  return hipGetLastError();
}

}  // namespace qg
