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

// One thread per (row n of the padded grid, k tile): quantizes the tile's four
// groups of that row and writes its 4 x 16 code bytes, 8 scale bytes and (5-bit)
// 4 x 4 high-bit bytes.  No two threads write the same byte.
template <int BITS>
__global__ void __launch_bounds__(256) pack_kernel(const float* __restrict__ W, int64_t ldw, int N,
                                                   int K, int nkt, int64_t total,
                                                   uint8_t* __restrict__ packed,
                                                   unsigned* __restrict__ flag) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int n = (int)(idx / nkt), kt = (int)(idx % nkt);
  const int r = n & 15;
  const int qmax = (1 << (BITS - 1)) - 1, bias = 1 << (BITS - 1);
  const int G = K / kGroup;
  uint8_t* tile = packed + ((int64_t)(n >> 4) * nkt + kt) * (BITS == 4 ? kTile4 : kTile5);
  uint32_t code[4][4];
  uint32_t hi[4] = {0, 0, 0, 0};
  uint16_t sc[4];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int g = 4 * kt + j;
    int u[32];
    uint16_t sb = 0;
    if (n < N && g < G) {
      const float* w = W + (int64_t)n * ldw + (int64_t)g * kGroup;
      float v[32];
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < 32; t++) {
        v[t] = w[t];
        if (!isfinite(v[t])) bad = true;
        amax = fmaxf(amax, fabsf(v[t]));
      }
      sb = f64_to_f16_bits((double)amax / (double)qmax);
      if ((sb & 0x7c00u) == 0x7c00u) bad = true;
      const double s = (double)__builtin_bit_cast(_Float16, sb);
#pragma unroll
      for (int t = 0; t < 32; t++) {
        int q = 0;
        if (s != 0.0 && isfinite(v[t]) && isfinite(s)) {
          double qq = rint((double)v[t] / s);
          qq = fmin(fmax(qq, (double)-qmax), (double)qmax);
          q = (int)qq;
        }
        u[t] = q + bias;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 32; t++) u[t] = bias;
    }
    sc[j] = sb;
#pragma unroll
    for (int c = 0; c < 4; c++) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        const int uu = u[8 * c + e];
        word |= (uint32_t)(uu & 15) << (4 * (e >> 1) + 16 * (e & 1));
        if (BITS == 5) hi[c] |= (uint32_t)((uu >> 4) & 1) << ((4 + 16 * (e & 1) + 4 * j + (e >> 1)) & 31);
      }
      code[c][j] = word;
    }
  }
#pragma unroll
  for (int c = 0; c < 4; c++) {
    u4_t v = {code[c][0], code[c][1], code[c][2], code[c][3]};
    *(u4_t*)(tile + 16 * (r + 16 * c)) = v;
    if (BITS == 5) *(uint32_t*)(tile + kHiOff + 4 * (r + 16 * c)) = hi[c];
  }
  u2_t s2 = {(uint32_t)sc[0] | ((uint32_t)sc[1] << 16), (uint32_t)sc[2] | ((uint32_t)sc[3] << 16)};
  *(u2_t*)(tile + kScaleOff + 8 * r) = s2;
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

template <typename T>
__device__ __forceinline__ const QG_GLOBAL T* gload_ptr(const void* p) {
  return (const QG_GLOBAL T*)p;
}

// Eight codes of one group chunk -> four fp16 pairs holding the exact q.
template <int BITS>
__device__ __forceinline__ h8_t unpack_chunk(uint32_t w, uint32_t hi, int j) {
  constexpr uint32_t kMagic = 0x64006400u;                       // (1024.0, 1024.0)
  constexpr _Float16 kOff = (_Float16)(1024 + (1 << (BITS - 1)));
  const h2_t off = {kOff, kOff};
  h8_t out;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    uint32_t t = ((w >> (4 * i)) & 0x000F000Fu) | kMagic;
    if (BITS == 5) {
      const int s = 4 * j + i;  // rotate right: bits (4+s, 20+s) of hi -> bits (4, 20)
      const uint32_t rot = (hi >> s) | (hi << ((32 - s) & 31));
      t |= rot & 0x00100010u;
    }
    const h2_t q = __builtin_bit_cast(h2_t, t) - off;
    out[2 * i] = q.x;
    out[2 * i + 1] = q.y;
  }
  return out;
}

// The weight part of one k tile as seen by lane l = r + 16c: its 16 code
// bytes (chunk c of the tile's four groups of row r), the four fp16 scales of
// row r, and (5-bit) the 32 high bits of its codes.
struct WRegs {
  u4_t wc;
  u2_t ws;
  uint32_t wh;
};

// Every tile issues the same three loads whatever its bit width (a 4-bit tile
// re-reads a word of its own scale block in place of the high bits), so the
// compiler can count outstanding loads exactly and never has to drain them.
__device__ __forceinline__ void load_w(WRegs& t, const uint8_t* tile, int bits, int lane) {
  t.wc = __builtin_nontemporal_load(gload_ptr<u4_t>(tile + 16 * lane));
  t.ws = __builtin_nontemporal_load(gload_ptr<u2_t>(tile + kScaleOff + 8 * (lane & 15)));
  const int hoff = bits == 5 ? kHiOff + 4 * lane : kScaleOff + 4 * (lane & 31);
  t.wh = __builtin_nontemporal_load(gload_ptr<uint32_t>(tile + hoff));  // unused when 4-bit
}

// One 16-byte piece of an X chunk.  Outside [0,M) x [0,K) it reads row 0, k 0
// (always valid) and the value is never used: rows m >= M only feed output
// rows that are not stored (MFMA rows are independent) and k >= K lies in
// groups the tile loop skips.  No select on the loaded value, so the load
// need not complete before the next ones are issued.
__device__ __forceinline__ u4_t load_x_piece(const uint16_t* X, int64_t ldx, int row, int k, int M, int K) {
  const bool ok = row < M && k < K;
  return *gload_ptr<u4_t>(X + (ok ? (int64_t)row * ldx + k : 0));
}

// X chunks are written to and read from LDS as the same 16-byte integer
// vector type (then bit-cast), so type-based alias analysis can never move a
// read above the write that produced it.
__device__ __forceinline__ h8_t lds_h8(const uint8_t* p) { return __builtin_bit_cast(h8_t, *(const u4_t*)p); }

// Two fp16 scales from one 32-bit word.  The word is taken by value: a
// bit_cast applied directly to an element of a vector register type was
// compiled to an undefined value (only element 0 survived).
__device__ __forceinline__ h2_t scale_pair(uint32_t word) { return __builtin_bit_cast(h2_t, word); }

// MFMA:  v_mfma_f32_16x16x32_f16, A = X (16 rows m x 32 k of one group),
//        B = codes (32 k x 16 rows n).  Lane l holds for A row m = l%16 and for
//        B row n = l%16, both k chunk l/16 of the same group; D lane l holds
//        (n = l%16, m = 4*(l/16) + i).  The group's fp32 scale multiplies the
//        16x16 partial before it is added to the accumulator.
template <int BITS, int MB>
__device__ __forceinline__ void mfma_tile(f4_t (&acc)[MB], const WRegs& w, const uint8_t* xs, int lane,
                                          int gleft) {
  const int r = lane & 15, c = lane >> 4;
  const h2_t s01 = scale_pair(w.ws.x), s23 = scale_pair(w.ws.y);
  const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (j < gleft) {
      const h8_t q = unpack_chunk<BITS>(w.wc[j], w.wh, j);
      const f4_t zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mb = 0; mb < MB; mb++) {
        const h8_t a = lds_h8(xs + (16 * mb + r) * kXRowBytes + 64 * j + 16 * c);
        const f4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q, zero, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; i++) acc[mb][i] = __builtin_fmaf(sc[j], p[i], acc[mb][i]);
      }
    }
  }
}

// GEMV: per lane and row m, four v_dot2_f32_f16 over the lane's 8 codes of a
// group, scaled by the group's scale; the four k chunks of a row (lanes r,
// r+16, r+32, r+48) are summed when the row block is flushed.
template <int BITS, int GM>
__device__ __forceinline__ void gemv_tile(float (&acc)[GM], const WRegs& w, const uint8_t* xs, int lane,
                                          int gleft, int M) {
  const int c = lane >> 4;
  const h2_t s01 = scale_pair(w.ws.x), s23 = scale_pair(w.ws.y);
  const float sc[4] = {(float)s01.x, (float)s01.y, (float)s23.x, (float)s23.y};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (j < gleft) {
      const h8_t q = unpack_chunk<BITS>(w.wc[j], w.wh, j);
      const h2_t q0 = {q[0], q[1]}, q1 = {q[2], q[3]}, q2 = {q[4], q[5]}, q3 = {q[6], q[7]};
#pragma unroll
      for (int m = 0; m < GM; m++) {
        if (m < M) {
          const h8_t x = lds_h8(xs + m * kXRowBytes + 64 * j + 16 * c);
          const h2_t x0 = {x[0], x[1]}, x1 = {x[2], x[3]}, x2 = {x[4], x[5]}, x3 = {x[6], x[7]};
          float d = __builtin_amdgcn_fdot2(q0, x0, 0.f, false);
          d = __builtin_amdgcn_fdot2(q1, x1, d, false);
          d = __builtin_amdgcn_fdot2(q2, x2, d, false);
          d = __builtin_amdgcn_fdot2(q3, x3, d, false);
          acc[m] = __builtin_fmaf(sc[j], d, acc[m]);
        }
      }
    }
  }
}

__device__ __forceinline__ const QG_CONST JobDesc* job_table(const SweepArgs& a) {
  return a.table ? (const QG_CONST JobDesc*)a.table : (const QG_CONST JobDesc*)&a.inl[0];
}

// --------------------------------------------------------------------------
// stream kernel: panels of at most 16 rows (GEMV, or MFMA with one m block)
// --------------------------------------------------------------------------
// The flat sequence of (job, row block, k tile) tiles is cut into `nwaves`
// equal contiguous ranges, one per wave, so every wave streams the same number
// of tiles.  A wave accumulates one row block at a time; a row block whose
// tiles all lie in one range is written to Y directly.  A row block cut by
// range ends gets one partial sum per contributing wave, stored into that
// wave's slot; the last contributor to arrive (per-row-block counter) adds the
// partials in wave order -- k order -- writes Y and resets the counter to
// zero.  Nothing waits on another wave.  The slots and counters are accessed
// with system-scope atomics: the per-XCD L2 caches are not coherent with each
// other, and system-scope accesses bypass them, so no cache-wide writeback or
// invalidate is needed on either side of the exchange.

// One k tile of the stream kernels.  kRagged: the tile may hold fewer than
// four groups (the last tile of a row when K % 128 != 0).
// MFMA: only the first NF of the lane's four accumulator rows are scaled and
// kept (rows 4*(l/16)+i, i < NF); panels of at most 4 rows need NF = M.
template <int BITS, int NF, bool kRagged>
__device__ __forceinline__ void mfma1_tile(f4_t& acc, const WRegs& w, const uint8_t* xs, int lane, int gleft) {
  const int r = lane & 15, c = lane >> 4;
  const h2_t s01 = scale_pair(w.ws.x), s23 = scale_pair(w.ws.y);
  const _Float16 sh[4] = {s01.x, s01.y, s23.x, s23.y};
  const f4_t zero = {0.f, 0.f, 0.f, 0.f};
  // all four groups' MFMAs are issued before any of their results is read,
  // so the MFMA latency overlaps with independent work instead of stalling
  f4_t p[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (!kRagged || j < gleft) {
      const h8_t q = unpack_chunk<BITS>(w.wc[j], w.wh, j);
      const h8_t a = lds_h8(xs + r * kXRowBytes + 64 * j + 16 * c);
      p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, q, zero, 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (!kRagged || j < gleft) {
      const float sj = (float)sh[j];
#pragma unroll
      for (int i = 0; i < NF; i++) acc[i] = __builtin_fmaf(sj, p[j][i], acc[i]);
    }
  }
}

template <int BITS, int GM, bool kRagged>
__device__ __forceinline__ void gemv1_tile(float (&acc)[GM], const WRegs& w, const uint8_t* xs, int lane,
                                           int gleft, int M) {
  const int c = lane >> 4;
  const h2_t s01 = scale_pair(w.ws.x), s23 = scale_pair(w.ws.y);
  const _Float16 sh[4] = {s01.x, s01.y, s23.x, s23.y};
#pragma unroll
  for (int j = 0; j < 4; j++) {
    if (!kRagged || j < gleft) {
      const h8_t q = unpack_chunk<BITS>(w.wc[j], w.wh, j);
      const h2_t q0 = {q[0], q[1]}, q1 = {q[2], q[3]}, q2 = {q[4], q[5]}, q3 = {q[6], q[7]};
      const float sj = (float)sh[j];
#pragma unroll
      for (int m = 0; m < GM; m++) {
        if (m < M) {
          const h8_t x = lds_h8(xs + m * kXRowBytes + 64 * j + 16 * c);
          const h2_t x0 = {x[0], x[1]}, x1 = {x[2], x[3]}, x2 = {x[4], x[5]}, x3 = {x[6], x[7]};
          float d = __builtin_amdgcn_fdot2(q0, x0, 0.f, false);
          d = __builtin_amdgcn_fdot2(q1, x1, d, false);
          d = __builtin_amdgcn_fdot2(q2, x2, d, false);
          d = __builtin_amdgcn_fdot2(q3, x3, d, false);
          acc[m] = __builtin_fmaf(sj, d, acc[m]);
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// stream kernel: panels of at most 16 rows (GEMV, or MFMA with one m block)
// --------------------------------------------------------------------------
// The flat sequence of (job, row block, k tile) tiles is cut into `nwaves`
// equal contiguous ranges, one per wave, so every wave streams the same number
// of tiles.  Within one job a wave's tiles are contiguous in memory (tile
// index rb * NKT + kt), so the weight pointer simply advances.  A wave
// accumulates one row block at a time; a row block whose tiles all lie in one
// range is written to Y directly.  A row block cut by range ends gets one
// partial sum per contributing wave, stored into that wave's slot; the last
// contributor to arrive (per-row-block counter) adds the partials in wave
// order -- k order -- writes Y and resets the counter to zero.  Nothing waits
// on another wave.  The slots and counters are accessed with system-scope
// atomics, which bypass the per-XCD L2 caches (not coherent with each other).
template <bool kMfma, int kCap>
struct Stream {
  static constexpr int kRows = kMfma ? 16 : kCap;                 // X rows staged in LDS
  static constexpr int kLoadRows = kCap;                          // X rows loaded per tile
  static constexpr int kPieces = (kLoadRows * 16 + 63) / 64;      // 16-byte X pieces per lane
  static constexpr int kNF = kCap < 4 ? kCap : 4;                 // MFMA accumulator rows kept
  // tiles in flight per wave (fewer where the panel's registers need room);
  // 2048..4096 waves x depth x 1.15 KB keeps >= ~16 MB of reads in flight
  static constexpr int kDepth = kCap <= 2 ? 8 : kCap == 4 ? 6 : kCap == 8 ? (kMfma ? 4 : 2) : 3;

  struct Regs {
    WRegs w;
    u4_t x[kPieces];
  };

  struct Acc {
    f4_t mf;
    float gv[kCap];
  };

  static __device__ __forceinline__ void zero(Acc& a) {
    a.mf = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < kCap; m++) a.gv[m] = 0.f;
  }

  static __device__ __forceinline__ int64_t wave_of(int64_t f, int64_t T, int64_t G) {
    const int64_t w = ((f + 1) * G - 1) / T;
    return w < G - 1 ? w : G - 1;
  }

  // Everything a wave needs to place one row block's sums.
  struct Ctx {
    const QG_CONST JobDesc* D;
    int* counters;
    float* slots;
    int64_t T, G;          // flat tiles, waves
    int slot_rows;
    int64_t gw, a, b;
    int lane;
    // split row blocks whose partial this wave stored (kind 0 / kind 1)
    int pend_j0, pend_rb0, pend_j1, pend_rb1;
  };

  // Write the finished sums of row block rb of job j to Y, or, for a row
  // block cut by this wave's range, store this wave's partial into its slot
  // (kind 0: the range's first row block, kind 1: its last) and note it; the
  // arrival is counted once, at the end of the range (see arrive), so the
  // stream never stalls on it.
  static __device__ __forceinline__ void flush(Acc acc, Ctx& cx, int j, int rb) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    const int M = D[j].M, N = D[j].N, nkt = D[j].nkt;
    const int64_t ldy = D[j].ldy;
    QG_GLOBAL float* Y = (QG_GLOBAL float*)D[j].Y;
    if constexpr (!kMfma) {
#pragma unroll
      for (int m = 0; m < kCap; m++) {
        float v = acc.gv[m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        acc.gv[m] = v;
      }
    }
    const int64_t first = D[j].tile_begin + (int64_t)rb * nkt;
    const int64_t last = first + nkt - 1;
    const int nn = lane & 15;
    const int n = rb * kTileRows + nn;
    if (first >= cx.a && last < cx.b) {
      if (n < N) {
        if constexpr (kMfma) {
#pragma unroll
          for (int i = 0; i < kNF; i++) {
            const int m = 4 * (lane >> 4) + i;
            if (m < M) Y[(int64_t)m * ldy + n] = acc.mf[i];
          }
        } else if (lane < 16) {
#pragma unroll
          for (int m = 0; m < kCap; m++)
            if (m < M) Y[(int64_t)m * ldy + n] = acc.gv[m];
        }
      }
      return;
    }
    const int slot_floats = cx.slot_rows * kTileRows;
    const int kind = cx.a >= first ? 0 : 1;
    float* mine = cx.slots + (cx.gw * 2 + kind) * slot_floats;
    if constexpr (kMfma) {
#pragma unroll
      for (int i = 0; i < kNF; i++) {
        const int m = 4 * (lane >> 4) + i;
        if (m < M) __hip_atomic_store(mine + m * kTileRows + nn, acc.mf[i], __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_SYSTEM);
      }
    } else if (lane < 16) {
#pragma unroll
      for (int m = 0; m < kCap; m++)
        if (m < M)
          __hip_atomic_store(mine + m * kTileRows + nn, acc.gv[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (kind == 0) {
      cx.pend_j0 = j;
      cx.pend_rb0 = rb;
    } else {
      cx.pend_j1 = j;
      cx.pend_rb1 = rb;
    }
  }

  // Count this wave's arrival at split row block rb of job j (its partial is
  // already stored and complete); the last of its contributors adds all
  // partials in wave order -- k order -- writes Y and resets the counter.
  static __device__ __forceinline__ void arrive(const Ctx& cx, int j, int rb) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    const int M = D[j].M, N = D[j].N, nkt = D[j].nkt;
    const int64_t ldy = D[j].ldy;
    QG_GLOBAL float* Y = (QG_GLOBAL float*)D[j].Y;
    const int64_t first = D[j].tile_begin + (int64_t)rb * nkt;
    const int64_t last = first + nkt - 1;
    const int64_t T = cx.T, G = cx.G;
    const int slot_floats = cx.slot_rows * kTileRows;
    const int64_t wf = wave_of(first, T, G), wl = wave_of(last, T, G);
    const int contributors = (int)(wl - wf + 1);
    int* ctr = cx.counters + D[j].rb_begin + rb;
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != contributors - 1) return;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int e = lane; e < M * kTileRows; e += 64) {
      const int m = e / kTileRows, col = e % kTileRows;
      float v = 0.f;
      for (int64_t w = wf; w <= wl; w++) {
        const int64_t aw = w * T / G;
        const int kw = aw >= first ? 0 : 1;
        v += __hip_atomic_load(cx.slots + (w * 2 + kw) * slot_floats + e, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_SYSTEM);
      }
      const int ncol = rb * kTileRows + col;
      if (ncol < N) Y[(int64_t)m * ldy + ncol] = v;
    }
    if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  }

  // xp points at X[0][kbase]; pieces with k = kbase + 8*col >= K or rows >= M
  // read X[0][0] and are never used.
  template <int BITS>
  static __device__ __forceinline__ void load(Regs& t, const uint8_t* wp, const uint16_t* X, int kbase,
                                              int lane, int M, int K, int64_t ldx) {
    t.w.wc = __builtin_nontemporal_load(gload_ptr<u4_t>(wp + 16 * lane));
    t.w.ws = __builtin_nontemporal_load(gload_ptr<u2_t>(wp + kScaleOff + 8 * (lane & 15)));
    if constexpr (BITS == 5) t.w.wh = __builtin_nontemporal_load(gload_ptr<uint32_t>(wp + kHiOff + 4 * lane));
    else t.w.wh = 0u;
#pragma unroll
    for (int p = 0; p < kPieces; p++) {
      const int piece = lane + 64 * p;
      const int row = piece >> 4, col = piece & 15;
      const int k = kbase + 8 * col;
      const bool ok = row < M && row < kLoadRows && k < K;
      t.x[p] = *gload_ptr<u4_t>(X + (ok ? (int64_t)row * ldx + k : 0));
    }
  }

  static __device__ __forceinline__ void stage(const Regs& t, uint8_t* xs, int lane) {
#pragma unroll
    for (int p = 0; p < kPieces; p++) {
      const int piece = lane + 64 * p;
      const int row = piece >> 4, col = piece & 15;
      if (row < kLoadRows) *(u4_t*)(xs + row * kXRowBytes + 16 * col) = t.x[p];
    }
  }

  // Tiles [s0, s1) of job j (local indices rb * NKT + kt), BITS fixed.
  template <int BITS>
  static __device__ __forceinline__ void segment(Ctx& cx, int j, int64_t s0, int64_t s1, uint8_t* xs) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    constexpr int TB = BITS == 4 ? kTile4 : kTile5;
    const int nkt = D[j].nkt, ngroups = D[j].ngroups, M = D[j].M, K = D[j].K;
    const int64_t ldx = D[j].ldx;
    const uint8_t* packed = D[j].packed;
    const uint16_t* X = D[j].X;
    const bool ragged_k = (ngroups & 3) != 0;
    // consume cursor
    int rb = (int)(s0 / nkt);
    int kt = (int)(s0 - (int64_t)rb * nkt);
    // prefetch cursor: stops at the segment's last tile (later loads re-read it)
    int64_t ps = s0;
    int pkt = kt;
    const uint8_t* pw = packed + s0 * TB;
    auto pf_advance = [&]() {
      if (ps < s1 - 1) {
        ps++;
        pw += TB;
        if (++pkt == nkt) pkt = 0;
      }
    };
    Regs buf[kDepth];
#pragma unroll
    for (int p = 0; p < kDepth; p++) {
      load<BITS>(buf[p], pw, X, pkt * kTileK, lane, M, K, ldx);
      pf_advance();
    }
    Acc acc;
    zero(acc);
    const int64_t n = s1 - s0;
    for (int64_t f = 0; f < n; f += kDepth) {
#pragma unroll
      for (int p = 0; p < kDepth; p++) {
        if (f + p < n) {
          stage(buf[p], xs, lane);
          __atomic_signal_fence(__ATOMIC_SEQ_CST);  // LDS writes stay before the reads
          const int gleft = ngroups - 4 * kt;
          if (!ragged_k || gleft >= 4) {
            if constexpr (kMfma) mfma1_tile<BITS, kNF, false>(acc.mf, buf[p].w, xs, lane, 4);
            else gemv1_tile<BITS, kCap, false>(acc.gv, buf[p].w, xs, lane, 4, M);
          } else {
            if constexpr (kMfma) mfma1_tile<BITS, kNF, true>(acc.mf, buf[p].w, xs, lane, gleft);
            else gemv1_tile<BITS, kCap, true>(acc.gv, buf[p].w, xs, lane, gleft, M);
          }
          if (kt == nkt - 1 || f + p == n - 1) {
            flush(acc, cx, j, rb);
            zero(acc);
          }
          if (++kt == nkt) {
            kt = 0;
            rb++;
          }
        }
        load<BITS>(buf[p], pw, X, pkt * kTileK, lane, M, K, ldx);
        pf_advance();
      }
    }
  }

  static __device__ void run(const SweepArgs& args, uint8_t* xs) {
    Ctx cx;
    cx.D = job_table(args);
    cx.counters = args.counters;
    cx.slots = args.slots;
    cx.T = args.total;
    cx.G = args.nwaves;
    cx.slot_rows = args.slot_rows;
    cx.lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane lets the compiler know it
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    cx.gw = (int64_t)blockIdx.x * kStreamWavesPerBlock + wave;
    const int64_t T = args.total, G = args.nwaves;
    cx.a = cx.gw * T / G;
    cx.b = (cx.gw + 1) * T / G;
    if (cx.gw >= G || cx.a >= cx.b) return;
    cx.pend_j0 = cx.pend_j1 = -1;
    cx.pend_rb0 = cx.pend_rb1 = 0;
    int j = 0;
    while (cx.a >= cx.D[j].tile_end) j++;
    // one segment per job the range touches
    for (int64_t f = cx.a; f < cx.b; j++) {
      const int64_t tb = cx.D[j].tile_begin;
      const int64_t e = cx.D[j].tile_end < cx.b ? cx.D[j].tile_end : cx.b;
      if (cx.D[j].bits == 4) segment<4>(cx, j, f - tb, e - tb, xs);
      else segment<5>(cx, j, f - tb, e - tb, xs);
      f = e;
    }
    if (cx.pend_j0 >= 0 || cx.pend_j1 >= 0) {
      // every slot store of this wave must be complete before any arrival
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (cx.pend_j0 >= 0) arrive(cx, cx.pend_j0, cx.pend_rb0);
      if (cx.pend_j1 >= 0) arrive(cx, cx.pend_j1, cx.pend_rb1);
    }
  }
};

// At least 4 waves per SIMD: 16 per CU keep every wave of the grid resident.
template <bool kMfma, int kCap>
__global__ void __launch_bounds__(64 * kStreamWavesPerBlock) __attribute__((amdgpu_waves_per_eu(4)))
stream_kernel(SweepArgs args) {
  using S = Stream<kMfma, kCap>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kStreamWavesPerBlock][S::kRows * kXRowBytes];
  S::run(args, xs[threadIdx.x >> 6]);
}

// --------------------------------------------------------------------------
// group kernel: panels of 17..64 rows (MFMA, 2..4 m blocks)
// --------------------------------------------------------------------------
// One workgroup of kGroupWaves waves per unit = (job, kGroupWaves row blocks),
// whole K.  Wave w owns row block kGroupWaves*g + w; the X chunk of each k tile
// is staged once in LDS for all waves (double buffered) and loaded kDepth tiles
// ahead together with the weight tiles.
template <int kMPad>
struct Group {
  static constexpr int kMb = kMPad / 16;
  static constexpr int kThreads = 64 * kGroupWaves;
  static constexpr int kPieces = (kMPad * 16 + kThreads - 1) / kThreads;
  static constexpr int kDepth = 3;

  struct Regs {
    WRegs w;
    u4_t x[kPieces];
  };

  // Waves whose row block lies past N read row block 0 and discard it, so
  // every wave issues the same loads.
  static __device__ __forceinline__ void load(Regs& t, const JobDesc& d, const uint8_t* wtile, int kt, int tid) {
    const int lane = tid & 63;
    load_w(t.w, wtile, d.bits, lane);
#pragma unroll
    for (int p = 0; p < kPieces; p++) {
      const int piece = tid + kThreads * p;
      const int row = piece >> 4, col = piece & 15;
      t.x[p] = load_x_piece(d.X, d.ldx, row, kt * kTileK + 8 * col, d.M, d.K);
    }
  }

  static __device__ __forceinline__ void stage(const Regs& t, uint8_t* xs, int tid) {
#pragma unroll
    for (int p = 0; p < kPieces; p++) {
      const int piece = tid + kThreads * p;
      const int row = piece >> 4, col = piece & 15;
      if (row < kMPad) *(u4_t*)(xs + row * kXRowBytes + 16 * col) = t.x[p];
    }
  }

  template <int BITS>
  static __device__ void run_unit(f4_t (&acc)[kMb], const JobDesc& d, int rb,
                                  uint8_t (*xs)[kMPad * kXRowBytes], int tid) {
    const bool rb_ok = rb < d.nrb;
    constexpr int tb = BITS == 4 ? kTile4 : kTile5;
    const uint8_t* wbase = d.packed + (int64_t)(rb_ok ? rb : 0) * d.nkt * tb;
    const int nkt = d.nkt;
    // prefetch runs kDepth tiles ahead and re-reads the last tile at the end
    Regs buf[kDepth];
#pragma unroll
    for (int p = 0; p < kDepth; p++) {
      const int lt = p < nkt ? p : nkt - 1;
      load(buf[p], d, wbase + (int64_t)lt * tb, lt, tid);
    }
    int parity = 0;
    for (int kt = 0; kt < nkt; kt += kDepth) {
#pragma unroll
      for (int p = 0; p < kDepth; p++) {
        const int t = kt + p;
        if (t < nkt) {
          uint8_t* xb = xs[parity];
          stage(buf[p], xb, tid);
          __syncthreads();
          if (rb_ok) mfma_tile<BITS, kMb>(acc, buf[p].w, xb, tid & 63, d.ngroups - 4 * t);
          parity ^= 1;
        }
        const int lt = t + kDepth < nkt ? t + kDepth : nkt - 1;
        load(buf[p], d, wbase + (int64_t)lt * tb, lt, tid);
      }
    }
    __syncthreads();  // both X buffers are free again
  }
};

template <int kMPad>
__global__ void __launch_bounds__(64 * kGroupWaves) group_kernel(SweepArgs args) {
  using S = Group<kMPad>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kMPad * kXRowBytes];
  const QG_CONST JobDesc* D = job_table(args);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int j = 0;
  for (int64_t u = blockIdx.x; u < args.total; u += gridDim.x) {
    while (u >= D[j].unit_end) j++;
    const JobDesc d = D[j];
    const int rb = (int)(u - d.unit_begin) * kGroupWaves + wave;
    f4_t acc[S::kMb];
#pragma unroll
    for (int mb = 0; mb < S::kMb; mb++) acc[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
    if (d.bits == 4) S::template run_unit<4>(acc, d, rb, xs, tid);
    else S::template run_unit<5>(acc, d, rb, xs, tid);
    const int n = rb * kTileRows + (lane & 15);
    if (rb < d.nrb && n < d.N) {
      QG_GLOBAL float* Y = (QG_GLOBAL float*)d.Y;
#pragma unroll
      for (int mb = 0; mb < S::kMb; mb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = 16 * mb + 4 * (lane >> 4) + i;
          if (m < d.M) Y[(int64_t)m * d.ldy + n] = acc[mb][i];
        }
    }
  }
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
  if (bits == 4)
    hipLaunchKernelGGL(pack_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, W, ldw, N, K, nkt,
                       total, (uint8_t*)packed, flag);
  else
    hipLaunchKernelGGL(pack_kernel<5>, dim3((unsigned)blocks), dim3(256), 0, stream, W, ldw, N, K, nkt,
                       total, (uint8_t*)packed, flag);
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
//       2 = group MFMA (cls = padded rows 32, 48, 64)
static sweep_fn pick(int kind, int cls) {
  if (kind == 0) {
    switch (cls) {
      case 1: return stream_kernel<false, 1>;
      case 2: return stream_kernel<false, 2>;
      case 4: return stream_kernel<false, 4>;
      case 8: return stream_kernel<false, 8>;
    }
  } else if (kind == 1) {
    switch (cls) {
      case 1: return stream_kernel<true, 1>;
      case 2: return stream_kernel<true, 2>;
      case 4: return stream_kernel<true, 4>;
      case 8: return stream_kernel<true, 8>;
      case 16: return stream_kernel<true, 16>;
    }
  } else {
    switch (cls) {
      case 32: return group_kernel<32>;
      case 48: return group_kernel<48>;
      case 64: return group_kernel<64>;
    }
  }
  return nullptr;
}

int sweep_threads(int kind) { return kind == 2 ? 64 * kGroupWaves : 64 * kStreamWavesPerBlock; }

int sweep_blocks_per_cu(int kind, int cls) {
  sweep_fn f = pick(kind, cls);
  if (!f) return 0;
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, (const void*)f, sweep_threads(kind), 0) != hipSuccess)
    return 0;
  return nb;
}

hipError_t launch_sweep(int kind, int cls, const SweepArgs& args, int grid, hipStream_t stream) {
  sweep_fn f = pick(kind, cls);
  if (!f) return hipErrorInvalidValue;
  hipLaunchKernelGGL(f, dim3(grid), dim3(sweep_threads(kind)), 0, stream, args);
  return hipGetLastError();
}

}  // namespace qg
