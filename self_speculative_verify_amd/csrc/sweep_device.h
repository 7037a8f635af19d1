// Device helpers shared by the sweep kernels (stream and group kernels):
// exact code unpack, scale conversion, argmax keys and LDS-direct copies.
// Internal to the library; included by the .hip translation units only.
//
// Exactness: codes are unpacked to exact fp16 integers (IEEE binary16 with
// exponent field 25 has unit spacing on [1024, 2048), so OR-ing a code into
// the mantissa of 1024.0 and subtracting 1024 + bias gives q exactly); every
// product q * x is exact in fp32 and each group's partial sum is scaled by
// its own fp32 scale.  Rounding a dequantized q*s to fp16 would not be exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm_internal.h"
#include "stream_plan.h"

namespace qg {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));
typedef float f2_t __attribute__((ext_vector_type(2)));

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
// A value the compiler must hold in a VGPR without knowing it (an empty asm
// that emits nothing): a constant passed through it stays a register operand
// instead of a literal.
__device__ __forceinline__ uint32_t in_reg(uint32_t v) {
  asm("" : "+v"(v));
  return v;
}

// (a & m) | o as one v_and_or_b32.  With two literal operands the compiler
// would split it into v_and + v_or (a VOP3 encoding holds no literal on this
// target), so constant operands are handed over as registers; and the result
// is pinned, or a chain (h & m1) | ((w & m0) | c) is re-associated into two
// v_and and a v_or3.  The instruction itself is the compiler's, so its
// hazard checks see it (an instruction written in asm would be invisible to
// them: next to an MFMA still writing a VGPR, that is a wrong result).
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  if (__builtin_constant_p(o)) o = in_reg(o);
  return in_reg((a & in_reg(m)) | o);
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
  const h2_t h = scale_pair(pair);
  float f = (float)(HI ? h.y : h.x);
  asm("" : "+v"(f));  // the fp32 value must exist: the conversion stays an instruction
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

}  // namespace qg
