// Internal definitions shared by the host dispatcher and the gfx950 kernels of
// the quantized weight sweep.  Not part of the public boundary.
#pragma once

#include <stdint.h>

namespace qg {

constexpr int kTileRows = 16;        // rows n per tile
constexpr int kTileK = 128;          // k per tile (four groups of 32)
constexpr int kGroup = 32;           // k per scale group
constexpr int kScaleOff = 1024;      // 16 rows x 4 fp16 scales
constexpr int kHiOff = 1152;         // 5-bit: bit 4 of every code
constexpr int kTile4 = 1152;
constexpr int kTile5 = 1408;

// Weight formats (the public format codes).  All share the tile grid and the
// 1024 code bytes of a tile; they differ in the scale group and what follows.
constexpr int kFmtQ4 = 4;            // 4-bit symmetric, group 32
constexpr int kFmtQ5 = 5;            // 5-bit symmetric, group 32 (high bits at kHiOff)
constexpr int kFmtG64 = 0x104;       // 4-bit symmetric, group 64: one scale per row and half tile
constexpr int kFmtZP = 0x204;        // 4-bit asymmetric, group 32: u stored, zero points at kZeroOff
constexpr int kZeroOff = 1152;       // kFmtZP: 16 rows x one 16-bit word of four 4-bit zero points
constexpr int kTileG64 = 1088;
constexpr int kTileZP = 1184;
inline __host__ __device__ constexpr bool valid_fmt(int f) {
  return f == kFmtQ4 || f == kFmtQ5 || f == kFmtG64 || f == kFmtZP;
}
inline __host__ __device__ constexpr int fmt_group(int f) { return f == kFmtG64 ? 64 : kGroup; }

constexpr int kMaxInline = 12;       // jobs passed by value in the kernel arguments
constexpr int kMaxDevices = 64;      // devices the allocation-free sweep keeps a scratch address for
constexpr int kXRowBytes = 272;      // LDS row stride of a staged X chunk (256 + 16 pad)

// stream kernel (panels of at most 16 rows): waves per workgroup, and the
// waves in the grid.  The count is chosen from the shapes alone -- never from
// the device or M -- so the K split of every row group, and with it every
// output bit, is reproducible.  Two waves per SIMD: while one computes a step
// (the unpack is VALU-bound) the other's loads are in flight.  A launch of at
// least kStreamBigBytes of weights is "big": on the MFMA path its steps span
// twice the row blocks (one X chunk serves eight weight tiles instead of four).
// A big launch takes three workgroups per CU (3072 waves, 1.5 times what
// is resident at two waves per SIMD): each CU's third workgroup starts when
// one of its first two ends, which evens out the end of the sweep (measured
// on the 5-bit stack, M = 1: 2.37 -> 2.27 ms; counts that do not give every
// CU the same number of workgroups, or give two full rounds, are slower).
constexpr int kStreamWavesPerBlock = 4;
constexpr int kStreamWaves = 2048;
constexpr int kStreamWavesBig = 3072;
constexpr int64_t kStreamBigBytes = (int64_t)4 << 30;
// group kernel (17..64 rows): waves per workgroup (three per SIMD where the
// registers allow it: padded rows 32 and 48), 16-row blocks per wave
// Waves of a group-kernel workgroup (one workgroup per CU): four per SIMD at
// 32 and 48 rows (128 VGPRs), two at 64.
constexpr int group_waves(int mpad) { return mpad >= 64 ? 8 : 16; }
constexpr int kGroupRows = 2;

// Stream kernels walk "steps": one k tile of a row group of stream_rows(big)
// consecutive 16-row blocks.  The same for every class of a path, so the K
// split of a row -- and with it every output bit -- does not depend on M.
constexpr int stream_rows(bool big) { return big ? 8 : 4; }

inline __host__ __device__ constexpr int tile_bytes(int f) {
  return f == kFmtQ5 ? kTile5 : f == kFmtG64 ? kTileG64 : f == kFmtZP ? kTileZP : kTile4;
}

// Stream kernels split work by weight bytes: a step weighs its tile bytes /
// 128 rounded to the nearest unit (9 for the 4-bit formats, 11 for 5-bit),
// and every wave gets at least kMaxUnitWeight units, so every wave holds at
// least one step.
inline __host__ __device__ constexpr int unit_weight(int f) { return (tile_bytes(f) + kTileK / 2) / kTileK; }
// x / unit_weight(f) for x >= 0, by constant divisors (the planning code's
// divisions are on the path to a wave's first load)
inline __host__ __device__ int div_unit_weight(int x, int f) {
  return unit_weight(f) == 11 ? (int)((uint32_t)x / 11u) : (int)((uint32_t)x / 9u);
}
// Multiplier and shift of an exact division by d (1 <= d <= 2^17) for
// dividends 0 <= s < 2^31 (Granlund and Montgomery, "Division by invariant
// integers using multiplication", PLDI 1994): l = ceil(log2 d),
// m = floor(2^(31 + l) / d) + 1 < 2^32, s / d = (s m) >> (31 + l).
inline void div_magic(uint32_t d, uint32_t& m, int32_t& sh) {
  int l = 0;
  while ((1u << l) < d) l++;
  m = (uint32_t)(((uint64_t)1 << (31 + l)) / d + 1);
  sh = 31 + l;
}
constexpr int kMaxUnitWeight = 11;
static_assert(unit_weight(kFmtQ4) == 9 && unit_weight(kFmtQ5) == 11 && unit_weight(kFmtG64) == 9 &&
                  unit_weight(kFmtZP) == 9,
              "unit weights (div_unit_weight knows only 9 and 11)");

// One job as the kernels see it.  All sizes are derived on the host.
struct JobDesc {
  const uint8_t* packed;
  const uint16_t* X;
  float* Y;              // null: outputs not written (verify head)
  unsigned long long* keys;  // null, or kKeyCopies x kKeyRows argmax keys (verify head)
  int64_t ldx;
  int64_t ldy;
  int32_t ubeg;          // stream kernel: units [ubeg, uend) of this job's steps
  int32_t uend;          //   (a step weighs unit_weight(bits) units)
  int32_t N, K;
  int32_t M, fmt;         // fmt: a weight format code (kFmt*)
  int32_t nkt;           // ceil(K / 128)
  int32_t ngroups;       // K / 32
  int32_t nrb;           // ceil(N / 16)
  int32_t nrg;           // stream kernel: row groups, ceil(nrb / rows per step)
  uint32_t nkt_m;        // s / nkt = (s * nkt_m) >> nkt_sh for 0 <= s < 2^31 (host-computed)
  int32_t nkt_sh;
  int32_t grp_begin;     // group kernel: first row-block group of this job
  int32_t grp_end;
};

// Argmax key of output value v in column n: the value's bits mapped to an
// order-preserving unsigned integer in the high word, the complement of n in
// the low word, so the maximum key is the largest value and, among equal
// values, the lowest column.  0 is below every key.
inline __host__ __device__ unsigned long long logit_key(float v, int n) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)o << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)n);
}
inline __host__ __device__ float key_value(unsigned long long k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __builtin_bit_cast(float, (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
inline __host__ __device__ int key_column(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)k);
}

constexpr int kMaxSlots = 64;  // verify head: slots per call (at most one per row)
// verify head: argmax keys are kept in kKeyCopies copies of the per-row
// array (copy = wave or workgroup index mod kKeyCopies), so that the atomics
// of the many waves finishing together spread over that many addresses per row
constexpr int kKeyCopies = 16;
constexpr int kKeyRows = 64;
struct AcceptArgs {
  int32_t nslots, M;
  int32_t row0[kMaxSlots];
  int32_t ndraft[kMaxSlots];
};

struct SweepArgs {
  int32_t total;         // stream kernel: flat units; group kernel: row-block groups (< 2^31)
  int32_t nwaves;        // stream kernel: waves in the grid (fixes the K split)
  int32_t q, rem;        // stream kernel: wave w takes q units, one more if w < rem
  int32_t njobs;
  int32_t bshift;        // stream kernel with a table: log2 of the units per bucket
  int32_t spin_limit;    // stream kernel: polls a reader makes before it gives up on a slot
  int32_t pad_;
  int64_t slot_bytes;    // stream kernel: bytes of the slot region
  const JobDesc* table;  // device copy of all jobs (when njobs > kMaxInline), else null
  const int32_t* index;  // with a table: uend of every job, then the first job of every bucket
  float* slots;          // stream kernel: two partial-sum slots per wave (all zero between calls)
#ifdef QG_TIMELINE
  unsigned long long* trace;  // timeline build only: kTraceWords stamps per stream wave
#endif
  JobDesc inl[kMaxInline];
};

#ifdef QG_TIMELINE
// Timeline build (a diagnostic variant of the library): per stream wave,
//   [0] start, [1] first step computed, [2] last step computed, [3] end
//   (s_memrealtime, 100 MHz), [4] time waiting for step data after the
//   first step, [5] phase mask, [6] plan complete (the first tile's address
//   known), [7] time computing steps (MFMA path).
constexpr int kTraceWords = 8;
#endif

// Stream kernel slots: per wave two slots (its head piece, its tail piece),
// each 64 lanes x rows * acc floats; acc = accumulators per row block (MFMA:
// ceil(class / 4), GEMV: class).
inline __host__ __device__ constexpr int stream_acc(bool mfma, int cls) { return mfma ? (cls + 3) / 4 : cls; }
inline __host__ __device__ constexpr int64_t stream_slot_bytes(int nwaves, int rows, bool mfma, int cls) {
  return (int64_t)nwaves * 2 * 64 * rows * stream_acc(mfma, cls) * 4;
}
// a reader's polls of one slot before it gives up (the wait ends long before
// in any sweep; the bound only guarantees that every wave exits)
constexpr int kSpinLimit = 1 << 20;

}  // namespace qg
