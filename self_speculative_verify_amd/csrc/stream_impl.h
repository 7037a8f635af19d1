// gfx950 stream kernels of the quantized weight sweep: panels of at most 16
// rows (GEMV, or MFMA with one m block).
//
// The method (Quasar/q27 wiki): decode streams every quantized linear weight
// once per step ("decode physics" paragraph: decode is bound by weight reads)
// and one weight read serves all draft positions of all slots (intro bullets
// on the fused verify sweep).  These kernels are the decode-sized end of that
// sweep: a single weight read per tile, the activation panel M <= 16 rows.
//
// Work is a flat sequence of steps (job, row group, k tile); a row group is
// kR consecutive 16-row blocks, and one step reads the kR tiles of its row
// group at one k tile.  Units of weight bytes (a step weighs its tile bytes /
// 128) are cut into `nwaves` equal contiguous ranges, one per wave; a wave
// owns the steps whose first unit lies in its range.  The cut depends on the
// shapes only, so every output bit is the same for every M of a class.
//
// A row group whose steps fall into several ranges ("split") is summed
// without counters (stream_plan.h has the rules): every contributor but the
// last stores its partial sums into a slot of its own, and the last one adds
// them in wave order (k order), its own last, writes Y and clears the slots.
// A wave takes the pieces it writes first and the piece it reads last, so a
// reader normally finds the first contributor's partial long written.  Slots
// hold the fp32 bits of the partials with +0 stored as -0; an all-zero word
// means "not yet written" and a workspace of zeros is empty, which every
// completed sweep leaves behind.  The reader polls (bounded) until every word
// of its sources is non-zero; it only ever waits for waves of lower index.
// Accumulators start at +0 and fp32 round-to-nearest never turns +0 into -0,
// so no partial is -0 itself, and a sum with a stored -0 is bitwise the sum
// with +0.
//
// Per step the X chunk (class rows x 128 k: 16 bytes per lane and load, one
// load for up to four rows) goes through a wave-private LDS buffer, from
// which the MFMA A fragments (or the GEMV operands) are read: one global load
// instruction per four panel rows and step instead of one per MFMA group.
//
// MFMA: v_mfma_f32_16x16x32_f16 with A = X (16 rows x 32 k of one group)
// and B = codes (32 k x 16 rows n): lane l supplies A row l%16 and B column
// n = l%16, both for k chunk l/16 -- exactly the lane's 16 code bytes -- and
// holds D rows 4(l/16) + i of column n.  X row m is placed at A row
// 4(m%4) + m/4, so it comes out in lane group g = m%4, accumulator i = m/4:
// a panel of at most 4 kA rows keeps kA = ceil(class / 4) accumulators per
// lane, and the group's scale multiplies only those.
// GEMV: lane l = r + 16c forms, for row n = r and each m, four
// v_dot2_f32_f16 over its 8 codes of a group, scaled by the group's scale;
// the four k chunks of a row (lanes r, r+16, r+32, r+48) are summed when the
// row group is written.
// Padding groups (beyond K) have codes q = 0 and scale +0, and their X reads
// are clamped into the row, so they add exact zeros: no tile needs a branch.
#pragma once

#include <utility>

#include "sweep_device.h"

namespace qg {

// format sets of a launch (bit i: format class i present)
constexpr int kSetQ4 = 1, kSetQ5 = 2, kSetG64 = 4, kSetZP = 8;

template <bool kMfma, int kCap, int kR, int kFS>
struct Stream {
  static constexpr int kA = kMfma ? (kCap + 3) / 4 : kCap;      // accumulators per row block
  static constexpr int kAcc = kR * kA;                         // partial-sum floats per lane
  static_assert(kAcc % 4 == 0, "slot words move in 16-byte stores");
  static constexpr int kXP = (kCap * 16 + 63) / 64;            // 16-byte X pieces per lane and step
  // steps in flight: one for MFMA class 16 in eight-block steps, whose two
  // step buffers would leave it one wave per SIMD (see kTwoPerSimd)
  static constexpr int kDepth = (kMfma && kCap == 16 && kR == 8) ? 1 : 2;
  static constexpr bool kSide = (kFS & (kSetQ5 | kSetZP)) != 0;
  static constexpr int kOnly = kFS == kSetQ4 ? kFmtQ4 : kFS == kSetQ5 ? kFmtQ5 : kFS == kSetG64 ? kFmtG64
                               : kFS == kSetZP ? kFmtZP : 0;   // the one format, or 0
  // The raised second dispatch half drops back to the base priority when a
  // quarter of its work is left (MFMA, four-block steps, at most four rows;
  // measured on gate+up 34816 x 5120 4-bit at M = 1, 2, 4: 23.2 -> 22.7,
  // 23.6 -> 22.8, 23.4 -> 22.6 us).  Applied to every kernel the same rule
  // made the big 5-bit stack 20 % slower and the M = 6 pair no faster.
  static constexpr bool kEvenEnd = kMfma && kR == 4 && kCap <= 4;

  struct Step {
    u4_t c[kR];
    u2_t s[kR];
    uint32_t h[kSide ? kR : 1];
    u4_t x[kXP];
  };

  using Phases = StreamPhases;
  using Pos = StreamPos;

  // ---------------------------------------------------------------- loads
  // kR weight tiles (non-temporal: streamed once), their scales and side
  // words, and the X chunk of k tile kt: lane l, piece p holds X[row][k0 +
  // 8 col ..] for row = 4p + l/16 (rows past M read row M-1) and col = l%16;
  // k is clamped into the row (padding groups multiply it by zero codes).
  // Per-lane byte offsets of a tile's loads, and of the lane's X piece in
  // its job's panel (row clamped to M - 1, k = 0), computed once per job: the
  // loads then take a uniform 64-bit base plus an unsigned 32-bit lane offset
  // (the global_load SGPR-base form), with no per-step address arithmetic.
  struct Lane {
    uint32_t code, scale, scale64, hi, zp;
    uint32_t x[kXP];
    uint32_t xcol;
  };
  static __device__ __forceinline__ void lane_offsets(Lane& o, int lane) {
    o.code = 16u * lane;
    o.scale = kScaleOff + 8u * (lane & 15);
    o.scale64 = kScaleOff + 4u * (lane & 15);
    o.hi = kHiOff + 4u * lane;
    o.zp = kZeroOff + 2u * (lane & 15);
    o.xcol = 16u * (lane & 15);
  }
  static __device__ __forceinline__ void x_offsets(Lane& o, const Pos& c, int lane) {
#pragma unroll
    for (int p = 0; p < kXP; p++) {
      const int row = 4 * p + (lane >> 4);
      const int m = row < c.M ? row : c.M - 1;
      o.x[p] = 2u * (uint32_t)(m * c.ldx) + o.xcol;
    }
  }
  template <typename T>
  static __device__ __forceinline__ T ldnt(const uint8_t* base, uint32_t off) {
    return __builtin_nontemporal_load((const QG_GLOBAL T*)((const QG_GLOBAL uint8_t*)base + off));
  }

  template <int F>
  static __device__ __forceinline__ void load_tiles(Step& t, const uint8_t* wp, const uint32_t (&roff)[kR],
                                                    bool spill, const Lane& o) {
#pragma unroll
    for (int r = 0; r < kR; r++) {
      const uint8_t* tp = wp + (spill ? 0u : roff[r]);
      t.c[r] = ldnt<u4_t>(tp, o.code);
      if constexpr (F == kFmtG64) {
        t.s[r].x = ldnt<uint32_t>(tp, o.scale64);
        t.s[r].y = 0u;
      } else {
        t.s[r] = ldnt<u2_t>(tp, o.scale);
      }
      if constexpr (kSide) {
        if constexpr (F == kFmtQ5) t.h[r] = ldnt<uint32_t>(tp, o.hi);
        else if constexpr (F == kFmtZP) t.h[r] = ldnt<uint16_t>(tp, o.zp);
        else t.h[r] = 0u;
      }
    }
  }

  // X chunk of k tile kt: lane l, piece p holds X[row][k0 + 8 col ..] for
  // row = 4p + l/16 (rows past M read row M-1) and col = l%16; in a k tile
  // past K's end, k is clamped into the row (padding groups multiply it by
  // zero codes).
  static __device__ __forceinline__ void load_x(Step& t, const Pos& c, const Lane& o, int lane) {
    const uint8_t* xb = (const uint8_t*)c.X;
    if ((c.kt + 1) * kTileK <= c.K) {
      const uint8_t* xk = xb + 2u * (uint32_t)(c.kt * kTileK);
#pragma unroll
      for (int p = 0; p < kXP; p++) t.x[p] = *(const QG_GLOBAL u4_t*)((const QG_GLOBAL uint8_t*)xk + o.x[p]);
    } else {
      int k = c.kt * kTileK + 8 * (lane & 15);
      k = k < c.K - 8 ? k : c.K - 8;
#pragma unroll
      for (int p = 0; p < kXP; p++)
        t.x[p] = *(const QG_GLOBAL u4_t*)((const QG_GLOBAL uint8_t*)xb + (o.x[p] - o.xcol + 2u * (uint32_t)k));
    }
  }

  // Loads of the step at c.  Past the wave's last step (spill != null) the
  // same loads (so the wait counts stay exact) go to `spill`: the X panel of
  // the cursor's job when it holds at least a 5-bit tile's bytes (every wave
  // reads X, so it stays cached), else that job's first tile, read in the
  // job's own format.  Tile r of the step sits roff[r] bytes after tile
  // (rg * kR, kt); blocks past the job's last re-read its last one (their
  // sums are never stored).
  static __device__ __forceinline__ void load(Step& t, const Pos& c, const uint8_t* spill, const Lane& o,
                                              int lane) {
    const int tb = tile_bytes(kOnly ? kOnly : c.fmt);
    const uint32_t rstride = (uint32_t)(c.nkt * tb);
    const int left = c.nrb - 1 - c.rg * kR;
    uint32_t roff[kR];
#pragma unroll
    for (int r = 0; r < kR; r++) roff[r] = (uint32_t)(r < left ? r : left) * rstride;
    const uint8_t* wp = spill ? spill : c.packed + ((int64_t)c.rg * kR * c.nkt + c.kt) * tb;
    const bool sp = spill != nullptr;
    if constexpr (kOnly) {
      load_tiles<kOnly>(t, wp, roff, sp, o);
    } else {
      if ((kFS & kSetQ4) && c.fmt == kFmtQ4) load_tiles<kFmtQ4>(t, wp, roff, sp, o);
      else if ((kFS & kSetQ5) && c.fmt == kFmtQ5) load_tiles<kFmtQ5>(t, wp, roff, sp, o);
      else if ((kFS & kSetG64) && c.fmt == kFmtG64) load_tiles<kFmtG64>(t, wp, roff, sp, o);
      else load_tiles<kFmtZP>(t, wp, roff, sp, o);
    }
    load_x(t, c, o, lane);
  }

  static __device__ __forceinline__ const uint8_t* spill_of(const JobDesc& d) {
    return 2 * ((int64_t)(d.M - 1) * d.ldx + d.K) >= kTile5 ? (const uint8_t*)d.X : d.packed;
  }

  // -------------------------------------------------------------- compute
  // The step's X chunk into the wave's LDS buffer (rows < class), then the
  // contraction of its kR tiles.
  static __device__ __forceinline__ void stage_x(const Step& t, uint8_t* xs, int lane) {
#pragma unroll
    for (int p = 0; p < kXP; p++) {
      const int row = 4 * p + (lane >> 4);
      if (row < kCap) *(u4_t*)(xs + row * kXRowBytes + 16 * (lane & 15)) = t.x[p];
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // LDS writes stay before the reads
  }

  template <int F>
  static __device__ __forceinline__ void compute(float (&acc)[kR][kA], const Step& t, const uint8_t* xs,
                                                 int lane) {
    if constexpr (kMfma) {
      const f4_t zero = {0.f, 0.f, 0.f, 0.f};
      // A row ar = l % 16 carries X row (ar / 4) + 4 (ar % 4); rows past the
      // class read the zero row after the staged ones (their outputs are
      // never stored; zeros rather than copies of a real row measured 0.3 -
      // 0.8 % faster on the 5-bit stack at M = 1, 4, 8)
      const int ar = lane & 15, c = lane >> 4;
      int mr = (ar >> 2) + 4 * (ar & 3);
      mr = mr < kCap ? mr : kCap;
      h8_t a[4];
#pragma unroll
      for (int j = 0; j < 4; j++) a[j] = lds_h8(xs + mr * kXRowBytes + 64 * j + 16 * c);
#pragma unroll
      for (int r = 0; r < kR; r++) {
        const uint32_t side = side_word<F>(t.h[kSide ? r : 0]);
        f4_t p[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          const h8_t q = unpack_chunk<F>(t.c[r][j], side, j);
          // group 64: the second half of a group accumulates onto the first
          const f4_t c0 = (F == kFmtG64 && (j & 1)) ? p[j ^ 1] : zero;
          p[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], q, c0, 0, 0, 0);
        }
        // each scale converted by an instruction of its own (left to itself
        // the compiler fuses the conversion into mixed-precision FMAs, which
        // issue more slowly)
        if constexpr (F == kFmtG64) {
          const float s0 = scale_f32<0>(t.s[r].x), s1 = scale_f32<1>(t.s[r].x);
#pragma unroll
          for (int i = 0; i < kA; i++) acc[r][i] = __builtin_fmaf(s0, p[1][i], acc[r][i]);
#pragma unroll
          for (int i = 0; i < kA; i++) acc[r][i] = __builtin_fmaf(s1, p[3][i], acc[r][i]);
        } else {
          const float sj[4] = {scale_f32<0>(t.s[r].x), scale_f32<1>(t.s[r].x), scale_f32<0>(t.s[r].y),
                               scale_f32<1>(t.s[r].y)};
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int i = 0; i < kA; i++) acc[r][i] = __builtin_fmaf(sj[j], p[j][i], acc[r][i]);
        }
      }
    } else {
      const int c = lane >> 4;
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
    }
  }

  static __device__ __forceinline__ void compute_any(float (&acc)[kR][kA], const Step& t, int fmt,
                                                     uint8_t* xs, int lane) {
    stage_x(t, xs, lane);
    if constexpr (kOnly) {
      compute<kOnly>(acc, t, xs, lane);
    } else {
      if ((kFS & kSetQ4) && fmt == kFmtQ4) compute<kFmtQ4>(acc, t, xs, lane);
      else if ((kFS & kSetQ5) && fmt == kFmtQ5) compute<kFmtQ5>(acc, t, xs, lane);
      else if ((kFS & kSetG64) && fmt == kFmtG64) compute<kFmtG64>(acc, t, xs, lane);
      else compute<kFmtZP>(acc, t, xs, lane);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the next step's LDS writes stay after these reads
  }

  static __device__ __forceinline__ void zero(float (&acc)[kR][kA]) {
#pragma unroll
    for (int r = 0; r < kR; r++)
#pragma unroll
      for (int i = 0; i < kA; i++) acc[r][i] = 0.f;
  }

  // ------------------------------------------------------------- epilogue
  struct Ctx {
    const QG_CONST JobDesc* D;
    float* slots;
    uint32_t slot_bytes;      // bytes of the slot region
    int q, rem;               // partition of the units over the waves
    int gw, lane;
    int spin_limit;
    // verify head: best argmax key of this lane's rows over the columns it
    // finished (accumulator i's row), published at the end of the range
    unsigned long long best[kA];
  };

  // slot (wave w, kind k) of the lane: kAcc floats at this byte offset
  static __device__ __forceinline__ uint32_t slot_off(int w, int k, int lane) {
    return (uint32_t)(((w * 2 + k) * 64 + lane) * kAcc) * 4u;
  }
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(const Ctx& cx) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)cx.slots, (short)0, (int)cx.slot_bytes, kBufWord3);
  }

  // Lanes' row m of accumulator i (MFMA), or m = i (GEMV)
  static __device__ __forceinline__ int row_of(int lane, int i) { return kMfma ? (lane >> 4) + 4 * i : i; }

  // GEMV: the four k chunks of each row summed across lanes (lanes < 16 hold
  // the totals)
  static __device__ __forceinline__ void lanes_sum(float (&acc)[kR][kA]) {
    if constexpr (!kMfma) {
#pragma unroll
      for (int r = 0; r < kR; r++)
#pragma unroll
        for (int m = 0; m < kA; m++) {
          float v = acc[r][m];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          acc[r][m] = v;
        }
    }
  }

  // Final sums of row group rg of job j to Y (and the argmax keys).
  static __device__ __forceinline__ void store_y(float (&acc)[kR][kA], Ctx& cx, int j, int rg) {
    const QG_CONST JobDesc* D = cx.D;
    const int lane = cx.lane;
    lanes_sum(acc);
    const int M = D[j].M, N = D[j].N;
    const int64_t ldy = D[j].ldy;
    QG_GLOBAL float* Y = (QG_GLOBAL float*)D[j].Y;
    const bool keys = D[j].keys != nullptr;
    const bool holder = kMfma || lane < 16;
#pragma unroll
    for (int r = 0; r < kR; r++) {
      const int n = (rg * kR + r) * kTileRows + (lane & 15);
      if (holder && n < N) {
#pragma unroll
        for (int i = 0; i < kA; i++) {
          const int m = row_of(lane, i);
          if (m < M) {
            if (Y) Y[(int64_t)m * ldy + n] = acc[r][i];
            if (keys) cx.best[i] = umax64(cx.best[i], logit_key(acc[r][i], n));
          }
        }
      }
    }
  }

  // Writer: this lane's partials, +0 stored as -0, into slot (gw, k).
  static __device__ __forceinline__ void store_partial(const float (&acc)[kR][kA], const Ctx& cx, int k) {
    const __amdgpu_buffer_rsrc_t sr = slot_rsrc(cx);
    const uint32_t o = slot_off(cx.gw, k, cx.lane);
    uint32_t w[kAcc];
#pragma unroll
    for (int r = 0; r < kR; r++)
#pragma unroll
      for (int i = 0; i < kA; i++) {
        const uint32_t b = __builtin_bit_cast(uint32_t, acc[r][i]);
        w[r * kA + i] = b ? b : 0x80000000u;
      }
#pragma unroll
    for (int e = 0; e < kAcc; e += 4)
      __builtin_amdgcn_raw_buffer_store_b128(u4_t{w[e], w[e + 1], w[e + 2], w[e + 3]}, sr, o + 4u * e, 0,
                                             kCoherent);
  }

  // Reader: the partial of slot (w, k) once every word of it is written
  // (bounded wait; on timeout the words read are used as they are), then
  // the slot cleared for the next sweep.
  static __device__ __forceinline__ void take_partial(uint32_t (&w)[kAcc], const Ctx& cx, int wsrc, int k) {
    const __amdgpu_buffer_rsrc_t sr = slot_rsrc(cx);
    const uint32_t o = slot_off(wsrc, k, cx.lane);
    for (int spin = 0;; spin++) {
      bool ready = true;
      load_words(w, sr, o);
#pragma unroll
      for (int e = 0; e < kAcc; e++) ready = ready && w[e] != 0u;
      if (__builtin_amdgcn_read_exec() == __ballot(ready) || spin >= cx.spin_limit) break;
      __builtin_amdgcn_s_sleep(2);
    }
#pragma unroll
    for (int e = 0; e < kAcc; e += 4)
      __builtin_amdgcn_raw_buffer_store_b128(u4_t{0u, 0u, 0u, 0u}, sr, o + 4u * e, 0, kCoherent);
  }

  static __device__ __forceinline__ void load_words(uint32_t (&w)[kAcc], __amdgpu_buffer_rsrc_t sr, uint32_t o) {
#pragma unroll
    for (int e = 0; e < kAcc; e += 4) {
      const u4_t v = __builtin_bit_cast(u4_t, __builtin_amdgcn_raw_buffer_load_b128(sr, o + 4u * e, 0, kCoherent));
      w[e] = v.x;
      w[e + 1] = v.y;
      w[e + 2] = v.z;
      w[e + 3] = v.w;
    }
  }

  // Reader of row group rg of job j (its last contributor, wave wl): the
  // partials of contributors wf .. wl - 1 in wave order, then its own, to Y.
  // The sources' slots are loaded kBatch at a time (all loads issued, then
  // each checked; one not yet complete falls back to the bounded poll), so
  // a row group split over many waves costs a few memory round trips, not
  // one per contributor; the sum keeps wave order, so the result is the
  // same bits.  Measured: a round of 256 one-matrix sweeps at M = 6 (row
  // groups split over up to ~26 waves) 6.09 -> 5.25 ms; gate+up at M = 1
  // 22.7 -> 22.1 us; the 1024 x 1024 sweep 7.5 -> 7.1 us.
  static constexpr int kBatch = kAcc >= 32 ? 1 : 32 / kAcc;
  static __device__ __forceinline__ void read_split(float (&acc)[kR][kA], Ctx& cx, int j, int rg) {
    int wf, wl;
    stream_contributors(cx.q, cx.rem, cx.D, j, rg, wf, wl);
    const __amdgpu_buffer_rsrc_t sr = slot_rsrc(cx);
    float v[kR][kA];
    for (int s0 = wf; s0 < wl; s0 += kBatch) {
      uint32_t w[kBatch][kAcc];
#pragma unroll
      for (int b = 0; b < kBatch; b++)
        if (s0 + b < wl) load_words(w[b], sr, slot_off(s0 + b, s0 + b == wf ? 1 : 0, cx.lane));
#pragma unroll
      for (int b = 0; b < kBatch; b++) {
        const int src = s0 + b;
        if (src >= wl) break;
        // the first contributor's piece is its tail (slot 1), the others' their whole range (slot 0)
        const int k = src == wf ? 1 : 0;
        bool ready = true;
#pragma unroll
        for (int e = 0; e < kAcc; e++) ready = ready && w[b][e] != 0u;
        if (__builtin_amdgcn_read_exec() == __ballot(ready)) {
          // complete: clear the slot for the next sweep
#pragma unroll
          for (int e = 0; e < kAcc; e += 4)
            __builtin_amdgcn_raw_buffer_store_b128(u4_t{0u, 0u, 0u, 0u}, sr, slot_off(src, k, cx.lane) + 4u * e, 0,
                                                   kCoherent);
        } else {
          take_partial(w[b], cx, src, k);
        }
#pragma unroll
        for (int r = 0; r < kR; r++)
#pragma unroll
          for (int i = 0; i < kA; i++) {
            const float x = __builtin_bit_cast(float, w[b][r * kA + i]);
            v[r][i] = src == wf ? x : v[r][i] + x;
          }
      }
    }
#pragma unroll
    for (int r = 0; r < kR; r++)
#pragma unroll
      for (int i = 0; i < kA; i++) acc[r][i] = v[r][i] + acc[r][i];
    store_y(acc, cx, j, rg);
  }

  // Verify head: the range's best key per row, over the 16 lanes holding the
  // row's columns, into the job's keys (one atomic per row and wave).
  static __device__ __forceinline__ void publish(Ctx& cx, unsigned long long* keys, int M) {
    const int lane = cx.lane;
#pragma unroll
    for (int i = 0; i < kA; i++) {
      const unsigned long long k = lanes_max<1, 16>(cx.best[i]);
      const int m = row_of(lane, i);
      if ((lane & 15) == 0 && (kMfma || lane == 0) && m < M && k != 0ull) key_max(keys + m, k);
      cx.best[i] = 0ull;
    }
  }

  // ----------------------------------------------------------------- main
#ifdef QG_TIMELINE
  // stamps on the MFMA path only (the GEMV kernels have no registers to spare)
  static constexpr bool kTrace = kMfma;
  // s_memrealtime after v is computed (the operand orders it after the work)
  static __device__ __forceinline__ unsigned long long trace_stamp(float v) {
    unsigned long long t;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : "v"(v) : "memory");
    return t;
  }
#endif
  template <typename F, int... P>
  static __device__ __forceinline__ void each_slot(F& f, std::integer_sequence<int, P...>) {
    (f(std::integral_constant<int, P>{}), ...);
  }

  // args: the kernel's argument where it lies (kernarg segment); the job
  // table pointer below may point into it.
  static __device__ __forceinline__ void run(const QG_CONST SweepArgs& args, uint8_t* xs) {
    Ctx cx;
    const QG_CONST JobDesc* D = job_table(args);
    cx.D = D;
    cx.slots = args.slots;
    cx.slot_bytes = (uint32_t)args.slot_bytes;
    cx.q = args.q;
    cx.rem = args.rem;
    cx.spin_limit = args.spin_limit;
    cx.lane = threadIdx.x & 63;
    const int lane = cx.lane;
    if constexpr (kMfma) {
      // the zero row after the staged X rows (read by the A rows past the class)
      const u4_t z4 = {0u, 0u, 0u, 0u};
      if (lane < 16) *(u4_t*)(xs + kCap * kXRowBytes + 16 * lane) = z4;
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    // wave-uniform by construction; readfirstlane lets the compiler know it
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    cx.gw = (int)blockIdx.x * kStreamWavesPerBlock + wave;
    if (cx.gw >= args.nwaves) return;
#ifdef QG_TIMELINE
    const unsigned long long t0 = kTrace ? trace_stamp(0.f) : 0ull;
    unsigned long long t1 = 0, t2 = 0, ta = 0, tb = 0, twait = 0, tcomp = 0;
    int nsteps = 0;
#endif
#pragma unroll
    for (int i = 0; i < kA; i++) cx.best[i] = 0ull;
    const int a = stream_start_of(cx.gw, cx.q, cx.rem);
    const int b = a + cx.q + (cx.gw < cx.rem ? 1 : 0);
    Phases P;
    const StreamGrid grid = {args.index, args.njobs, args.bshift, cx.q, cx.rem};
    if (args.njobs == 1) stream_plan<true>(P, grid, D, cx.gw, a, b);
    else stream_plan<false>(P, grid, D, cx.gw, a, b);

    Pos pc, cc;
    stream_start(pc, D, P);
    cc = pc;
    const int njobs = args.njobs;
    Lane lo;
    lane_offsets(lo, lane);
    x_offsets(lo, pc, lane);
    int xjob = pc.j;  // the job lo.x was computed for
#ifdef QG_TIMELINE
    // the plan is complete once the first tile's address is known
    unsigned long long tplan = 0;
    if (kTrace) {
      asm volatile("" ::"s"(pc.packed), "s"(pc.X));
      tplan = trace_stamp(0.f);
    }
#endif
    const uint8_t* spill = nullptr;
    Step buf[kDepth];
#pragma unroll
    for (int p = 0; p < kDepth; p++) {
      load(buf[p], pc, spill, lo, lane);
      if (!spill) {
        stream_advance(pc, D, P, njobs);
        if (pc.ph == 4) {
          if (pc.j >= njobs) stream_load_job(pc, D, njobs - 1);
          spill = spill_of(D[pc.j]);
        }
        if (pc.j != xjob) {
          x_offsets(lo, pc, lane);
          xjob = pc.j;
        }
      }
    }
    float acc[kR][kA];
    zero(acc);
    bool done = false;
    // the wave's units still to compute (kEvenEnd), and whether it runs raised
    const int utot = b - a;
    int urem = utot;
    bool raised = cx.gw >= args.nwaves / 2;
    // one pipeline slot: consume buffer p (while steps are left), then refill
    // it kDepth steps ahead; p is a constant in every instance, so the
    // buffers stay in registers
    auto slot = [&](auto pc_) {
      constexpr int p = decltype(pc_)::value;
      if (!done) {
#ifdef QG_TIMELINE
        if (kTrace) {
          // every load of the step has landed: the time since the previous
          // step's compute ended was spent waiting for it
          asm volatile("" ::"v"(buf[p].c[kR - 1]), "v"(buf[p].s[kR - 1]), "v"(buf[p].x[kXP - 1]));
          ta = trace_stamp(0.f);
          if (nsteps) twait += ta - tb;
        }
#endif
        compute_any(acc, buf[p], cc.fmt, xs, lane);
        if constexpr (kEvenEnd) {
          urem -= cc.fmt == kFmtQ5 ? unit_weight(kFmtQ5) : unit_weight(kFmtQ4);
          if (raised && 4 * urem <= utot) {
            __builtin_amdgcn_s_setprio(0);
            raised = false;
          }
        }
#ifdef QG_TIMELINE
        if (kTrace) {
          tb = trace_stamp(acc[kR - 1][kA - 1]);
          tcomp += tb - ta;
        }
#endif
        const int j = cc.j, rg = cc.rg, ph = cc.ph;
        const bool rg_end = cc.kt == cc.nkt - 1;
        stream_advance(cc, D, P, njobs);
        if (rg_end || cc.ph != ph) {
          if (ph == 2) store_y(acc, cx, j, rg);
          else if (ph == 3) read_split(acc, cx, j, rg);
          else store_partial(acc, cx, ph == 0 ? 1 : 0);
          zero(acc);
        }
        done = cc.ph == 4;
#ifdef QG_TIMELINE
        if (kTrace && nsteps++ == 0) t1 = trace_stamp(acc[0][0]);
        if (kTrace && done) t2 = trace_stamp(acc[0][0]);
#endif
      }
      load(buf[p], pc, spill, lo, lane);
      if (!spill) {
        stream_advance(pc, D, P, njobs);
        if (pc.ph == 4) {
          if (pc.j >= njobs) stream_load_job(pc, D, njobs - 1);
          spill = spill_of(D[pc.j]);
        }
        if (pc.j != xjob) {
          x_offsets(lo, pc, lane);
          xjob = pc.j;
        }
      }
    };
    // Two waves share each SIMD: the first half of the grid is dispatched
    // first, the second half joins while those already stream.  The later
    // waves run at a raised priority, so that their planning and first loads
    // are not held behind their partners' unpacking (measured: the M = 6
    // verify workload 42.4 -> 39.9 us, the rest unchanged or faster).  With
    // kEvenEnd they drop back once a quarter of their work is left, so that
    // the first half, which has lost the arbitration until then, catches up
    // and the two halves end together.
    if (raised) __builtin_amdgcn_s_setprio(1);
    while (!done) each_slot(slot, std::make_integer_sequence<int, kDepth>{});
#ifdef QG_TIMELINE
    if (kTrace) __builtin_amdgcn_s_waitcnt(0);
    const unsigned long long t3 = kTrace ? trace_stamp(0.f) : 0ull;
    if (kTrace && args.trace && lane == 0) {
      unsigned long long* tr = args.trace + (size_t)cx.gw * kTraceWords;
      tr[0] = t0;
      tr[1] = t1;
      tr[2] = t2;
      tr[3] = t3;
      tr[4] = twait;
      tr[6] = tplan;
      tr[5] = (unsigned long long)P.mask;
      tr[7] = tcomp;
    }
#endif
    const QG_CONST JobDesc& dk = D[0];
    if (dk.keys) publish(cx, dk.keys + (cx.gw % kKeyCopies) * kKeyRows, dk.M);
  }
};

// The grid holds two waves per SIMD.  The MFMA class-8 kernel in
// eight-block steps is built under that register budget: left to itself it
// takes 198 VGPRs + 66 AGPRs (one wave per SIMD); within 256 it keeps its
// MFMA results in VGPRs and fits two (the 5-bit stack at M = 8: 2.70 ->
// 2.60 ms).  Class 16 in eight-block steps took 254 VGPRs + 136 AGPRs (one
// wave per SIMD); with one step in flight instead of two it fits two in 245
// VGPRs (the 5-bit stack at M = 9 / 12 / 16: 3.04 / 3.07 / 3.14 -> 2.85 /
// 2.93 / 3.02 ms).  The others already fit two (or, GEMV class 8, would
// spill under the budget) and keep the plain bounds.
template <bool kMfma, int kCap, int kR>
constexpr bool kTwoPerSimd = kMfma && kR == 8 && kCap >= 8;

template <bool kMfma, int kCap, int kR, int kFS>
__global__ void __launch_bounds__(64 * kStreamWavesPerBlock) stream_kernel(SweepArgs) {
  using S = Stream<kMfma, kCap, kR, kFS>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kStreamWavesPerBlock][(kCap + 1) * kXRowBytes];
  S::run(kernel_args(), xs[threadIdx.x >> 6]);
}

template <bool kMfma, int kCap, int kR, int kFS>
__global__ void __launch_bounds__(64 * kStreamWavesPerBlock) __attribute__((amdgpu_waves_per_eu(2)))
stream_kernel2(SweepArgs) {
  using S = Stream<kMfma, kCap, kR, kFS>;
  __shared__ __attribute__((aligned(16))) uint8_t xs[kStreamWavesPerBlock][(kCap + 1) * kXRowBytes];
  S::run(kernel_args(), xs[threadIdx.x >> 6]);
}

typedef void (*sweep_fn)(SweepArgs);

template <bool kMfma, int kCap, int kR, int kFS>
static sweep_fn kernel_of() {
  if constexpr (kTwoPerSimd<kMfma, kCap, kR>) return stream_kernel2<kMfma, kCap, kR, kFS>;
  else return stream_kernel<kMfma, kCap, kR, kFS>;
}

template <bool kMfma, int kR, int kFS>
static sweep_fn pick_cls(int cls) {
  switch (cls) {
    case 1: return kernel_of<kMfma, 1, kR, kFS>();
    case 2: return kernel_of<kMfma, 2, kR, kFS>();
    case 4: return kernel_of<kMfma, 4, kR, kFS>();
    case 8: return kernel_of<kMfma, 8, kR, kFS>();
  }
  if constexpr (kMfma)
    if (cls == 16) return kernel_of<kMfma, 16, kR, kFS>();
  return nullptr;
}

// The stream kernels of one format set: GEMV (four row blocks per step) and
// MFMA (four or eight).
template <int kFS>
static sweep_fn pick_set(bool mfma, int cls, int rows) {
  if (!mfma) return rows == 4 ? pick_cls<false, 4, kFS>(cls) : nullptr;
  if (rows == 8) return pick_cls<true, 8, kFS>(cls);
  if (rows == 4) return pick_cls<true, 4, kFS>(cls);
  return nullptr;
}

}  // namespace qg
