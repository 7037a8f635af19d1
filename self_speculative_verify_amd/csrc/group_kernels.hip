// gfx950 group kernel of the quantized weight sweep: panels of 17..64 rows.
//
// The method (Quasar/q27 wiki): decode streams every quantized linear weight
// once per step ("decode physics" paragraph) and one weight read serves all
// draft positions of all slots (intro bullets on the fused verify sweep;
// "Batching & prefill notes" on the verify GEMM flat in the weights).
#include "sweep_device.h"

namespace qg {

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
group_kernel(SweepArgs) {
  using S = Group<kMPad>;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[S::kLdsBytes];
  const uint32_t xs_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)xs;
  const QG_CONST SweepArgs& args = kernel_args();
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

typedef void (*sweep_fn)(SweepArgs);

// padded rows 32, 48, 64; all: some job uses a format other than the 4- and
// 5-bit group-32 ones
sweep_fn pick_group(int cls, bool all) {
  switch (cls) {
    case 32: return all ? group_kernel<32, true> : group_kernel<32, false>;
    case 48: return all ? group_kernel<48, true> : group_kernel<48, false>;
    case 64: return all ? group_kernel<64, true> : group_kernel<64, false>;
  }
  return nullptr;
}

}  // namespace qg
