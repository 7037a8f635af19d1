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
// One workgroup of kW waves per unit = (job, kW * kRG row blocks, or fewer in
// a re-sliced last round, see rounds_of), whole K:
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
  // 48 rows: the staging would not fit beside the ring at 16 waves, so the
  // outputs are stored from the MFMA layout (64-byte row pieces, once per
  // unit), and each row block's products are scaled right after its MFMAs
  // (half the product registers live, which keeps the kernel in 128 VGPRs)
  static constexpr bool kDirectY = kMPad == 48;
  static constexpr bool kPerBlock = kMPad == 48;
  static constexpr int kYBytes = kDirectY ? 0 : kW * kMPad * kYRow * 4;   // output staging, after the ring
  static constexpr int kRingBytes = kBufs * kBufBytes;
  static constexpr int kLdsBytes = kRingBytes + kYBytes + kMPad * 8;  // then one argmax key per row
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one workgroup");

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

  // What a wave's loads of one unit need: the unit's job (X panel and k
  // extent) and the wave's row blocks.
  struct Unit {
    const uint16_t* X;
    const uint8_t* wbase;  // tile 0 of the wave's first row block (its job's last when the wave has none)
    int64_t ldx;
    int64_t rstride;       // bytes of one row block's tiles
    int K, M, nkt;
    int nr;                // row blocks the loads cover (1 or 2)
    uint32_t soff;         // the lane's scale-copy offset from a tile
    bool busy;             // the wave has rows in the unit (else its code loads are empty and it computes nothing)
  };
  // rb0: the unit's first row block; urb: its row blocks (kUnitRB, or kFine
  // in a re-sliced last round)
  template <int F>
  static __device__ __forceinline__ Unit unit_of(const JobDesc& d, int rb0, int urb, int wave, int lane) {
    constexpr int TB = tile_bytes(F);
    Unit u;
    u.X = d.X;
    u.ldx = d.ldx;
    u.K = d.K;
    u.M = d.M;
    u.nkt = d.nkt;
    u.rstride = (int64_t)d.nkt * TB;
    const int rbw = rb0 + kRG * wave;
    const int nrows = d.nrb - rbw;                     // valid row blocks (may be <= 0)
    u.busy = kRG * wave < urb && nrows > 0;
    const int rbl = nrows > 0 ? rbw : d.nrb - 1;       // waves past the job point at its last block
    u.nr = nrows > 0 ? (nrows < kRG ? nrows : kRG) : 1;
    u.wbase = d.packed + (int64_t)rbl * u.rstride;
    const int srb = ((lane >> 1) & 1) < u.nr ? (lane >> 1) & 1 : u.nr - 1;
    // group 64: a row's two scales are one word, which both lanes of the
    // pair copy (so words 0 and 1 of a row block are the same)
    u.soff = (uint32_t)(srb * u.rstride) + (uint32_t)(F == kFmtG64 ? kScaleOff + 4 * (lane >> 2)
                                                                  : kScaleOff + 8 * (lane >> 2) + 4 * (lane & 1));
    return u;
  }

  // Direct-to-LDS copy of this wave's X slots of k tile kt (clamped to the
  // last) into the buffer at LDS address buf.  Slot rows past M repeat row
  // M-1 and k is clamped into the row (padding groups then add exact zeros:
  // their codes are 0).
  static __device__ __forceinline__ void copy_x(const Unit& u, int kt, uint32_t buf, int wave, int lane) {
    kt = kt < u.nkt ? kt : u.nkt - 1;
#pragma unroll
    for (int i = 0; i < kND; i++) {
      const int s = 64 * (wave * kND + i) + lane;
      const int row = s >> 4;
      const int col = (s & 15) ^ (row & 15);
      const int m = row < u.M ? row : u.M - 1;
      const int kk = kt * kTileK + 8 * col;
      const int k = kk < u.K - 8 ? kk : u.K - 8;
      lds_copy16(u.X + (int64_t)m * u.ldx + k, buf + 1024u * (uint32_t)(wave * kND + i));
    }
  }

  // The code loads of one tile per row block as raw buffer loads over that
  // tile alone (non-temporal).  A tile past the job's last (the prefetch
  // running ahead of the final tiles with no next unit to run into) gets a
  // zero-length range: its loads return zeros without touching memory but
  // still count for the waits.
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
  static __device__ __forceinline__ void copies(const Unit& u, int kx, uint32_t buf, int wave, int lane) {
    constexpr int TB = tile_bytes(F);
    const uint8_t* tile = u.wbase + (int64_t)(kx < u.nkt ? kx : u.nkt - 1) * TB;
    copy_x(u, kx, buf, wave, lane);
    lds_copy4(tile + u.soff, buf + (uint32_t)(kXBytes + 256 * wave));
  }
  template <int F>
  static __device__ __forceinline__ void codes(const Unit& u, int kw, Tiles<F>& t, int lane) {
    constexpr int TB = tile_bytes(F);
    load_w<F>(t, u.wbase + (int64_t)(kw < u.nkt ? kw : u.nkt - 1) * TB, u.rstride, u.nr, u.busy && kw < u.nkt ? TB : 0,
              lane);
  }

  template <typename Fn, int... P>
  static __device__ __forceinline__ void each_p_(Fn&& f, std::integer_sequence<int, P...>) {
    (f(std::integral_constant<int, P>{}), ...);
  }

  // The units this workgroup takes, in order: round i of the grid takes
  // units [i G, (i + 1) G) in alternating directions, so the longest-first
  // order of the jobs evens out across workgroups.
  static __device__ __forceinline__ int unit_index(int i, int G, int b) { return i * G + ((i & 1) ? G - 1 - b : b); }

  // The last, partial round of the grid: when its units all lie in the last
  // job, that job's row blocks from there on are cut into units of kFine row
  // blocks (kFine / kRG busy waves, the rest idle: their code loads are
  // empty and they only copy X and keep the barriers) if they then still fit
  // in one round, so that more workgroups share the round and fewer waves
  // share each SIMD.  Measured with 12-wave workgroups (16-row fine units):
  // the 248320-row verify head at M = 48 (647 units over 256 workgroups)
  // 240 -> 236 us, the 5-bit stack at M = 32 and 48 about 1 % faster.  The
  // gain is small because a wave's row blocks over the whole K take about as
  // long with two busy waves per SIMD as with three.
  static constexpr int kUnitRB = kW * kRG;
  static constexpr int kFine = 8;   // four busy waves, one per SIMD
  static_assert(kFine % (4 * kRG) == 0 && kFine < kUnitRB, "fine units keep the busy waves spread over the SIMDs");
  struct Rounds {
    int total;   // units, the fine ones included
    int fbeg;    // first fine unit (total when there are none)
    int rbf;     // the last job's first row block in fine units
    int jl;      // the last job
  };
  static __device__ __forceinline__ Rounds rounds_of(const QG_CONST JobDesc* D, int njobs, int total, int G) {
    Rounds r;
    r.total = total;
    r.fbeg = total;
    r.rbf = 0;
    r.jl = njobs - 1;
    const int full = total - total % G;
    const JobDesc& l = D[r.jl];
    if (full < total && l.grp_begin <= full) {
      const int rbf = (full - l.grp_begin) * kUnitRB;
      const int nf = (l.nrb - rbf + kFine - 1) / kFine;
      if (nf <= G) {
        r.total = full + nf;
        r.fbeg = full;
        r.rbf = rbf;
      }
    }
    return r;
  }
  // unit u (< R.total): its job j (searched forward from j), first row block
  // and row blocks
  static __device__ __forceinline__ void locate(const QG_CONST JobDesc* D, const Rounds& R, int u, int& j, int& rb0,
                                                int& nrb) {
    if (u >= R.fbeg) {
      j = R.jl;
      rb0 = R.rbf + (u - R.fbeg) * kFine;
      nrb = kFine;
      return;
    }
    while (u >= D[j].grp_end) j++;
    rb0 = (u - D[j].grp_begin) * kUnitRB;
    nrb = kUnitRB;
  }

  // This workgroup's units from round i on while their jobs have format F;
  // returns the first round it did not run (a unit of another format, or
  // past the end).  Within such a run the prefetch does not drain between
  // units: the last k tiles of a unit issue the first tiles of the next one
  // (whose job must also be format F, with the current job's k-tile count a
  // multiple of kDepth, so its tiles land in the ring slots and code
  // buffers its loop reads them from).  The loads past a unit's end run in
  // exactly the order a unit's own start would issue them, so the next
  // unit's wait counts hold unchanged.  Y leaves through LDS staging of its
  // own, so nothing waits for the ring at a unit's end.
  template <int F>
  static __device__ __forceinline__ int run_units(const QG_CONST JobDesc* D, int& j, int i, const Rounds& R,
                                                  uint8_t* xs, uint32_t xs_lds, int tid) {
    constexpr int TB = tile_bytes(F);
    (void)TB;
    // Issue order: codes of tile 0, then per tile t (the start for
    // t < kDepth - 1, else the end of tile t - kDepth + 1): copies of tile t,
    // codes of tile t + 1.  The copies of tile kt are therefore complete once
    // at most this many younger loads of this wave are outstanding: the codes
    // of tile kt + 1 and kDepth - 2 whole tiles.
    constexpr int kXWait = kLoadsW<F> + (kDepth - 2) * kLoadsTile<F>;
    static_assert(kXWait < 64, "vmcnt range");
    // s_waitcnt encoding (gfx9): vmcnt low 4 bits, expcnt 7, lgkmcnt 15, vmcnt high 2 bits
    constexpr int kXWaitImm = (kXWait & 15) | (7 << 4) | (15 << 8) | ((kXWait >> 4) << 14);
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    uint8_t* ystage = xs + kRingBytes;
    unsigned long long* best = (unsigned long long*)(ystage + kYBytes);
    // A fragment of group j, m block mb: row 16 mb + (lane mod 16), chunk
    // 4 j + lane / 16, at its swizzled slot
    const int mr = lane & 15, c = lane >> 4;
    uint32_t aoff[4];
#pragma unroll
    for (int g = 0; g < 4; g++) aoff[g] = (uint32_t)(256 * mr + 16 * ((4 * g + c) ^ mr));
    const uint32_t sread = (uint32_t)(kXBytes + 256 * wave + 16 * mr);
    const f4_t zero = {0.f, 0.f, 0.f, 0.f};
    Tiles<F> buf[kDepth];
    // p = 0 .. kDepth - 1 as compile-time constants (the code buffers stay in registers)
    auto each_p = [&](auto&& f) { each_p_(f, std::make_integer_sequence<int, kDepth>{}); };
    bool primed = false;  // this unit's first tiles were issued by the previous one
    for (;; i++) {
      const int u = unit_index(i, G, b);
      if (u >= R.total) break;
      int rb0, urb;
      locate(D, R, u, j, rb0, urb);
      const QG_CONST JobDesc& d = D[j];
      if (d.fmt != F) break;
      const Unit cur = unit_of<F>(d, rb0, urb, wave, lane);
      // the next unit, when its first tiles can be issued from this one
      const int un = unit_index(i + 1, G, b);
      int jn = j, rbn = 0, urbn = 0;
      if (un < R.total) locate(D, R, un, jn, rbn, urbn);
      const bool chain = un < R.total && D[jn].fmt == F && d.nkt % kDepth == 0;
      const Unit nxt = chain ? unit_of<F>(D[jn], rbn, urbn, wave, lane) : cur;
      const int nkt = d.nkt;
      if (!primed) {
        __builtin_amdgcn_sched_barrier(0);
        codes<F>(cur, 0, buf[0], lane);
#pragma unroll
        for (int p = 0; p < kDepth - 1; p++) {
          __builtin_amdgcn_sched_barrier(0);
          copies<F>(cur, p, xs_lds + (uint32_t)(p * kBufBytes), wave, lane);
          __builtin_amdgcn_sched_barrier(0);
          codes<F>(cur, p + 1, buf[p + 1], lane);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      f4_t acc[kRG][kMb];
#pragma unroll
      for (int r = 0; r < kRG; r++)
#pragma unroll
        for (int mb = 0; mb < kMb; mb++) acc[r][mb] = zero;
      // one k tile: wait for its copies, then its MFMAs and scales
      auto tile = [&](auto pc_, int kt) {
        constexpr int p = decltype(pc_)::value;
        // this wave's copies of tile kt have landed; after the barrier every
        // wave's have, and every wave is done with tile kt - 1
        __builtin_amdgcn_s_waitcnt(kXWaitImm);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        (void)kt;
        // a wave with no rows in the unit only copies and keeps the barriers
        if (!cur.busy) return;
        const uint8_t* xb = xs + p * kBufBytes;
        // scales of row mr: words 0, 1 of row block 0, then of row block 1
        const u4_t sc = *(const u4_t*)(xb + sread);
        f4_t pr[kRG][kMb];
        // group by group: the A fragments of group g serve all kRG row blocks
#pragma unroll
        for (int g = 0; g < 4; g++) {
          h8_t a[kMb];
#pragma unroll
          for (int mb = 0; mb < kMb; mb++) a[mb] = lds_h8(xb + aoff[g] + 4096 * mb);
          // every MFMA of the group is issued before the first of its
          // results is scaled, so the matrix-core latency overlaps
          // group 64: the odd half of a group accumulates onto the even
          // half's products, which are scaled once, after it
          constexpr bool kG64 = F == kFmtG64;
          if constexpr (kPerBlock && !kG64) {
#pragma unroll
            for (int r = 0; r < kRG; r++) {
              const h8_t q = unpack_chunk<F>(buf[p].c[r][g], side_word<F>(buf[p].h[kSide<F> ? r : 0]), g);
              f4_t pq[kMb];
#pragma unroll
              for (int mb = 0; mb < kMb; mb++) pq[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], q, zero, 0, 0, 0);
              const uint32_t sp = sc[2 * r + (g >> 1)];
              const float sj = (g & 1) ? scale_f32<1>(sp) : scale_f32<0>(sp);
#pragma unroll
              for (int mb = 0; mb < kMb; mb++)
#pragma unroll
                for (int e = 0; e < 4; e++) acc[r][mb][e] = __builtin_fmaf(sj, pq[mb][e], acc[r][mb][e]);
            }
            continue;
          }
#pragma unroll
          for (int r = 0; r < kRG; r++) {
            const h8_t q = unpack_chunk<F>(buf[p].c[r][g], side_word<F>(buf[p].h[kSide<F> ? r : 0]), g);
#pragma unroll
            for (int mb = 0; mb < kMb; mb++)
              pr[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mb], q, (kG64 && (g & 1)) ? pr[r][mb] : zero, 0, 0, 0);
          }
          if (!kG64 || (g & 1)) {
#pragma unroll
            for (int r = 0; r < kRG; r++) {
              // group 32: word g / 2 of the row block holds groups (g & ~1, g | 1);
              // group 64: word 0 holds halves (0, 1)
              const uint32_t sp = sc[2 * r + (kG64 ? 0 : g >> 1)];
              const int hi = kG64 ? g >> 1 : g & 1;
              const float sj = hi ? scale_f32<1>(sp) : scale_f32<0>(sp);
#pragma unroll
              for (int mb = 0; mb < kMb; mb++)
#pragma unroll
                for (int e = 0; e < 4; e++) acc[r][mb][e] = __builtin_fmaf(sj, pr[r][mb][e], acc[r][mb][e]);
            }
          }
        }
      };
      // copies of tile kt + kDepth - 1 into the buffer of tile kt - 1 (every
      // wave is past it), codes of tile kt + kDepth: of this unit, where past
      // its last k tile they (kept for exact wait counts) re-read the last
      // tile into buffers no wave reads again
      auto refill = [&](auto pc_, int kt) {
        constexpr int p = decltype(pc_)::value;
        __builtin_amdgcn_sched_barrier(0);
        copies<F>(cur, kt + kDepth - 1, xs_lds + (uint32_t)(((p + kDepth - 1) % kBufs) * kBufBytes), wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        codes<F>(cur, kt + kDepth, buf[p], lane);
        __builtin_amdgcn_sched_barrier(0);
      };
      const int kmain = chain ? nkt - kDepth : nkt;
      for (int kt0 = 0; kt0 < kmain; kt0 += kDepth) {
        each_p([&](auto pc_) {
          constexpr int p = decltype(pc_)::value;
          const int kt = kt0 + p;
          if (kt < nkt) tile(pc_, kt);
          refill(pc_, kt);
        });
      }
      if (chain) {
        // the last kDepth tiles (nkt is a multiple of kDepth): their loads
        // past the end are the next unit's first tiles, in the order its own
        // start would issue them (copies of tile t into ring slot t, codes
        // of tile t into buf[t])
        each_p([&](auto pc_) {
          constexpr int p = decltype(pc_)::value;
          tile(pc_, nkt - kDepth + p);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (p == 0) copies<F>(cur, nkt - 1, xs_lds + (uint32_t)((kDepth - 1) * kBufBytes), wave, lane);
          else copies<F>(nxt, p - 1, xs_lds + (uint32_t)((p - 1) * kBufBytes), wave, lane);
          __builtin_amdgcn_sched_barrier(0);
          codes<F>(nxt, p, buf[p], lane);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      const int rbw = rb0 + kRG * wave;
      if (cur.busy) store_y(d, acc, rbw, ystage + kMPad * kYRow * 4 * wave, best, lane);
      if (d.keys) {
        // the unit's argmax keys are complete and go to the job's keys
        __syncthreads();
        if (tid < d.M) {
          const unsigned long long k = best[tid];
          if (k != 0ull) key_max(d.keys + (blockIdx.x % kKeyCopies) * kKeyRows + tid, k);
          best[tid] = 0ull;
        }
      }
      if (!chain) {
        // the loads past the end re-read tiles into ring slots: every one has
        // landed and every wave is past the ring before another start
        __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
        __syncthreads();
      }
      primed = chain;
    }
    return i;
  }

  // The wave's outputs (rows m < kMPad, n = 16 rbw .. 16 rbw + 31) go through
  // its slice of the LDS ring, row-major with 16-byte chunks swizzled by
  // m mod 8, and leave as whole 128-byte row segments: lane L of store t
  // writes row 8 t + L / 8, outputs 4 (L mod 8) .. + 3.
  static __device__ __forceinline__ void store_y(const JobDesc& d, const f4_t (&acc)[kRG][kMb], int rbw,
                                                 uint8_t* st, unsigned long long* best, int lane) {
    if constexpr (kDirectY) {
      // lane (c, mr) holds rows 16 mb + 4 c + i of output n = 16 (rbw + r) + mr;
      // the lane index is opaque so the addresses stay in the unit loop
      asm volatile("" : "+v"(lane));
      const int mr = lane & 15, c = lane >> 4;
      QG_GLOBAL float* Y = (QG_GLOBAL float*)d.Y;
#pragma unroll
      for (int mb = 0; mb < kMb; mb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int m = 16 * mb + 4 * c + i;
          unsigned long long k = 0ull;
#pragma unroll
          for (int r = 0; r < kRG; r++) {
            const int n = kTileRows * (rbw + r) + mr;
            if (m < d.M && n < d.N && Y) Y[(int64_t)m * d.ldy + n] = acc[r][mb][i];
            if (d.keys && n < d.N) k = umax64(k, logit_key(acc[r][mb][i], n));
          }
          if (d.keys) {
            // verify head: the best of the row's 32 outputs (16 lanes), into
            // the workgroup's key of row m
            k = lanes_max<1, 16>(k);
            if (mr == 0 && m < d.M && k != 0ull)
              __hip_atomic_fetch_max(best + m, k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      return;
    }
    // Left to itself the compiler hoists the staging addresses below (two
    // dozen per lane) out of the unit loop and, short of registers, spills
    // them: at 48 rows with 12-wave workgroups every wave then wrote and read
    // back about 6 KB of scratch before its first loads, and the first unit
    // started about 7 us after the kernel.  An opaque copy of the lane index
    // keeps them in the loop (recomputed once per unit, no scratch; the
    // verify head at M = 48 237 -> 229 us then), and at 32 rows it is what
    // lets four waves per SIMD fit in 128 VGPRs.  At 64 rows the hoisted
    // form spills at most a few words and measured about 1 % faster.
    if constexpr (kMPad <= 48) asm volatile("" : "+v"(lane));
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
__global__ void __launch_bounds__(64 * group_waves(kMPad)) __attribute__((amdgpu_waves_per_eu(group_waves(kMPad) / 4)))
group_kernel(SweepArgs) {
  using S = Group<kMPad>;
  __shared__ __attribute__((aligned(1024))) uint8_t xs[S::kLdsBytes];
  const uint32_t xs_lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)xs;
  const QG_CONST SweepArgs& args = kernel_args();
  const QG_CONST JobDesc* D = job_table(args);
  const int tid = threadIdx.x;
  // argmax keys of the verify head start at 0 (the first unit's barriers
  // order this before any use)
  if (tid < kMPad) ((unsigned long long*)(xs + S::kRingBytes + S::kYBytes))[tid] = 0ull;
  int j = 0;
  const typename S::Rounds R = S::rounds_of(D, args.njobs, args.total, (int)gridDim.x);
  // runs of units of one format (a launch mixes formats only by job)
  for (int i = 0;;) {
    const int u = S::unit_index(i, (int)gridDim.x, (int)blockIdx.x);
    if (u >= R.total) break;
    int rb0, urb;
    S::locate(D, R, u, j, rb0, urb);
    const int f = D[j].fmt;
    if (f == kFmtQ4) i = S::template run_units<kFmtQ4>(D, j, i, R, xs, xs_lds, tid);
    else if (!kAll || f == kFmtQ5) i = S::template run_units<kFmtQ5>(D, j, i, R, xs, xs_lds, tid);
    else if (f == kFmtG64) i = S::template run_units<kFmtG64>(D, j, i, R, xs, xs_lds, tid);
    else i = S::template run_units<kFmtZP>(D, j, i, R, xs, xs_lds, tid);
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
