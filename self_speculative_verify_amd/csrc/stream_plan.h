// Work planning of the stream kernels (panels of at most 16 rows): which
// steps a wave owns, in which order it takes them and which of its row-group
// sums it writes to Y, stores as a partial or reads back.  Host and device
// code: the kernels run it per wave, and the host-side checks run the same
// code for every wave of a launch.
//
// Work is a flat sequence of steps (job, row group, k tile); a row group is R
// consecutive 16-row blocks and one step reads the R tiles of its row group
// at one k tile.  Units of weight bytes (a step weighs its tile bytes / 128)
// are cut into nwaves equal contiguous ranges (q units each, one more for the
// first rem waves); a wave owns the steps whose first unit lies in its range,
// at least one (q >= the largest step weight).
//
// A row group whose steps fall into several ranges is "split".  Its last
// contributor (the wave holding its last step) reads it: every other
// contributor stores its partial sums into a slot of its own (slot 1 for the
// first contributor, whose piece is its range's last row group; slot 0 for
// the middle ones, whose whole range lies in the row group), and the last one
// adds them in wave order (k order) with its own last and writes Y.  A wave
// takes its pieces in the order
//   0: the tail piece it writes (its last row group, split past its range)
//   1: its whole range, when that lies inside one row group split at both ends
//   2: its whole row groups (Y written directly)
//   3: the head piece it reads (its first row group, split before its range)
// so that partials are written early and read late.  A reader waits only for
// waves of lower index, which are dispatched no later than itself, and
// writers wait for nothing: the waits always end, whatever part of the grid
// is resident.
#pragma once

#include "qgemm_internal.h"

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

// Every function here is force-inlined: a call would need the kernel
// argument in memory, and the compiler then copies the whole argument into
// private memory.  They take scalars, never the argument struct itself.
#define QG_PLAN __host__ __device__ __forceinline__

namespace qg {

// The kernels reach their argument only through the kernarg segment (a
// pointer in the constant address space), never through the C++ parameter:
// a reference to the parameter lets the compiler copy the whole argument into
// private memory, and the inline job table must be read where it lies.
QG_PLAN const QG_CONST JobDesc* job_table(const QG_CONST SweepArgs& a) {
  return a.table ? (const QG_CONST JobDesc*)a.table : (const QG_CONST JobDesc*)&a.inl[0];
}
#if defined(__HIP_DEVICE_COMPILE__)
// the launch's SweepArgs: the kernels' only explicit argument, at offset 0
__device__ __forceinline__ const QG_CONST SweepArgs& kernel_args() {
  return *(const QG_CONST SweepArgs*)__builtin_amdgcn_kernarg_segment_ptr();
}
#elif defined(__HIPCC__)
__device__ const SweepArgs& kernel_args();  // host pass: declared, never emitted
#endif

// Wave w takes units [start(w), start(w + 1)); the wave holding unit f.
QG_PLAN int stream_start_of(int w, int q, int rem) { return w * q + (w < rem ? w : rem); }
QG_PLAN int stream_wave_of(int f, int q, int rem) {
  const int edge = rem * (q + 1);
  return f < edge ? f / (q + 1) : rem + (f - edge) / q;
}

// The wave's phases.  A position is (job j, local step s = rg * nkt + kt);
// a run ending at a job's last step ends at (j + 1, 0).  With A the first
// step of the range, H the end of its first row group (or of the range, when
// the range lies in one row group), T the first step of the last row group
// and E the end of the range: phase 0 is [T, E), phases 1 and 3 [A, H),
// phase 2 [head ? H : A, tail ? T : E).  Bits 0..3 of mask: phases present;
// bits 4, 5: first row group split at the head, last one at the tail.
struct StreamPhases {
  int mask;
  int jA, sA, jH, sH, jT, sT, jE, sE;
};

// Scalar cursor: phase (4: done), job, row group, k tile, and what the loads
// of a step need of its job (kept in scalar registers rather than read from
// the job table every step).
struct StreamPos {
  int ph, j, rg, kt;
  int nkt, nrg, nrb, fmt;
  uint32_t nkt_m;
  int nkt_sh;
  const uint8_t* packed;
  const uint16_t* X;
  int ldx, M, K;
};

// the first present phase after ph (4: none)
QG_PLAN int stream_next_phase(const StreamPhases& P, int ph) {
  const unsigned m = ((unsigned)P.mask & 15u) >> (ph + 1);
  return m ? ph + 1 + __builtin_ctz(m) : 4;
}
// (values are selected, never references: a select between addresses would
// keep the struct in memory on the device)
QG_PLAN void stream_phase_begin(const StreamPhases& P, int ph, int& j, int& s) {
  const bool h = (P.mask >> 4) & 1;
  const int jA = P.jA, sA = P.sA, jH = P.jH, sH = P.sH, jT = P.jT, sT = P.sT;
  const bool t0 = ph == 0, th = ph == 2 && h;
  j = t0 ? jT : th ? jH : jA;
  s = t0 ? sT : th ? sH : sA;
}
QG_PLAN void stream_phase_end(const StreamPhases& P, int ph, int& j, int& s) {
  const bool t = (P.mask >> 5) & 1;
  const int jH = P.jH, sH = P.sH, jT = P.jT, sT = P.sT, jE = P.jE, sE = P.sE;
  const bool e = ph == 0 || (ph == 2 && !t), h = ph == 1 || ph == 3;
  j = e ? jE : h ? jH : jT;
  s = e ? sE : h ? sH : sT;
}

// s / nkt of job j (0 <= s < 2^31), by the job's multiplier
QG_PLAN int div_nkt(int s, uint32_t m, int sh) { return (int)(((uint64_t)(uint32_t)s * m) >> sh); }

QG_PLAN void stream_load_job(StreamPos& c, const QG_CONST JobDesc* D, int j) {
  c.j = j;
  c.nkt = D[j].nkt;
  c.nkt_m = D[j].nkt_m;
  c.nkt_sh = D[j].nkt_sh;
  c.nrg = D[j].nrg;
  c.nrb = D[j].nrb;
  c.fmt = D[j].fmt;
  c.packed = D[j].packed;
  c.X = D[j].X;
  c.ldx = (int)D[j].ldx;  // <= 2^24 (host check)
  c.M = D[j].M;
  c.K = D[j].K;
}
QG_PLAN void stream_seek(StreamPos& c, const QG_CONST JobDesc* D, int j, int s) {
  stream_load_job(c, D, j);
  c.rg = div_nkt(s, c.nkt_m, c.nkt_sh);
  c.kt = s - c.rg * c.nkt;
}
QG_PLAN void stream_start(StreamPos& c, const QG_CONST JobDesc* D, const StreamPhases& P) {
  c.ph = stream_next_phase(P, -1);
  int j, s;
  stream_phase_begin(P, c.ph, j, s);
  stream_seek(c, D, j, s);
}

// One step forward; at a phase end, on to the next phase (c.ph == 4: done,
// with c.j possibly njobs).
QG_PLAN void stream_advance(StreamPos& c, const QG_CONST JobDesc* D, const StreamPhases& P,
                                               int njobs) {
  if (++c.kt == c.nkt) {
    c.kt = 0;
    if (++c.rg == c.nrg) {
      c.rg = 0;
      if (c.j + 1 < njobs) stream_load_job(c, D, c.j + 1);
      else c.j++;
    }
  }
  int ej, es;
  stream_phase_end(P, c.ph, ej, es);
  if (c.j == ej && c.rg * c.nkt + c.kt == es) {
    c.ph = stream_next_phase(P, c.ph);
    if (c.ph < 4) {
      int j, s;
      stream_phase_begin(P, c.ph, j, s);
      stream_seek(c, D, j, s);
    }
  }
}

// The partition and job lookup of a launch (scalars of its arguments).
struct StreamGrid {
  const int32_t* index;  // with a job table: uend of every job, then the first job of every bucket
  int njobs, bshift, q, rem;
};

// Job holding unit u: a bucket index into the uend list when the jobs come
// from a table, else a scan of the (at most kMaxInline) inline jobs.
QG_PLAN int stream_job_of(const StreamGrid& g, const QG_CONST JobDesc* D, int u) {
  int j = 0;
  if (g.index) {
    const QG_CONST int32_t* ends = (const QG_CONST int32_t*)g.index;
    j = ends[g.njobs + (u >> g.bshift)];
    while (u >= ends[j]) j++;
  } else {
    while (u >= D[j].uend) j++;
  }
  return j;
}

// The phases of wave gw's range [a, b) (a non-empty set of steps).
// kOne: the launch has one job, so both lookups are job 0 and its
// descriptor's loads wait for no search (a launch of one matrix, the common
// case, reaches its first load sooner: gate+up M = 1 22.0 -> 21.6 us, the
// 1024 x 1024 sweep 7.0 -> 6.7 us).
template <bool kOne = false>
QG_PLAN void stream_plan(StreamPhases& P, const StreamGrid& g, const QG_CONST JobDesc* D, int gw, int a, int b) {
  // first step (jA, sA): the first step of job jA whose first unit is >= a
  int jA = kOne ? 0 : stream_job_of(g, D, a);
  const int wA = unit_weight(D[jA].fmt), dA = a - D[jA].ubeg;
  int sA = dA <= 0 ? 0 : div_unit_weight(dA + wA - 1, D[jA].fmt);
  if (sA == D[jA].nrg * D[jA].nkt) {
    jA++;
    sA = 0;
  }
  // last step (jL, sL): the last step whose first unit is <= b - 1
  const int jL = kOne ? 0 : stream_job_of(g, D, b - 1);
  const int sL = div_unit_weight(b - 1 - D[jL].ubeg, D[jL].fmt);
  const int nktA = D[jA].nkt, nktL = D[jL].nkt;
  const int rgA = div_nkt(sA, D[jA].nkt_m, D[jA].nkt_sh), rgL = div_nkt(sL, D[jL].nkt_m, D[jL].nkt_sh);
  const bool head = sA != rgA * nktA;             // first row group began before a
  const bool tail = sL != rgL * nktL + nktL - 1;  // last row group runs past b
  const bool one = jA == jL && rgA == rgL;        // the range lies in one row group
  (void)gw;
  P.jA = jA;
  P.sA = sA;
  // E: (jL, sL) + 1, normalized
  P.jE = jL;
  P.sE = sL + 1;
  if (P.sE == D[jL].nrg * nktL) {
    P.jE = jL + 1;
    P.sE = 0;
  }
  if (one) {
    P.jH = P.jE;
    P.sH = P.sE;
  } else {
    P.jH = jA;
    P.sH = (rgA + 1) * nktA;
    if (P.sH == D[jA].nrg * nktA) {
      P.jH = jA + 1;
      P.sH = 0;
    }
  }
  P.jT = jL;
  P.sT = one ? sA : rgL * nktL;
  int m = (head ? 16 : 0) | (tail ? 32 : 0);
  if (one) {
    // whole (body), or a piece of a split row group: the tail of the range
    // continues it (the first contributor writes it, a middle one too), or
    // the range holds its last step (read here)
    m |= !head && !tail ? 4 : !tail ? 8 : head ? 2 : 1;
  } else {
    // the first row group ends inside the range: its head piece is read here
    if (tail) m |= 1;
    if (head) m |= 8;
    // body: from the end of the head piece to the start of the tail piece
    const int jb0 = head ? P.jH : jA, sb0 = head ? P.sH : sA;
    const int jb1 = tail ? jL : P.jE, sb1 = tail ? P.sT : P.sE;
    if (jb0 != jb1 || sb0 != sb1) m |= 4;
  }
  P.mask = m;
}

// Contributors wf .. wl of row group rg of job j.
QG_PLAN void stream_contributors(int q, int rem, const QG_CONST JobDesc* D, int j, int rg,
                                                    int& wf, int& wl) {
  const int wt = unit_weight(D[j].fmt), nkt = D[j].nkt;
  const int u0 = D[j].ubeg + rg * nkt * wt;
  wf = stream_wave_of(u0, q, rem);
  wl = stream_wave_of(u0 + (nkt - 1) * wt, q, rem);
}

}  // namespace qg
