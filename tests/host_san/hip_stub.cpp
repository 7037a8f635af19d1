// Host-only stand-ins for the HIP runtime calls and the kernel launchers that
// the library's host code (qgemm_host.cpp, attn_host.cpp) makes, for building
// that code under AddressSanitizer and UndefinedBehaviorSanitizer on a machine
// without a GPU.  Every "device" buffer is then host memory, so each
// launcher stand-in touches the memory its kernel would touch -- the first
// and last element of every region the kernel reads or writes, as the kernel
// computes it from its arguments -- and checks the arguments' invariants.  A
// workspace sized too small, a job table written past its region or a kernel
// argument that points outside its buffer then shows up as a sanitizer error
// or a failed check (exit status 3).  Stream capture records the launches and
// a graph launch replays them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <functional>
#include <vector>

#include "attn_internal.h"
#include "qgemm.h"
#include "qgemm_internal.h"
#include "stream_plan.h"

long g_launches = 0;      // kernels run or recorded, for the fuzz driver
long g_big_launches = 0;  // of which sweeps with the big step shape
size_t g_scratch_bytes = (size_t)256 << 10;  // the stand-in scratch of the allocation-free sweep

#define CHECK(c)                                                                    \
  do {                                                                              \
    if (!(c)) {                                                                     \
      std::fprintf(stderr, "stub check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
      std::exit(3);                                                                 \
    }                                                                               \
  } while (0)

namespace {

// read or write one byte (volatile, so the access is kept)
void touch_r(const void* p) { (void)*(const volatile uint8_t*)p; }
void touch_w(void* p) { *(volatile uint8_t*)p = *(volatile uint8_t*)p; }
// first and last byte of [p, p + n)
void span_r(const void* p, size_t n) {
  CHECK(p != nullptr && n > 0);
  touch_r(p);
  touch_r((const uint8_t*)p + n - 1);
}
void span_w(void* p, size_t n) {
  CHECK(p != nullptr && n > 0);
  touch_w(p);
  touch_w((uint8_t*)p + n - 1);
}

struct Graph {
  std::vector<std::function<void()>> nodes;
};
hipStream_t g_capturing = nullptr;
Graph* g_graph = nullptr;

void run_or_record(hipStream_t s, std::function<void()> f) {
  g_launches++;
  if (g_capturing && s == g_capturing) {
    g_graph->nodes.push_back(std::move(f));
    return;
  }
  CHECK(!g_capturing || s != g_capturing);
  f();
}

int64_t tiles_bytes(const qg::JobDesc& d) { return (int64_t)d.nrb * d.nkt * qg::tile_bytes(d.fmt); }

// Every wave of a stream launch through the kernels' own planning code
// (stream_plan.h): each step is taken by exactly one wave, each row group's
// sums reach Y exactly once -- directly when one wave holds all its steps,
// else by its last contributor, which reads the partials of all other
// contributors (slot 1 of the first, slot 0 of the middle ones), each written
// exactly once -- and no wave writes a slot twice.
void stream_schedule_check(const qg::SweepArgs& a, const std::vector<qg::JobDesc>& D) {
  std::vector<int64_t> first(a.njobs + 1, 0);
  for (int j = 0; j < a.njobs; j++) first[j + 1] = first[j] + (int64_t)D[j].nrg * D[j].nkt;
  std::vector<uint8_t> taken((size_t)first[a.njobs], 0);
  // per row group: [Y writes, reads, reader wave]; per (wave, slot): row group written
  std::vector<int64_t> rgbase(a.njobs + 1, 0);
  for (int j = 0; j < a.njobs; j++) rgbase[j + 1] = rgbase[j] + D[j].nrg;
  std::vector<int> ywrites((size_t)rgbase[a.njobs], 0), reader((size_t)rgbase[a.njobs], -1);
  std::vector<int64_t> slot_rg((size_t)a.nwaves * 2, -1);
  for (int w = 0; w < a.nwaves; w++) {
    const int u0 = qg::stream_start_of(w, a.q, a.rem), u1 = u0 + a.q + (w < a.rem ? 1 : 0);
    qg::StreamPhases P;
    const qg::StreamGrid g = {a.index, a.njobs, a.bshift, a.q, a.rem};
    qg::stream_plan(P, g, D.data(), w, u0, u1);
    CHECK((P.mask & 15) != 0);
    if (a.njobs == 1) {
      // the one-job plan the kernels take for such launches: the same phases
      qg::StreamPhases P1;
      qg::stream_plan<true>(P1, g, D.data(), w, u0, u1);
      CHECK(P1.mask == P.mask && P1.jA == P.jA && P1.sA == P.sA && P1.jH == P.jH && P1.sH == P.sH &&
            P1.jT == P.jT && P1.sT == P.sT && P1.jE == P.jE && P1.sE == P.sE);
    }
    qg::StreamPos c;
    qg::stream_start(c, D.data(), P);
    int steps = 0;
    while (c.ph < 4) {
      CHECK(c.j >= 0 && c.j < a.njobs && c.rg >= 0 && c.rg < D[c.j].nrg && c.kt >= 0 && c.kt < D[c.j].nkt);
      const qg::JobDesc& d = D[c.j];
      const int64_t s = (int64_t)c.rg * d.nkt + c.kt;
      // the step's first unit lies in the wave's range
      const int64_t fu = d.ubeg + s * qg::unit_weight(d.fmt);
      CHECK(fu >= u0 && fu < u1);
      CHECK(taken[first[c.j] + s]++ == 0);
      steps++;
      const int j = c.j, rg = c.rg, ph = c.ph;
      const bool rg_end = c.kt == d.nkt - 1;
      qg::stream_advance(c, D.data(), P, a.njobs);
      if (rg_end || c.ph != ph) {
        const int64_t r = rgbase[j] + rg;
        if (ph == 2) {
          ywrites[r]++;
        } else if (ph == 3) {
          ywrites[r]++;
          CHECK(reader[r] == -1);
          reader[r] = w;
        } else {
          const int slot = ph == 0 ? 1 : 0;
          CHECK(slot_rg[2 * w + slot] == -1);
          slot_rg[2 * w + slot] = r;
        }
      }
    }
    CHECK(steps >= 1);
  }
  for (size_t i = 0; i < taken.size(); i++) CHECK(taken[i] == 1);
  std::vector<int> reads(a.nwaves * 2, 0);
  for (int j = 0; j < a.njobs; j++)
    for (int rg = 0; rg < D[j].nrg; rg++) {
      const int64_t r = rgbase[j] + rg;
      CHECK(ywrites[r] == 1);
      int wf, wl;
      qg::stream_contributors(a.q, a.rem, D.data(), j, rg, wf, wl);
      if (wf == wl) {
        CHECK(reader[r] == -1);
        continue;
      }
      CHECK(reader[r] == wl);
      CHECK(slot_rg[2 * wf + 1] == r);
      reads[2 * wf + 1]++;
      for (int src = wf + 1; src < wl; src++) {
        CHECK(slot_rg[2 * src] == r);
        reads[2 * src]++;
      }
    }
  // every written slot is read exactly once (and so left empty)
  for (int i = 0; i < a.nwaves * 2; i++) CHECK((slot_rg[i] >= 0) == (reads[i] == 1) && reads[i] <= 1);
}

// What one sweep launch touches, from its arguments alone.
void sweep_footprint(int kind, int cls, int fs, int rows, const qg::SweepArgs a, int grid) {
  CHECK(a.njobs >= 1 && a.total >= 1 && grid >= 1);
  std::vector<qg::JobDesc> D(a.njobs);
  if (a.table) {
    CHECK(a.njobs > qg::kMaxInline);
    span_r(a.table, a.njobs * sizeof(qg::JobDesc));
    std::memcpy(D.data(), a.table, a.njobs * sizeof(qg::JobDesc));
  } else {
    CHECK(a.njobs <= qg::kMaxInline && a.index == nullptr);
    for (int j = 0; j < a.njobs; j++) D[j] = a.inl[j];
  }
  const bool stream = kind != 2;
  CHECK(rows == 4 || (rows == 8 && kind == 1));
  const int R = rows;
  int seen = 0;
  for (int j = 0; j < a.njobs; j++) {
    const qg::JobDesc& d = D[j];
    CHECK(qg::valid_fmt(d.fmt) && d.M >= 1 && d.M <= QGEMM_MAX_M && d.N >= 1 && d.K >= 32);
    CHECK(d.nkt == (d.K + qg::kTileK - 1) / qg::kTileK && d.nrb == (d.N + qg::kTileRows - 1) / qg::kTileRows);
    seen |= d.fmt == qg::kFmtQ4 ? 1 : d.fmt == qg::kFmtQ5 ? 2 : d.fmt == qg::kFmtG64 ? 4 : 8;
    span_r(d.packed, (size_t)tiles_bytes(d));
    span_r(d.X, (size_t)((int64_t)(d.M - 1) * d.ldx + d.K) * 2);
    if (d.Y) span_w(d.Y, (size_t)((int64_t)(d.M - 1) * d.ldy + d.N) * 4);
    if (d.keys) span_w(d.keys, (size_t)qg::kKeyCopies * qg::kKeyRows * 8);
    if (stream) {
      CHECK(d.M <= cls && cls <= 16);
      // units of the jobs tile [0, total) in order
      CHECK(d.ubeg == (j == 0 ? 0 : D[j - 1].uend));
      CHECK(d.uend - d.ubeg == (int64_t)d.nrg * d.nkt * qg::unit_weight(d.fmt));
      CHECK(d.nrg == (d.nrb + R - 1) / R);
    } else {
      CHECK(d.M <= cls && cls >= 17 && cls <= 64);
      CHECK(d.grp_begin == (j == 0 ? 0 : D[j - 1].grp_end));
      const int per = qg::group_waves(cls) * qg::kGroupRows;
      CHECK(d.grp_end - d.grp_begin == (d.nrb + per - 1) / per);
    }
  }
  CHECK(seen == fs);
  if (stream) {
    CHECK(D[a.njobs - 1].uend == a.total);
    CHECK(a.nwaves >= 1 && (int64_t)grid * qg::kStreamWavesPerBlock >= a.nwaves);
    CHECK(a.q == a.total / a.nwaves && a.rem == a.total % a.nwaves);
    CHECK(a.q >= qg::kMaxUnitWeight || a.nwaves == 1);  // every wave holds at least one step
    CHECK(a.spin_limit > 0);
    CHECK(a.slot_bytes == qg::stream_slot_bytes(a.nwaves, R, kind == 1, cls));
    span_w(a.slots, (size_t)a.slot_bytes);
    // the kernels read a non-zero slot word as a written partial: every slot
    // is empty (zero) when a launch starts
    {
      const uint32_t* w = (const uint32_t*)a.slots;
      for (int64_t i = 0; i < a.slot_bytes / 4; i++) CHECK(w[i] == 0u);
    }
    if (a.index) {
      // uend of every job, then the job holding the first unit of each bucket
      const int64_t nb = ((int64_t)a.total >> a.bshift) + 1;
      span_r(a.index, (size_t)(a.njobs + nb) * sizeof(int32_t));
      for (int j = 0; j < a.njobs; j++) CHECK(a.index[j] == D[j].uend);
      for (int64_t b = 0; b < nb; b++) {
        const int64_t f = std::min<int64_t>(b << a.bshift, a.total - 1);
        const int j = a.index[a.njobs + b];
        CHECK(j >= 0 && j < a.njobs && D[j].ubeg <= f && f < D[j].uend);
      }
    }
    stream_schedule_check(a, D);
  } else {
    CHECK(D[a.njobs - 1].grp_end == a.total);
    CHECK(a.table == nullptr || a.index == nullptr);
  }
}

}  // namespace

// --------------------------------------------------------------------------
// kernel launchers
// --------------------------------------------------------------------------
namespace qg {

hipError_t launch_pack(const float* W, int64_t ldw, int N, int K, int bits, void* packed, unsigned* flag,
                       hipStream_t stream) {
  const size_t pb = qgemm_packed_bytes(bits, N, K);
  CHECK(pb > 0 && ldw >= K);
  run_or_record(stream, [=] {
    span_r(W, (size_t)((int64_t)(N - 1) * ldw + K) * 4);
    std::memset(packed, 0, pb);  // every byte, padding included
    span_w(flag, sizeof(unsigned));
  });
  return hipSuccess;
}

// The allocation-free sweep's scratch: host memory that starts out non-zero
// (the library may assume nothing about it before its first call), and far
// smaller than the device's, so that the fuzz driver's job sets fill it and
// a sweep's slots often reach bytes an earlier sweep's job tables wrote.
hipError_t scratch_base(uint8_t** base, size_t* bytes) {
  static uint8_t* buf = [] {
    uint8_t* b = (uint8_t*)std::aligned_alloc(256, g_scratch_bytes);
    std::memset(b, 0xA5, g_scratch_bytes);
    return b;
  }();
  *base = buf;
  *bytes = g_scratch_bytes;
  return hipSuccess;
}

hipError_t launch_fill_zero(void* p, int64_t words, hipStream_t stream) {
  CHECK(words >= 0);
  run_or_record(stream, [=] {
    if (words > 0) std::memset(p, 0, (size_t)words * 4);
  });
  return hipSuccess;
}

hipError_t launch_sweep(int kind, int cls, int fs, int rows, const SweepArgs& args, int grid,
                        hipStream_t stream) {
  CHECK(kind >= 0 && kind <= 2 && fs >= 1 && fs <= 15);
  const SweepArgs a = args;  // by value, as a kernel argument
  if (rows == 8) g_big_launches++;
  run_or_record(stream, [=] { sweep_footprint(kind, cls, fs, rows, a, grid); });
  return hipSuccess;
}

hipError_t launch_accept(const AcceptArgs& args, unsigned long long* keys, const int32_t* drafts, int32_t* argmax,
                         float* maxval, int32_t* accepted, hipStream_t stream) {
  const AcceptArgs a = args;
  CHECK(a.M >= 1 && a.M <= kKeyRows && a.nslots >= 1 && a.nslots <= kMaxSlots);
  run_or_record(stream, [=] {
    span_w(keys, (size_t)kKeyCopies * kKeyRows * 8);
    span_w(argmax, (size_t)a.M * 4);
    if (maxval) span_w(maxval, (size_t)a.M * 4);
    span_w(accepted, (size_t)a.nslots * 4);
    for (int t = 0; t < a.nslots; t++) {
      CHECK(a.row0[t] >= 0 && a.ndraft[t] >= 0 && a.row0[t] + a.ndraft[t] < a.M);
      if (a.ndraft[t] > 0) span_r(drafts + a.row0[t], (size_t)a.ndraft[t] * 4);
    }
  });
  return hipSuccess;
}

int sweep_blocks_per_cu(int kind, int cls, int fs, int rows) { return (void)kind, (void)cls, (void)fs, (void)rows, 2; }

}  // namespace qg

namespace qa {

hipError_t launch_attn(const AttnArgs& args, bool fp8, int max_chunks, hipStream_t stream) {
  const AttnArgs a = args;
  CHECK(a.nslots >= 1 && a.nslots <= kMaxSlots && a.chunk >= kBlk && a.chunk % kBlk == 0);
  run_or_record(stream, [=] {
    const size_t esz = fp8 ? 1 : 2;
    int32_t parts = 0;
    for (int i = 0; i < a.nslots; i++) {
      const AttnSlot& s = a.s[i];
      CHECK(s.W >= 1 && s.W <= kMaxW && s.L >= s.W);
      CHECK(s.nchunks >= 1 && s.nchunks <= max_chunks);
      CHECK((int64_t)s.nchunks * a.chunk >= s.L && (int64_t)(s.nchunks - 1) * a.chunk < s.L);
      CHECK(s.part0 == parts);
      parts += s.nchunks * kHkv;
      span_r(s.Q, (size_t)s.W * kHq * kD * 2);
      span_r(s.K, (size_t)s.L * kHkv * kD * esz);
      span_r(s.V, (size_t)s.L * kHkv * kD * esz);
      span_w(s.O, (size_t)s.W * kHq * kD * 4);
    }
    span_w(a.part_o, (size_t)parts * kMaxRows * kD * 4);
    span_w(a.part_ml, (size_t)parts * kMaxRows * 2 * 4);
  });
  g_launches++;  // the merge kernel
  return hipSuccess;
}

}  // namespace qa

// --------------------------------------------------------------------------
// HIP runtime
// --------------------------------------------------------------------------
hipError_t hipMalloc(void** p, size_t n) {
  if (posix_memalign(p, 256, n ? n : 1) != 0) return hipErrorOutOfMemory;
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t s) {
  CHECK(!g_capturing || s != g_capturing);
  std::memset(p, v, n);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind kind, hipStream_t s) {
  (void)kind;
  CHECK(!g_capturing || s != g_capturing);
  if (n) std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t s) {
  CHECK(!g_capturing || s != g_capturing);
  return hipSuccess;
}
hipError_t hipDeviceSynchronize() {
  CHECK(!g_capturing);
  return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipGetDeviceProperties(hipDeviceProp_t* p, int d) {
  (void)d;
  std::memset((void*)p, 0, sizeof(*p));
  p->multiProcessorCount = 256;
  return hipSuccess;
}
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int flags) {
  (void)flags;
  *s = (hipStream_t) new char;
  return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
  CHECK(s != g_capturing);
  delete (char*)s;
  return hipSuccess;
}
hipError_t hipStreamBeginCapture(hipStream_t s, hipStreamCaptureMode mode) {
  (void)mode;
  CHECK(g_capturing == nullptr && s != nullptr);
  g_capturing = s;
  g_graph = new Graph();
  return hipSuccess;
}
hipError_t hipStreamEndCapture(hipStream_t s, hipGraph_t* g) {
  CHECK(g_capturing == s);
  *g = (hipGraph_t)g_graph;
  g_capturing = nullptr;
  g_graph = nullptr;
  return hipSuccess;
}
hipError_t hipGraphInstantiate(hipGraphExec_t* e, hipGraph_t g, hipGraphNode_t* node, char* log, size_t n) {
  (void)node, (void)log, (void)n;
  *e = (hipGraphExec_t) new Graph(*(Graph*)g);
  return hipSuccess;
}
hipError_t hipGraphLaunch(hipGraphExec_t e, hipStream_t s) {
  CHECK(!g_capturing || s != g_capturing);
  for (auto& f : ((Graph*)e)->nodes) f();
  return hipSuccess;
}
hipError_t hipGraphExecDestroy(hipGraphExec_t e) {
  delete (Graph*)e;
  return hipSuccess;
}
hipError_t hipGraphDestroy(hipGraph_t g) {
  delete (Graph*)g;
  return hipSuccess;
}
