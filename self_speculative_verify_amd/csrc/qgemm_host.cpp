// Host side of the quantized weight sweep: argument validation, path choice,
// work planning, workspace layout and kernel launch.  Validation is pure host
// code and runs before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <list>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "qgemm.h"
#include "qgemm_internal.h"

namespace qg {
hipError_t launch_pack(const float* W, int64_t ldw, int N, int K, int bits, void* packed,
                       unsigned* flag, hipStream_t stream);
hipError_t launch_fill_zero(void* p, int64_t words, hipStream_t stream);
hipError_t scratch_base(uint8_t** base, size_t* bytes);
int sweep_blocks_per_cu(int kind, int cls, int fs, int rows);
hipError_t launch_sweep(int kind, int cls, int fs, int rows, const SweepArgs& args, int grid, hipStream_t stream);
hipError_t launch_accept(const AcceptArgs& a, unsigned long long* keys, const int32_t* drafts, int32_t* argmax,
                         float* maxval, int32_t* accepted, hipStream_t stream);
}  // namespace qg

#ifdef QG_TIMELINE
// Timeline build only: the stamp buffer every stream launch writes (null: none).
static unsigned long long* g_trace = nullptr;
extern "C" void qgemm_timeline_set(void* trace) { g_trace = (unsigned long long*)trace; }
#endif

namespace {

using qg::JobDesc;

constexpr int64_t kMaxN = (int64_t)1 << 30;    // keeps row-block math in 32 bits
constexpr int64_t kMaxK = (int64_t)1 << 24;    // keeps row-group and X byte offsets in 32 bits

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t nkt_of(int64_t K) { return (K + qg::kTileK - 1) / qg::kTileK; }
int64_t nrb_of(int64_t N) { return (N + qg::kTileRows - 1) / qg::kTileRows; }

// bits: a format code (4, 5 or the QGEMM_FMT_* variants)
bool valid_shape(int bits, int64_t N, int64_t K) {
  return qg::valid_fmt(bits) && N >= 1 && N <= kMaxN && K >= qg::fmt_group(bits) && K <= kMaxK &&
         K % qg::fmt_group(bits) == 0;
}

int path_of(int path, int M) {
  // AUTO: MFMA at every M (measured no slower than GEMV at M = 1, faster
  // above; one bitwise class with the verify panels up to 16 rows)
  if (path == QGEMM_PATH_AUTO) return (void)M, QGEMM_PATH_MFMA;
  return path;
}

// A byte range [a, b) a call reads or writes.
struct Span {
  uintptr_t a, b;
  bool write;
};
Span written(const void* p, size_t bytes) { return {(uintptr_t)p, (uintptr_t)p + bytes, true}; }

// No buffer a call writes (each job's Y, and the `extra` spans: workspace,
// verify outputs) overlaps any other buffer it reads or writes (reads may
// share memory).  Intervals sorted by start; an interval overlaps an earlier
// one iff that one ends after it starts, so it suffices to track the largest
// end so far over all intervals and over the written ones.
bool overlap_free(const qgemm_job* jobs, int njobs, const std::vector<Span>& extra) {
  std::vector<Span> v(extra);
  v.reserve(extra.size() + (size_t)njobs * 3);
  for (int i = 0; i < njobs; i++) {
    const qgemm_job& j = jobs[i];
    const uintptr_t x0 = (uintptr_t)j.X, p0 = (uintptr_t)j.packed;
    v.push_back({x0, x0 + (uintptr_t)(((j.M - 1) * j.ldx + j.K) * sizeof(uint16_t)), false});
    v.push_back({p0, p0 + (uintptr_t)(nrb_of(j.N) * nkt_of(j.K) * qg::tile_bytes(j.bits)), false});
    if (j.Y) {
      const uintptr_t y0 = (uintptr_t)j.Y;
      v.push_back({y0, y0 + (uintptr_t)(((j.M - 1) * j.ldy + j.N) * sizeof(float)), true});
    }
  }
  std::sort(v.begin(), v.end(), [](const Span& p, const Span& q) { return p.a < q.a; });
  uintptr_t end_any = 0, end_write = 0;
  for (const Span& s : v) {
    if ((s.write ? end_any : end_write) > s.a) return false;
    end_any = std::max(end_any, s.b);
    if (s.write) end_write = std::max(end_write, s.b);
  }
  return true;
}

// y_optional: the verify head, whose Y may be null (no outputs written);
// extra: further buffers the call writes
qgemm_status validate(const qgemm_job* jobs, int njobs, int path, bool y_optional = false,
                      const std::vector<Span>& extra = {}) {
  if (njobs < 1 || jobs == nullptr) return QGEMM_ERR_INVALID_ARG;
  if (path != QGEMM_PATH_AUTO && path != QGEMM_PATH_GEMV && path != QGEMM_PATH_MFMA)
    return QGEMM_ERR_INVALID_ARG;
  for (int i = 0; i < njobs; i++) {
    const qgemm_job& j = jobs[i];
    if (!valid_shape(j.bits, j.N, j.K)) return QGEMM_ERR_INVALID_ARG;
    if (j.M < 1 || j.M > QGEMM_MAX_M) return QGEMM_ERR_INVALID_ARG;
    if (!j.packed || !j.X) return QGEMM_ERR_INVALID_ARG;
    if (!aligned(j.packed, 256) || !aligned(j.X, 16)) return QGEMM_ERR_INVALID_ARG;
    if (j.ldx < j.K || j.ldx % 8 != 0 || j.ldx > kMaxK) return QGEMM_ERR_INVALID_ARG;
    if (path == QGEMM_PATH_GEMV && j.M > QGEMM_GEMV_MAX_M) return QGEMM_ERR_INVALID_ARG;
    if (!j.Y) {
      if (y_optional) continue;
      return QGEMM_ERR_INVALID_ARG;
    }
    if (!aligned(j.Y, 16)) return QGEMM_ERR_INVALID_ARG;
    if (j.ldy < j.N || j.ldy % 4 != 0) return QGEMM_ERR_INVALID_ARG;
  }
  return overlap_free(jobs, njobs, extra) ? QGEMM_OK : QGEMM_ERR_INVALID_ARG;
}

// ---------------------------------------------------------------------------
// planning: jobs are grouped by kernel (kind, class); the workspace holds the
// job tables of launches with many jobs and the stream kernels' partial-sum
// slots (each region 256-byte aligned)
// ---------------------------------------------------------------------------
enum Kind { kStreamGemv = 0, kStreamMfma = 1, kGroupMfma = 2 };

struct Launch {
  int kind;
  int cls;
  int fs = 0;                 // formats of its jobs (bit 0: 4-bit, 1: 5-bit, 2: group-64, 3: zero-point)
  bool big = false;           // stream: at least kStreamBigBytes of weights
  int rows = 4;               // stream: row blocks per step
  int64_t bytes = 0;          // weight bytes of its jobs
  std::vector<JobDesc> descs;
  int64_t total = 0;          // stream: flat units; group: row-block groups
  size_t table_off = 0, slots_off = 0;
  int nwaves = 0;
  int bshift = 0;             // stream with a table: log2 of the units per bucket
  std::vector<int32_t> index; // stream with a table: uend per job, first job per bucket
};

int fmt_bit(int f) { return f == qg::kFmtQ4 ? 1 : f == qg::kFmtQ5 ? 2 : f == qg::kFmtG64 ? 4 : 8; }

// Flat units and row-block groups are 32-bit in the kernels.
constexpr int64_t kMaxSteps = ((int64_t)1 << 31) - 1;

// Workspace of a plan: the job tables of its launches, then the stream
// kernels' partial-sum slots (two regions, each a 256-byte multiple).  Every
// completed sweep leaves its slots at zero, so sweeps that run one after
// another may share one slot region whatever their jobs.
struct Plan {
  std::vector<Launch> launches;
  size_t table_bytes = 0;
  size_t slot_bytes = 0;
  size_t total = 0;           // both regions, at least 256
  bool ok = true;             // false: a launch exceeds the 32-bit unit range
};

int kind_of(int path, int M) {
  const int p = path_of(path, M);
  if (p == QGEMM_PATH_GEMV) return kStreamGemv;
  return M <= 16 ? kStreamMfma : kGroupMfma;
}

int class_of(int kind, int M) {
  if (kind == kStreamGemv) return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  if (kind == kStreamMfma) return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
  return (M + 15) / 16 * 16;
}

int cu_count();

// Waves of a stream launch: kStreamWaves (kStreamWavesBig for a big launch),
// but a launch too small to give every wave kMinSteps steps takes fewer
// waves -- down to kFloorWaves, below which every wave holds at least one
// step, as many as that allows.  Fewer waves split a row group over fewer
// contributors: a 5120 x 5120 matrix at M = 6 has 3200 steps, 1.6 per wave
// of 2048 and a row group of 40 k tiles split over up to 26 of them
// (measured: a round of 256 one-matrix sweeps 5.27 -> 4.82 ms; a 1024 x 1024
// matrix keeps its 104 waves, which its latency needs).  Depends on the
// shapes only, never on M.
constexpr int64_t kMinSteps = 4, kFloorWaves = 512;
int64_t stream_waves(int64_t T, bool big) {
  const int64_t cap = big ? qg::kStreamWavesBig : qg::kStreamWaves;
  const int64_t one = T / qg::kMaxUnitWeight;  // waves that hold at least one step each
  const int64_t w = std::max(T / (kMinSteps * qg::kMaxUnitWeight), std::min(one, kFloorWaves));
  return std::max<int64_t>(1, std::min(cap, w));
}

Plan make_plan(const qgemm_job* jobs, int njobs, int path, unsigned long long* keys = nullptr) {
  Plan P;
  // Jobs of the group kernel go longest K first (their units are whole-K,
  // so the long ones are dealt out before the short ones fill the gaps);
  // stream jobs keep the caller's order.
  std::vector<int> order(njobs);
  for (int i = 0; i < njobs; i++) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    const bool ga = kind_of(path, jobs[a].M) == kGroupMfma, gb = kind_of(path, jobs[b].M) == kGroupMfma;
    if (ga != gb) return gb;  // stream jobs first, in order
    return ga && jobs[a].K > jobs[b].K;
  });
  // each job's launch (kind, class), and every launch's weight bytes, which
  // decide its step shape before any job is laid out
  std::vector<int> dst_of(njobs);
  for (int i : order) {
    const qgemm_job& j = jobs[i];
    const int kind = kind_of(path, j.M);
    const int cls = class_of(kind, j.M);
    int li = -1;
    for (size_t k = 0; k < P.launches.size(); k++)
      if (P.launches[k].kind == kind && P.launches[k].cls == cls) li = (int)k;
    if (li < 0) {
      P.launches.push_back(Launch{});
      li = (int)P.launches.size() - 1;
      P.launches[li].kind = kind;
      P.launches[li].cls = cls;
    }
    dst_of[i] = li;
    P.launches[li].bytes += nrb_of(j.N) * nkt_of(j.K) * qg::tile_bytes(j.bits);
  }
  // the MFMA stream kernel has the eight-block step shape for big launches
  for (auto& l : P.launches) {
    l.big = l.bytes >= qg::kStreamBigBytes;
    l.rows = qg::stream_rows(l.big && l.kind == kStreamMfma);
  }
  for (int i : order) {
    const qgemm_job& j = jobs[i];
    Launch* dst = &P.launches[dst_of[i]];
    const int kind = dst->kind, cls = dst->cls;
    dst->fs |= fmt_bit(j.bits);
    JobDesc d;
    std::memset(&d, 0, sizeof(d));
    d.packed = (const uint8_t*)j.packed;
    d.X = j.X;
    d.Y = j.Y;
    d.keys = keys;
    d.ldx = j.ldx;
    d.ldy = j.ldy;
    d.N = (int32_t)j.N;
    d.K = (int32_t)j.K;
    d.M = j.M;
    d.fmt = j.bits;
    d.nkt = (int32_t)nkt_of(j.K);
    qg::div_magic((uint32_t)d.nkt, d.nkt_m, d.nkt_sh);
    d.ngroups = (int32_t)(j.K / qg::kGroup);
    d.nrb = (int32_t)nrb_of(j.N);
    if (kind == kGroupMfma) {
      const int64_t per = (int64_t)qg::group_waves(cls) * qg::kGroupRows;
      const int64_t groups = (d.nrb + per - 1) / per;
      d.grp_begin = (int32_t)dst->total;
      dst->total += groups;
      d.grp_end = (int32_t)std::min(dst->total, kMaxSteps);
    } else {
      const int R = dst->rows;
      d.nrg = (d.nrb + R - 1) / R;
      d.ubeg = (int32_t)std::min(dst->total, kMaxSteps);
      dst->total += (int64_t)d.nrg * d.nkt * qg::unit_weight(d.fmt);
      d.uend = (int32_t)std::min(dst->total, kMaxSteps);
    }
    dst->descs.push_back(d);
  }
  size_t off = 0, soff = 0;
  for (auto& l : P.launches) {
    if (l.total > kMaxSteps) {
      P.ok = false;
      return P;
    }
    if ((int)l.descs.size() > qg::kMaxInline) {
      if (l.kind != kGroupMfma) {
        // uend of every job, then for bucket b (units [b << bshift, ...))
        // the job holding its first unit
        while ((l.total >> l.bshift) > 1024) l.bshift++;
        const int64_t nb = (l.total >> l.bshift) + 1;
        l.index.reserve(l.descs.size() + nb);
        for (const auto& d : l.descs) l.index.push_back(d.uend);
        size_t j = 0;
        for (int64_t b = 0; b < nb; b++) {
          const int64_t f = std::min(b << l.bshift, l.total - 1);
          while (f >= l.descs[j].uend) j++;
          l.index.push_back((int32_t)j);
        }
      }
      l.table_off = off;
      off = round_up(off + l.descs.size() * sizeof(JobDesc) + l.index.size() * sizeof(int32_t), 256);
    }
    if (l.kind != kGroupMfma) {
      l.nwaves = (int)stream_waves(l.total, l.big);
      l.slots_off = soff;
      soff = round_up(soff + (size_t)qg::stream_slot_bytes(l.nwaves, l.rows, l.kind == kStreamMfma, l.cls), 256);
    }
  }
  P.table_bytes = off;
  P.slot_bytes = soff;
  P.total = std::max<size_t>(off + soff, 256);
  return P;
}

int blocks_per_cu(int kind, int cls, int fs, int rows) {
  static std::mutex mu;
  static int cache[16][2][3][65] = {};
  std::lock_guard<std::mutex> g(mu);
  int& c = cache[fs & 15][rows == 8 ? 1 : 0][kind][cls];
  if (c == 0) {
    c = qg::sweep_blocks_per_cu(kind, cls, fs, rows);
    if (c <= 0) c = 1;
  }
  return c;
}

int cu_count() {
  static std::once_flag once;
  static int cus = 256;
  std::call_once(once, [] {
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess)
      cus = prop.multiProcessorCount;
  });
  return cus;
}

qgemm_status run_plan(Plan& P, void* workspace, void* stream);
qgemm_status upload_tables(const Plan& P, uint8_t* tables, hipStream_t s);
qgemm_status launch_plan(const Plan& P, uint8_t* tables, uint8_t* slots, hipStream_t s);
int grid_of(const Launch& l);

}  // namespace

extern "C" {

size_t qgemm_packed_bytes(int bits, int64_t N, int64_t K) {
  if (!valid_shape(bits, N, K)) return 0;
  return (size_t)(nrb_of(N) * nkt_of(K) * qg::tile_bytes(bits));
}

qgemm_status qgemm_pack(const float* W, int64_t ldw, int64_t N, int64_t K, int bits, void* packed,
                        void* stream) {
  if (!valid_shape(bits, N, K) || !W || !packed || ldw < K || !aligned(packed, 256) || !aligned(W, 4))
    return QGEMM_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  unsigned* flag = nullptr;
  if (hipMalloc(&flag, sizeof(unsigned)) != hipSuccess) return QGEMM_ERR_HIP;
  unsigned host_flag = 0;
  qgemm_status st = QGEMM_OK;
  if (hipMemsetAsync(flag, 0, sizeof(unsigned), s) != hipSuccess ||
      qg::launch_pack(W, ldw, (int)N, (int)K, bits, packed, flag, s) != hipSuccess ||
      hipMemcpyAsync(&host_flag, flag, sizeof(unsigned), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess) {
    st = QGEMM_ERR_HIP;
  } else if (host_flag) {
    st = QGEMM_ERR_NONFINITE;
  }
  if (hipFree(flag) != hipSuccess && st == QGEMM_OK) st = QGEMM_ERR_HIP;
  return st;
}

size_t qgemm_workspace_bytes(const qgemm_job* jobs, int njobs, int path) {
  if (validate(jobs, njobs, path) != QGEMM_OK) return 0;
  const Plan P = make_plan(jobs, njobs, path);
  return P.ok ? P.total : 0;
}

qgemm_status qgemm_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256) || ws_bytes % 4 != 0) return QGEMM_ERR_INVALID_ARG;
  return qg::launch_fill_zero(workspace, (int64_t)(ws_bytes / 4), (hipStream_t)stream) == hipSuccess
             ? QGEMM_OK
             : QGEMM_ERR_HIP;
}

qgemm_status qgemm_validate(const qgemm_job* jobs, int njobs, int path, void* workspace,
                            size_t ws_bytes) {
  qgemm_status st = validate(jobs, njobs, path, false, {written(workspace, ws_bytes)});
  if (st != QGEMM_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  const Plan P = make_plan(jobs, njobs, path);
  if (!P.ok) return QGEMM_ERR_UNSUPPORTED;
  if (ws_bytes < P.total) return QGEMM_ERR_INVALID_ARG;
  return QGEMM_OK;
}

qgemm_status qgemm_sweep_path(const qgemm_job* jobs, int njobs, int path, void* workspace,
                              size_t ws_bytes, void* stream) {
  qgemm_status st = qgemm_validate(jobs, njobs, path, workspace, ws_bytes);
  if (st != QGEMM_OK) return st;
  Plan P = make_plan(jobs, njobs, path);
  return run_plan(P, workspace, stream);
}

// Allocation-free sweep: the current device's static scratch in place of a
// workspace, split-K slots at its bottom and job tables at its top.  Per
// device, [0, clean) is known to be zero: every completed sweep leaves its
// slots zero, and only table copies (or the unknown contents before the
// first call) can leave a byte non-zero.  A call whose slots reach past
// `clean` clears [clean, slot end) first with the fill kernel.
qgemm_status qgemm_sweep_noalloc(const qgemm_job* jobs, int njobs, int path, void* stream) {
  qgemm_status st = validate(jobs, njobs, path, false, {});
  if (st != QGEMM_OK) return st;
  Plan P = make_plan(jobs, njobs, path);
  if (!P.ok) return QGEMM_ERR_UNSUPPORTED;
  if (P.total > QGEMM_NOALLOC_SCRATCH_BYTES) return QGEMM_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= qg::kMaxDevices) return QGEMM_ERR_HIP;
  uint8_t* base = nullptr;
  size_t kScratch = 0;  // QGEMM_NOALLOC_SCRATCH_BYTES (less in host-only test builds)
  if (qg::scratch_base(&base, &kScratch) != hipSuccess) return QGEMM_ERR_HIP;
  if (P.total > kScratch) return QGEMM_ERR_INVALID_ARG;
  static std::mutex mu;
  static size_t clean[qg::kMaxDevices] = {};
  std::lock_guard<std::mutex> g(mu);
  hipStream_t s = (hipStream_t)stream;
  size_t& c = clean[dev];
  if (P.slot_bytes > c) {
    if (qg::launch_fill_zero(base + c, (int64_t)((P.slot_bytes - c) / 4), s) != hipSuccess) return QGEMM_ERR_HIP;
    c = P.slot_bytes;
  }
  uint8_t* tables = base + (kScratch - P.table_bytes);
  c = std::min(c, kScratch - P.table_bytes);
  if ((st = upload_tables(P, tables, s)) != QGEMM_OK) return st;
  return launch_plan(P, tables, base, s);
}

// verify head workspace: the sweep's, then one argmax key per row
static size_t verify_keys_off(const Plan& P) { return round_up(P.total, 256); }
static size_t verify_total(const Plan& P) {
  return verify_keys_off(P) + (size_t)qg::kKeyCopies * qg::kKeyRows * sizeof(unsigned long long);
}

size_t qgemm_verify_workspace_bytes(const qgemm_job* head) {
  if (validate(head, 1, QGEMM_PATH_AUTO, true) != QGEMM_OK) return 0;
  const Plan P = make_plan(head, 1, QGEMM_PATH_AUTO);
  return P.ok ? verify_total(P) : 0;
}

}  // extern "C"

namespace {

// Checks of a verify head call (host only) and the acceptance kernel's
// arguments.
// The outputs argmax [M], maxlogit [M] (optional) and accepted [nslots] and
// the workspace are written spans: none may overlap another or the job's
// buffers.
qgemm_status head_args(const qgemm_job* head, const int32_t* drafts, const qgemm_slot* slots, int nslots,
                       const int32_t* argmax, const float* maxlogit, const int32_t* accepted,
                       const void* workspace, size_t ws_bytes, qg::AcceptArgs& a) {
  if (!head || !argmax || !accepted) return QGEMM_ERR_INVALID_ARG;
  if (!slots || nslots < 1 || nslots > qg::kMaxSlots) return QGEMM_ERR_INVALID_ARG;
  if (head->M < 1 || head->M > QGEMM_MAX_M) return QGEMM_ERR_INVALID_ARG;
  std::vector<Span> outs = {written(argmax, (size_t)head->M * 4), written(accepted, (size_t)nslots * 4),
                            written(workspace, ws_bytes)};
  if (maxlogit) outs.push_back(written(maxlogit, (size_t)head->M * 4));
  qgemm_status st = validate(head, 1, QGEMM_PATH_AUTO, true, outs);
  if (st != QGEMM_OK) return st;
  std::memset(&a, 0, sizeof(a));
  a.nslots = nslots;
  a.M = head->M;
  bool any_draft = false;
  for (int i = 0; i < nslots; i++) {
    const qgemm_slot& sl = slots[i];
    if (sl.row0 < 0 || sl.ndraft < 0 || (int64_t)sl.row0 + sl.ndraft >= head->M) return QGEMM_ERR_INVALID_ARG;
    any_draft = any_draft || sl.ndraft > 0;
    a.row0[i] = sl.row0;
    a.ndraft[i] = sl.ndraft;
  }
  if (any_draft && !drafts) return QGEMM_ERR_INVALID_ARG;
  return QGEMM_OK;
}

constexpr size_t kKeyBytes = (size_t)qg::kKeyCopies * qg::kKeyRows * sizeof(unsigned long long);

}  // namespace

extern "C" {

qgemm_status qgemm_verify_head(const qgemm_job* head, const int32_t* drafts, const qgemm_slot* slots, int nslots,
                               int32_t* argmax, float* maxlogit, int32_t* accepted, void* workspace,
                               size_t ws_bytes, void* stream) {
  qg::AcceptArgs a;
  qgemm_status st = head_args(head, drafts, slots, nslots, argmax, maxlogit, accepted, workspace, ws_bytes, a);
  if (st != QGEMM_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  const Plan P0 = make_plan(head, 1, QGEMM_PATH_AUTO);
  if (!P0.ok) return QGEMM_ERR_UNSUPPORTED;
  if (ws_bytes < verify_total(P0)) return QGEMM_ERR_INVALID_ARG;
  unsigned long long* keys = (unsigned long long*)((uint8_t*)workspace + verify_keys_off(P0));
  Plan P = make_plan(head, 1, QGEMM_PATH_AUTO, keys);
  st = run_plan(P, workspace, stream);
  if (st != QGEMM_OK) return st;
  return qg::launch_accept(a, keys, drafts, argmax, maxlogit, accepted, (hipStream_t)stream) == hipSuccess
             ? QGEMM_OK
             : QGEMM_ERR_HIP;
}

// ---------------------------------------------------------------------------
// round replay: the sweeps of a round and its verify head as one HIP graph
// ---------------------------------------------------------------------------
}  // extern "C"

struct qgemm_round_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int kernels = 0;
};

namespace {

// Plans of a round and its workspace layout: every sweep's tables one after
// another, then one slot region that all sweeps share (they run in order and
// each leaves it at zero; as large as the largest sweep's), then the head's
// argmax keys.
struct RoundPlan {
  std::vector<Plan> sweeps;
  Plan head;
  bool has_head = false;
  std::vector<size_t> table_off;
  size_t head_table_off = 0, slots_off = 0, keys_off = 0, total = 0;
};

// keys_base: the workspace (null when only sizing), ws_bytes its size; the
// workspace may overlap no sweep's buffers
qgemm_status round_plan(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head, RoundPlan& R,
                        unsigned long long* keys_base, size_t ws_bytes = 0) {
  const std::vector<Span> ws_span = keys_base ? std::vector<Span>{written(keys_base, ws_bytes)} : std::vector<Span>{};
  if (nsweeps < 0 || (nsweeps > 0 && !sweeps) || (nsweeps == 0 && !head)) return QGEMM_ERR_INVALID_ARG;
  size_t tables = 0, slots = 0;
  for (int i = 0; i < nsweeps; i++) {
    const qgemm_status st = validate(sweeps[i].jobs, sweeps[i].njobs, sweeps[i].path, false, ws_span);
    if (st != QGEMM_OK) return st;
    R.sweeps.push_back(make_plan(sweeps[i].jobs, sweeps[i].njobs, sweeps[i].path));
    if (!R.sweeps.back().ok) return QGEMM_ERR_UNSUPPORTED;
    R.table_off.push_back(tables);
    tables += R.sweeps.back().table_bytes;
    slots = std::max(slots, R.sweeps.back().slot_bytes);
  }
  if (head) {
    const qgemm_status st = validate(head, 1, QGEMM_PATH_AUTO, true);
    if (st != QGEMM_OK) return st;
    R.has_head = true;
    R.head_table_off = tables;
    R.head = make_plan(head, 1, QGEMM_PATH_AUTO);
    if (!R.head.ok) return QGEMM_ERR_UNSUPPORTED;
    tables += R.head.table_bytes;
    slots = std::max(slots, R.head.slot_bytes);
  }
  R.slots_off = tables;
  R.keys_off = round_up(tables + slots, 256);
  R.total = std::max<size_t>(R.keys_off + (head ? kKeyBytes : 0), 256);
  if (head && keys_base) {
    // the head's jobs carry the key pointer
    R.head = make_plan(head, 1, QGEMM_PATH_AUTO, (unsigned long long*)((uint8_t*)keys_base + R.keys_off));
  }
  return QGEMM_OK;
}

}  // namespace

extern "C" {

size_t qgemm_round_workspace_bytes(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head) {
  RoundPlan R;
  return round_plan(sweeps, nsweeps, head, R, nullptr) == QGEMM_OK ? R.total : 0;
}

qgemm_status qgemm_round_create(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head,
                                const int32_t* drafts, const qgemm_slot* slots, int nslots, int32_t* argmax,
                                float* maxlogit, int32_t* accepted, void* workspace, size_t ws_bytes,
                                void* stream, qgemm_round** out) {
  if (!out) return QGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  if (!workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  qg::AcceptArgs a;
  if (head) {
    const qgemm_status st = head_args(head, drafts, slots, nslots, argmax, maxlogit, accepted, workspace,
                                      ws_bytes, a);
    if (st != QGEMM_OK) return st;
  }
  RoundPlan R;
  qgemm_status st = round_plan(sweeps, nsweeps, head, R, (unsigned long long*)workspace, ws_bytes);
  if (st != QGEMM_OK) return st;
  if (ws_bytes < R.total) return QGEMM_ERR_INVALID_ARG;
  uint8_t* ws = (uint8_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  // tables in place (and every kernel's grid known) before recording starts
  for (size_t i = 0; i < R.sweeps.size(); i++) {
    if ((st = upload_tables(R.sweeps[i], ws + R.table_off[i], s)) != QGEMM_OK) return st;
    for (const auto& l : R.sweeps[i].launches) (void)grid_of(l);
  }
  if (R.has_head) {
    if ((st = upload_tables(R.head, ws + R.head_table_off, s)) != QGEMM_OK) return st;
    for (const auto& l : R.head.launches) (void)grid_of(l);
  }
  if (hipStreamSynchronize(s) != hipSuccess) return QGEMM_ERR_HIP;
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return QGEMM_ERR_HIP;
  qgemm_round* r = new qgemm_round();
  bool ok = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) == hipSuccess;
  bool capturing = ok;
  for (size_t i = 0; ok && i < R.sweeps.size(); i++) {
    ok = launch_plan(R.sweeps[i], ws + R.table_off[i], ws + R.slots_off, cs) == QGEMM_OK;
    r->kernels += (int)R.sweeps[i].launches.size();
  }
  if (ok && R.has_head) {
    ok = launch_plan(R.head, ws + R.head_table_off, ws + R.slots_off, cs) == QGEMM_OK &&
         qg::launch_accept(a, (unsigned long long*)(ws + R.keys_off), drafts, argmax, maxlogit, accepted, cs) ==
             hipSuccess;
    r->kernels += (int)R.head.launches.size() + 1;
  }
  if (capturing) ok = hipStreamEndCapture(cs, &r->graph) == hipSuccess && ok;
  ok = ok && hipGraphInstantiate(&r->exec, r->graph, nullptr, nullptr, 0) == hipSuccess;
  if (hipStreamDestroy(cs) != hipSuccess) ok = false;
  if (!ok) {
    qgemm_round_destroy(r);
    return QGEMM_ERR_HIP;
  }
  *out = r;
  return QGEMM_OK;
}

qgemm_status qgemm_round_launch(const qgemm_round* r, void* stream) {
  if (!r || !r->exec) return QGEMM_ERR_INVALID_ARG;
  return hipGraphLaunch(r->exec, (hipStream_t)stream) == hipSuccess ? QGEMM_OK : QGEMM_ERR_HIP;
}

int qgemm_round_kernels(const qgemm_round* r) { return r ? r->kernels : 0; }

void qgemm_round_destroy(qgemm_round* r) {
  if (!r) return;
  if (r->exec) (void)hipGraphExecDestroy(r->exec);
  if (r->graph) (void)hipGraphDestroy(r->graph);
  delete r;
}

}  // extern "C"

// The round cache: an LRU list of (key, round, its workspace) and a map from
// key to list position; calls are serialized by the cache's mutex.
struct qgemm_round_cache_s {
  struct Entry {
    std::string key;
    qgemm_round* round;
    void* ws;
  };
  int cap = 0;
  std::list<Entry> lru;  // front: most recently used
  std::unordered_map<std::string, std::list<Entry>::iterator> index;
  std::mutex mu;
  uint64_t hits = 0, misses = 0, evictions = 0;
};

namespace {

template <typename T>
void key_put(std::string& k, T v) {
  k.append((const char*)&v, sizeof(v));
}
// field by field (never the raw structs, whose padding is not theirs to fix)
void key_job(std::string& k, const qgemm_job& j) {
  key_put(k, (uintptr_t)j.packed);
  key_put(k, (uintptr_t)j.X);
  key_put(k, (uintptr_t)j.Y);
  key_put(k, j.N);
  key_put(k, j.K);
  key_put(k, j.ldx);
  key_put(k, j.ldy);
  key_put(k, j.M);
  key_put(k, j.bits);
}
// the key of a round: everything qgemm_round_create fixes but the workspace
std::string round_key(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head, const int32_t* drafts,
                      const qgemm_slot* slots, int nslots, const int32_t* argmax, const float* maxlogit,
                      const int32_t* accepted) {
  std::string k;
  key_put(k, nsweeps);
  for (int i = 0; i < nsweeps; i++) {
    key_put(k, sweeps[i].path);
    key_put(k, sweeps[i].njobs);
    for (int j = 0; j < sweeps[i].njobs; j++) key_job(k, sweeps[i].jobs[j]);
  }
  key_put(k, head != nullptr);
  if (head) {
    key_job(k, *head);
    key_put(k, (uintptr_t)drafts);
    key_put(k, nslots);
    for (int i = 0; i < nslots; i++) {
      key_put(k, slots[i].row0);
      key_put(k, slots[i].ndraft);
    }
    key_put(k, (uintptr_t)argmax);
    key_put(k, (uintptr_t)maxlogit);
    key_put(k, (uintptr_t)accepted);
  }
  return k;
}

void drop_entry(qgemm_round_cache_s::Entry& e) {
  qgemm_round_destroy(e.round);
  if (e.ws) (void)hipFree(e.ws);
  e.round = nullptr;
  e.ws = nullptr;
}

}  // namespace

extern "C" {

qgemm_status qgemm_round_cache_create(int capacity, qgemm_round_cache** out) {
  if (!out) return QGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  if (capacity < 1 || capacity > QGEMM_ROUND_CACHE_MAX) return QGEMM_ERR_INVALID_ARG;
  qgemm_round_cache* c = new qgemm_round_cache();
  c->cap = capacity;
  *out = c;
  return QGEMM_OK;
}

qgemm_status qgemm_round_cache_run(qgemm_round_cache* c, const qgemm_round_sweep* sweeps, int nsweeps,
                                   const qgemm_job* head, const int32_t* drafts, const qgemm_slot* slots,
                                   int nslots, int32_t* argmax, float* maxlogit, int32_t* accepted,
                                   void* stream, int* hit) {
  if (hit) *hit = 0;
  if (!c || !hit) return QGEMM_ERR_INVALID_ARG;
  if (nsweeps < 0 || (nsweeps > 0 && !sweeps) || (nsweeps == 0 && !head)) return QGEMM_ERR_INVALID_ARG;
  for (int i = 0; i < nsweeps; i++)
    if (sweeps[i].njobs < 1 || !sweeps[i].jobs) return QGEMM_ERR_INVALID_ARG;
  if (head && (nslots < 0 || (nslots > 0 && !slots))) return QGEMM_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> g(c->mu);
  const std::string key = round_key(sweeps, nsweeps, head, drafts, slots, head ? nslots : 0, argmax, maxlogit,
                                    accepted);
  auto it = c->index.find(key);
  if (it != c->index.end()) {
    c->lru.splice(c->lru.begin(), c->lru, it->second);
    c->hits++;
    *hit = 1;
    return qgemm_round_launch(c->lru.front().round, stream);
  }
  // a miss: the round's plan first (every argument error before any HIP
  // call), then its recording, and only then an eviction, so that a call
  // that fails leaves the cache as it was
  RoundPlan R;
  qgemm_status st = round_plan(sweeps, nsweeps, head, R, nullptr);
  if (st != QGEMM_OK) return st;
  if (head) {
    qg::AcceptArgs a;  // (the recording builds its own)
    if ((st = head_args(head, drafts, slots, nslots, argmax, maxlogit, accepted, nullptr, 0, a)) != QGEMM_OK)
      return st;
  }
  void* ws = nullptr;
  if (hipMalloc(&ws, R.total) != hipSuccess) return QGEMM_ERR_HIP;
  qgemm_round* r = nullptr;
  if (hipMemsetAsync(ws, 0, R.total, (hipStream_t)stream) != hipSuccess) {
    (void)hipFree(ws);
    return QGEMM_ERR_HIP;
  }
  st = qgemm_round_create(sweeps, nsweeps, head, drafts, slots, nslots, argmax, maxlogit, accepted, ws, R.total,
                          stream, &r);
  if (st != QGEMM_OK) {
    (void)hipStreamSynchronize((hipStream_t)stream);
    (void)hipFree(ws);
    return st;
  }
  if ((int)c->lru.size() >= c->cap) {
    // a replay of the evicted round may still run: wait for the device
    if (hipDeviceSynchronize() != hipSuccess) {
      qgemm_round_destroy(r);
      (void)hipFree(ws);
      return QGEMM_ERR_HIP;
    }
    qgemm_round_cache_s::Entry& e = c->lru.back();
    c->index.erase(e.key);
    drop_entry(e);
    c->lru.pop_back();
    c->evictions++;
  }
  c->lru.push_front(qgemm_round_cache_s::Entry{key, r, ws});
  c->index[key] = c->lru.begin();
  c->misses++;
  return qgemm_round_launch(r, stream);
}

qgemm_status qgemm_round_cache_stats(const qgemm_round_cache* c, int* size, uint64_t* hits, uint64_t* misses,
                                     uint64_t* evictions) {
  if (!c) return QGEMM_ERR_INVALID_ARG;
  qgemm_round_cache* m = const_cast<qgemm_round_cache*>(c);
  std::lock_guard<std::mutex> g(m->mu);
  if (size) *size = (int)c->lru.size();
  if (hits) *hits = c->hits;
  if (misses) *misses = c->misses;
  if (evictions) *evictions = c->evictions;
  return QGEMM_OK;
}

void qgemm_round_cache_destroy(qgemm_round_cache* c) {
  if (!c) return;
  // replays of the held rounds may still run on the callers' streams
  if (!c->lru.empty()) (void)hipDeviceSynchronize();
  for (auto& e : c->lru) drop_entry(e);
  delete c;
}

}  // extern "C"

namespace {

qgemm_status run_plan(Plan& P, void* workspace, void* stream) {
  uint8_t* ws = (uint8_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const qgemm_status st = upload_tables(P, ws, s);
  if (st != QGEMM_OK) return st;
  return launch_plan(P, ws, ws + P.table_bytes, s);
}

// One copy per launch with more than kMaxInline jobs: its job table, then
// the stream kernel's job index, at its offset in the table region.
qgemm_status upload_tables(const Plan& P, uint8_t* tables, hipStream_t s) {
  for (const auto& l : P.launches) {
    if ((int)l.descs.size() <= qg::kMaxInline) continue;
    const size_t tb = l.descs.size() * sizeof(JobDesc);
    std::vector<uint8_t> host(tb + l.index.size() * sizeof(int32_t));
    std::memcpy(host.data(), l.descs.data(), tb);
    if (!l.index.empty()) std::memcpy(host.data() + tb, l.index.data(), l.index.size() * sizeof(int32_t));
    if (hipMemcpyAsync(tables + l.table_off, host.data(), host.size(), hipMemcpyHostToDevice, s) != hipSuccess)
      return QGEMM_ERR_HIP;
  }
  return QGEMM_OK;
}

// The grid of a launch (queries the device on first use of a kernel, so a
// graph recording calls this for every launch before it starts).
int grid_of(const Launch& l) {
  if (l.kind == kGroupMfma)
    return (int)std::max<int64_t>(1, std::min<int64_t>(l.total, (int64_t)cu_count() * blocks_per_cu(l.kind, l.cls, l.fs, l.rows)));
  return (l.nwaves + qg::kStreamWavesPerBlock - 1) / qg::kStreamWavesPerBlock;
}

// The kernels of a plan whose tables are in place: nothing but launches, so
// it can be recorded into a graph.
qgemm_status launch_plan(const Plan& P, uint8_t* tables, uint8_t* slots, hipStream_t s) {
  for (const auto& l : P.launches) {
    qg::SweepArgs args;
    std::memset(&args, 0, sizeof(args));
    args.njobs = (int32_t)l.descs.size();
    args.total = (int32_t)l.total;
    if ((int)l.descs.size() > qg::kMaxInline) {
      uint8_t* table = tables + l.table_off;
      args.table = (const JobDesc*)table;
      args.index = l.index.empty() ? nullptr : (const int32_t*)(table + l.descs.size() * sizeof(JobDesc));
      args.bshift = l.bshift;
    } else {
      for (size_t i = 0; i < l.descs.size(); i++) args.inl[i] = l.descs[i];
      args.table = nullptr;
      args.index = nullptr;
    }
    if (l.kind != kGroupMfma) {
      args.slots = (float*)(slots + l.slots_off);
#ifdef QG_TIMELINE
      args.trace = g_trace;
#endif
      args.slot_bytes = qg::stream_slot_bytes(l.nwaves, l.rows, l.kind == kStreamMfma, l.cls);
      args.spin_limit = qg::kSpinLimit;
      args.nwaves = l.nwaves;
      args.q = (int32_t)(l.total / l.nwaves);
      args.rem = (int32_t)(l.total % l.nwaves);
    }
    if (qg::launch_sweep(l.kind, l.cls, l.fs, l.rows, args, grid_of(l), s) != hipSuccess)
      return QGEMM_ERR_HIP;
  }
  return QGEMM_OK;
}

}  // namespace

extern "C" {

qgemm_status qgemm_sweep(const qgemm_job* jobs, int njobs, void* workspace, size_t ws_bytes, void* stream) {
  return qgemm_sweep_path(jobs, njobs, QGEMM_PATH_AUTO, workspace, ws_bytes, stream);
}

int qgemm_auto_path(int M) {
  if (M < 1 || M > QGEMM_MAX_M) return -1;
  return path_of(QGEMM_PATH_AUTO, M);
}

const char* qgemm_status_string(qgemm_status s) {
  switch (s) {
    case QGEMM_OK: return "ok";
    case QGEMM_ERR_INVALID_ARG: return "invalid argument";
    case QGEMM_ERR_UNSUPPORTED: return "unsupported";
    case QGEMM_ERR_NONFINITE: return "non-finite weight or fp16 scale overflow";
    case QGEMM_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

}  // extern "C"
