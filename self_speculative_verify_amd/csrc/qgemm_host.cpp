// Host side of the quantized weight sweep: argument validation, path choice,
// work planning, workspace layout and kernel launch.  Validation is pure host
// code and runs before any HIP call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "qgemm.h"
#include "qgemm_internal.h"

namespace qg {
hipError_t launch_pack(const float* W, int64_t ldw, int N, int K, int bits, void* packed,
                       unsigned* flag, hipStream_t stream);
hipError_t launch_fill_zero(void* p, int64_t words, hipStream_t stream);
int sweep_blocks_per_cu(int kind, int cls);
hipError_t launch_sweep(int kind, int cls, const SweepArgs& args, int grid, hipStream_t stream);
}  // namespace qg

namespace {

using qg::JobDesc;

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // N, K limits (32-bit tile math)
constexpr int kAutoGemvMaxM = 4;               // AUTO: GEMV for M <= 4, MFMA above

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t nkt_of(int64_t K) { return (K + qg::kTileK - 1) / qg::kTileK; }
int64_t nrb_of(int64_t N) { return (N + qg::kTileRows - 1) / qg::kTileRows; }

bool valid_shape(int bits, int64_t N, int64_t K) {
  return (bits == 4 || bits == 5) && N >= 1 && N <= kMaxDim && K >= qg::kGroup && K <= kMaxDim &&
         K % qg::kGroup == 0;
}

int path_of(int path, int M) {
  if (path == QGEMM_PATH_AUTO) return M <= kAutoGemvMaxM ? QGEMM_PATH_GEMV : QGEMM_PATH_MFMA;
  return path;
}

qgemm_status validate(const qgemm_job* jobs, int njobs, int path) {
  if (njobs < 1 || jobs == nullptr) return QGEMM_ERR_INVALID_ARG;
  if (path != QGEMM_PATH_AUTO && path != QGEMM_PATH_GEMV && path != QGEMM_PATH_MFMA)
    return QGEMM_ERR_INVALID_ARG;
  for (int i = 0; i < njobs; i++) {
    const qgemm_job& j = jobs[i];
    if (!valid_shape(j.bits, j.N, j.K)) return QGEMM_ERR_INVALID_ARG;
    if (j.M < 1 || j.M > QGEMM_MAX_M) return QGEMM_ERR_INVALID_ARG;
    if (!j.packed || !j.X || !j.Y) return QGEMM_ERR_INVALID_ARG;
    if (!aligned(j.packed, 256) || !aligned(j.X, 16) || !aligned(j.Y, 16)) return QGEMM_ERR_INVALID_ARG;
    if (j.ldx < j.K || j.ldx % 8 != 0) return QGEMM_ERR_INVALID_ARG;
    if (j.ldy < j.N || j.ldy % 4 != 0) return QGEMM_ERR_INVALID_ARG;
    if (path == QGEMM_PATH_GEMV && j.M > QGEMM_GEMV_MAX_M) return QGEMM_ERR_INVALID_ARG;
    // Y must not overlap X or the packed weights of this job
    const uintptr_t y0 = (uintptr_t)j.Y;
    const uintptr_t y1 = y0 + (uintptr_t)(((j.M - 1) * j.ldy + j.N) * sizeof(float));
    const uintptr_t x0 = (uintptr_t)j.X;
    const uintptr_t x1 = x0 + (uintptr_t)(((j.M - 1) * j.ldx + j.K) * sizeof(uint16_t));
    const uintptr_t p0 = (uintptr_t)j.packed;
    const uintptr_t p1 = p0 + (uintptr_t)(nrb_of(j.N) * nkt_of(j.K) * qg::tile_bytes(j.bits));
    if (y0 < x1 && x0 < y1) return QGEMM_ERR_INVALID_ARG;
    if (y0 < p1 && p0 < y1) return QGEMM_ERR_INVALID_ARG;
  }
  return QGEMM_OK;
}

// ---------------------------------------------------------------------------
// planning: jobs are grouped by kernel (kind, class); the workspace holds the
// job tables of launches with many jobs, the stream kernels' arrival counters
// and partial-sum slots (each region 256-byte aligned)
// ---------------------------------------------------------------------------
enum Kind { kStreamGemv = 0, kStreamMfma = 1, kGroupMfma = 2 };

struct Launch {
  int kind;
  int cls;
  std::vector<JobDesc> descs;
  int64_t total = 0;          // stream: flat tiles; group: units
  int64_t rbs = 0;            // stream: row blocks (arrival counters)
  size_t table_off = 0, counters_off = 0, slots_off = 0;
  int nwaves = 0;
};

struct Plan {
  std::vector<Launch> launches;
  size_t total = 0;
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

// Wave range boundaries (w * T / W) that fall inside a row block: each one
// costs a partial-sum exchange between two waves.
int64_t cut_row_blocks(const std::vector<JobDesc>& descs, int64_t T, int64_t W) {
  int64_t cuts = 0;
  size_t j = 0;
  for (int64_t w = 1; w < W; w++) {
    const int64_t f = w * T / W;
    while (f >= descs[j].tile_end) j++;
    if ((f - descs[j].tile_begin) % descs[j].nkt != 0) cuts++;
  }
  return cuts;
}

// Waves of a stream launch.  Every wave must get a non-empty tile range
// (contributor counts rely on it), so W <= T.  Otherwise W is chosen in
// [kStreamMinWaves, kStreamWaves] -- enough to fill the chip -- among a few
// candidates, by the fewest cut row blocks, then the most waves.  Candidates
// include the counts that give every wave a whole number of one job's row
// blocks (T / (k * NKT)).  Depends on the shapes only, never on M.
int64_t stream_waves_uncached(const std::vector<JobDesc>& descs, int64_t T) {
  if (T <= qg::kStreamMinWaves) return T;
  std::vector<int64_t> cand = {qg::kStreamMinWaves, 3072, qg::kStreamWaves};
  for (const auto& d : descs)
    for (int64_t k = 1; k <= 8; k++) {
      const int64_t per = k * d.nkt;
      if (T % per == 0) cand.push_back(T / per);
    }
  int64_t best = -1, best_cuts = 0;
  for (int64_t W : cand) {
    if (W < qg::kStreamMinWaves || W > qg::kStreamWaves || W > T) continue;
    const int64_t cuts = cut_row_blocks(descs, T, W);
    if (best < 0 || cuts < best_cuts || (cuts == best_cuts && W > best)) {
      best = W;
      best_cuts = cuts;
    }
  }
  return best < 0 ? std::min<int64_t>(T, qg::kStreamWaves) : best;
}

// The choice above walks up to kStreamWaves boundaries per candidate, which
// is too slow to repeat on every sweep call; it is a pure function of the
// launch's row-block shapes, so it is memoized per shape signature (a bounded
// cache; shapes only, never pointers or M).
int64_t stream_waves(const std::vector<JobDesc>& descs, int64_t T) {
  if (T <= qg::kStreamMinWaves) return T;
  std::vector<int64_t> key;
  key.reserve(2 * descs.size() + 1);
  key.push_back(T);
  for (const auto& d : descs) {
    key.push_back(d.nkt);
    key.push_back(d.nrb);
  }
  static std::mutex mu;
  static std::map<std::vector<int64_t>, int64_t> cache;
  {
    std::lock_guard<std::mutex> g(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  const int64_t W = stream_waves_uncached(descs, T);
  std::lock_guard<std::mutex> g(mu);
  if (cache.size() >= 256) cache.clear();
  cache.emplace(std::move(key), W);
  return W;
}

Plan make_plan(const qgemm_job* jobs, int njobs, int path) {
  Plan P;
  for (int i = 0; i < njobs; i++) {
    const qgemm_job& j = jobs[i];
    const int kind = kind_of(path, j.M);
    const int cls = class_of(kind, j.M);
    Launch* dst = nullptr;
    for (auto& l : P.launches)
      if (l.kind == kind && l.cls == cls) dst = &l;
    if (!dst) {
      P.launches.push_back(Launch{});
      dst = &P.launches.back();
      dst->kind = kind;
      dst->cls = cls;
    }
    JobDesc d;
    std::memset(&d, 0, sizeof(d));
    d.packed = (const uint8_t*)j.packed;
    d.X = j.X;
    d.Y = j.Y;
    d.ldx = j.ldx;
    d.ldy = j.ldy;
    d.N = (int32_t)j.N;
    d.K = (int32_t)j.K;
    d.M = j.M;
    d.bits = j.bits;
    d.nkt = (int32_t)nkt_of(j.K);
    d.ngroups = (int32_t)(j.K / qg::kGroup);
    d.nrb = (int32_t)nrb_of(j.N);
    if (kind == kGroupMfma) {
      const int64_t units = (d.nrb + qg::kGroupWaves - 1) / qg::kGroupWaves;
      d.unit_begin = (int32_t)dst->total;
      dst->total += units;
      d.unit_end = (int32_t)dst->total;
    } else {
      d.tile_begin = dst->total;
      dst->total += (int64_t)d.nrb * d.nkt;
      d.tile_end = dst->total;
      d.rb_begin = (int32_t)dst->rbs;
      dst->rbs += d.nrb;
    }
    dst->descs.push_back(d);
  }
  size_t off = 0;
  for (auto& l : P.launches) {
    if ((int)l.descs.size() > qg::kMaxInline) {
      l.table_off = off;
      off = round_up(off + l.descs.size() * sizeof(JobDesc), 256);
    }
    if (l.kind != kGroupMfma) {
      l.nwaves = (int)stream_waves(l.descs, l.total);
      l.counters_off = off;
      off = round_up(off + (size_t)l.rbs * sizeof(int), 256);
      l.slots_off = off;
      const int rows = l.cls;
      off = round_up(off + (size_t)2 * l.nwaves * rows * qg::kTileRows * sizeof(float), 256);
    }
  }
  P.total = off ? off : 256;
  return P;
}

int blocks_per_cu(int kind, int cls) {
  static std::mutex mu;
  static int cache[3][65] = {};
  std::lock_guard<std::mutex> g(mu);
  int& c = cache[kind][cls];
  if (c == 0) {
    c = qg::sweep_blocks_per_cu(kind, cls);
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
  return make_plan(jobs, njobs, path).total;
}

qgemm_status qgemm_workspace_init(void* workspace, size_t ws_bytes, void* stream) {
  if (!workspace || !aligned(workspace, 256) || ws_bytes % 4 != 0) return QGEMM_ERR_INVALID_ARG;
  return qg::launch_fill_zero(workspace, (int64_t)(ws_bytes / 4), (hipStream_t)stream) == hipSuccess
             ? QGEMM_OK
             : QGEMM_ERR_HIP;
}

qgemm_status qgemm_validate(const qgemm_job* jobs, int njobs, int path, void* workspace,
                            size_t ws_bytes) {
  qgemm_status st = validate(jobs, njobs, path);
  if (st != QGEMM_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  if (ws_bytes < make_plan(jobs, njobs, path).total) return QGEMM_ERR_INVALID_ARG;
  return QGEMM_OK;
}

qgemm_status qgemm_sweep_path(const qgemm_job* jobs, int njobs, int path, void* workspace,
                              size_t ws_bytes, void* stream) {
  qgemm_status st = validate(jobs, njobs, path);
  if (st != QGEMM_OK) return st;
  if (!workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  Plan P = make_plan(jobs, njobs, path);
  if (ws_bytes < P.total) return QGEMM_ERR_INVALID_ARG;
  uint8_t* ws = (uint8_t*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const int cus = cu_count();
  for (auto& l : P.launches) {
    qg::SweepArgs args;
    std::memset(&args, 0, sizeof(args));
    args.njobs = (int32_t)l.descs.size();
    args.total = l.total;
    if ((int)l.descs.size() > qg::kMaxInline) {
      JobDesc* table = (JobDesc*)(ws + l.table_off);
      if (hipMemcpyAsync(table, l.descs.data(), l.descs.size() * sizeof(JobDesc), hipMemcpyHostToDevice,
                         s) != hipSuccess)
        return QGEMM_ERR_HIP;
      args.table = table;
    } else {
      for (size_t i = 0; i < l.descs.size(); i++) args.inl[i] = l.descs[i];
      args.table = nullptr;
    }
    int grid;
    if (l.kind == kGroupMfma) {
      grid = (int)std::max<int64_t>(1, std::min<int64_t>(l.total, (int64_t)cus * blocks_per_cu(l.kind, l.cls)));
    } else {
      args.counters = (int*)(ws + l.counters_off);
      args.slots = (float*)(ws + l.slots_off);
      args.nwaves = l.nwaves;
      args.slot_rows = l.cls;
      grid = (l.nwaves + qg::kStreamWavesPerBlock - 1) / qg::kStreamWavesPerBlock;
    }
    if (qg::launch_sweep(l.kind, l.cls, args, grid, s) != hipSuccess) return QGEMM_ERR_HIP;
  }
  return QGEMM_OK;
}

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
