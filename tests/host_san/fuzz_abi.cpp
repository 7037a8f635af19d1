// Randomized calls through the library's C boundary, for a build of its host
// code under AddressSanitizer and UndefinedBehaviorSanitizer (the kernel
// launchers and HIP runtime replaced by the host stand-ins of hip_stub.cpp).
// Valid calls get buffers of exactly the documented sizes -- packed bytes,
// X and Y extents, the workspace the library asks for -- so any access past
// them is a sanitizer error; invalid calls (one argument broken) must return
// QGEMM_ERR_INVALID_ARG without launching anything.
// Usage: fuzz_abi SEED ITERATIONS.  Prints "ok <calls>" and exits 0.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <algorithm>
#include <list>
#include <vector>

#include <hip/hip_runtime.h>

#include "qgemm.h"
#include "qgemm_internal.h"

extern long g_launches;
extern long g_big_launches;
extern size_t g_scratch_bytes;

#define EXPECT(c)                                                                         \
  do {                                                                                    \
    if (!(c)) {                                                                           \
      std::fprintf(stderr, "fuzz check failed: %s (line %d, iteration %ld)\n", #c, __LINE__, g_iter); \
      std::exit(4);                                                                       \
    }                                                                                     \
  } while (0)

namespace {

long g_iter = 0;
long g_calls = 0;
std::mt19937_64 rng;
std::vector<void*> g_allocs;

int64_t rnd(int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); }

// exactly n bytes (ASan's redzone starts at byte n), 256-byte aligned
void* alloc(size_t n) {
  void* p = nullptr;
  if (posix_memalign(&p, 256, n ? n : 1) != 0) std::abort();
  g_allocs.push_back(p);
  return p;
}
void free_all() {
  for (void* p : g_allocs) std::free(p);
  g_allocs.clear();
}

const int kFmts[4] = {QGEMM_FMT_Q4, QGEMM_FMT_Q5, QGEMM_FMT_Q4_G64, QGEMM_FMT_Q4_ZP};

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

qgemm_job make_job(int M, bool big = false) {
  qgemm_job j;
  std::memset(&j, 0, sizeof(j));
  j.bits = kFmts[rnd(0, 3)];
  const int g = j.bits == QGEMM_FMT_Q4_G64 ? 64 : 32;
  j.N = big && rnd(0, 3) == 0 ? rnd(20000, 70000) : rnd(1, 3000);
  j.K = g * rnd(1, big ? 200 : 60);
  j.M = M;
  j.ldx = round_up(j.K, 8) + 8 * rnd(0, 2);
  j.ldy = round_up(j.N, 4) + 4 * rnd(0, 2);
  const size_t pb = qgemm_packed_bytes(j.bits, j.N, j.K);
  EXPECT(pb > 0);
  j.packed = alloc(pb);
  j.X = (const uint16_t*)alloc((size_t)((M - 1) * j.ldx + j.K) * 2);
  j.Y = (float*)alloc((size_t)((M - 1) * j.ldy + j.N) * 4);
  return j;
}

std::vector<qgemm_job> make_jobs(int path) {
  const int n = rnd(0, 4) == 0 ? (int)rnd(13, 40) : (int)rnd(1, 12);
  const int maxM = path == QGEMM_PATH_GEMV ? QGEMM_GEMV_MAX_M : QGEMM_MAX_M;
  std::vector<qgemm_job> jobs;
  for (int i = 0; i < n; i++) jobs.push_back(make_job((int)rnd(1, maxM), n < 4));
  // some jobs share one X (allowed: inputs may be shared)
  if (n > 1 && rnd(0, 1)) {
    const qgemm_job& a = jobs[0];
    for (auto& j : jobs)
      if (j.K == a.K && j.M == a.M && j.ldx == a.ldx) j.X = a.X;
  }
  return jobs;
}

void* workspace(size_t n) {
  EXPECT(n > 0 && n % 256 == 0);
  void* ws = alloc(n);
  EXPECT(qgemm_workspace_init(ws, n, nullptr) == QGEMM_OK);
  return ws;
}

// One argument of a valid job set broken; the call must reject it before
// any launch.
void broken_sweep(std::vector<qgemm_job> jobs, int path, void* ws, size_t wsb) {
  qgemm_job& j = jobs[rnd(0, (int64_t)jobs.size() - 1)];
  switch (rnd(0, 13)) {
    case 0: j.M = 0; break;
    case 1: j.M = QGEMM_MAX_M + 1; break;
    case 2: j.K += 16; break;
    case 3: j.N = 0; break;
    case 4: j.bits = 3; break;
    case 5: j.ldx = j.K - 8; break;
    case 6: j.ldx += 4; break;
    case 7: j.ldy = j.N - 1; break;
    case 8: j.packed = (const uint8_t*)j.packed + 128; break;
    case 9: j.X = j.X + 4; break;
    case 10: j.Y = j.Y + 1; break;
    case 11: j.Y = (float*)j.X; break;          // output over its own input
    case 12: j.Y = (float*)j.packed; break;     // output over weights
    case 13: j.packed = nullptr; break;
  }
  const long before = g_launches;
  g_calls++;
  EXPECT(qgemm_sweep_path(jobs.data(), (int)jobs.size(), path, ws, wsb, nullptr) == QGEMM_ERR_INVALID_ARG);
  EXPECT(qgemm_workspace_bytes(jobs.data(), (int)jobs.size(), path) == 0);
  EXPECT(g_launches == before);
}

void sweep_case() {
  const int path = (int)rnd(0, 2);
  std::vector<qgemm_job> jobs = make_jobs(path);
  const size_t wsb = qgemm_workspace_bytes(jobs.data(), (int)jobs.size(), path);
  void* ws = workspace(wsb);
  g_calls++;
  EXPECT(qgemm_validate(jobs.data(), (int)jobs.size(), path, ws, wsb) == QGEMM_OK);
  EXPECT(qgemm_sweep_path(jobs.data(), (int)jobs.size(), path, ws, wsb, nullptr) == QGEMM_OK);
  // a workspace one 256-byte step short is rejected
  if (wsb > 256) EXPECT(qgemm_sweep_path(jobs.data(), (int)jobs.size(), path, ws, wsb - 256, nullptr) ==
                        QGEMM_ERR_INVALID_ARG);
  // a second job's output over the first's: rejected
  if (jobs.size() > 1 && rnd(0, 1)) {
    std::vector<qgemm_job> bad = jobs;
    bad[1].Y = bad[0].Y;
    EXPECT(qgemm_sweep_path(bad.data(), (int)bad.size(), path, ws, wsb, nullptr) == QGEMM_ERR_INVALID_ARG);
  }
  broken_sweep(jobs, path, ws, wsb);
}

// Allocation-free sweeps: a few job sets in a row on the shared scratch (the
// stand-in kernels check that every launch finds its slots empty).  A set
// whose workspace exceeds the scratch is rejected before any launch.
void noalloc_case() {
  for (int i = 0, n = (int)rnd(2, 4); i < n; i++) {
    const int path = (int)rnd(0, 2);
    std::vector<qgemm_job> jobs = make_jobs(path);
    const size_t wsb = qgemm_workspace_bytes(jobs.data(), (int)jobs.size(), path);
    EXPECT(wsb > 0);
    const long before = g_launches;
    g_calls++;
    if (wsb <= g_scratch_bytes) {
      EXPECT(qgemm_sweep_noalloc(jobs.data(), (int)jobs.size(), path, nullptr) == QGEMM_OK);
      EXPECT(g_launches > before);
    } else {
      EXPECT(qgemm_sweep_noalloc(jobs.data(), (int)jobs.size(), path, nullptr) == QGEMM_ERR_INVALID_ARG);
      EXPECT(g_launches == before);
    }
  }
  // 13..40 panel-class jobs (group kernel: a job table at the top of the
  // scratch, no slots), then one sweep whose slots fill the whole scratch:
  // it must clear what the table left there
  std::vector<qgemm_job> many;
  for (int i = 0, n = (int)rnd(13, 40); i < n; i++) many.push_back(make_job((int)rnd(17, QGEMM_MAX_M)));
  EXPECT(qgemm_sweep_noalloc(many.data(), (int)many.size(), QGEMM_PATH_AUTO, nullptr) == QGEMM_OK);
  qgemm_job full;
  std::memset(&full, 0, sizeof(full));
  full.bits = QGEMM_FMT_Q4;
  full.N = 64;       // one row group of 157 k tiles: 1413 units, 128 waves
  full.K = 157 * 128;
  full.M = 1;
  full.ldx = full.K;
  full.ldy = 64;
  full.packed = alloc(qgemm_packed_bytes(full.bits, full.N, full.K));
  full.X = (const uint16_t*)alloc((size_t)full.K * 2);
  full.Y = (float*)alloc((size_t)full.N * 4);
  EXPECT(qgemm_workspace_bytes(&full, 1, QGEMM_PATH_MFMA) == g_scratch_bytes);
  EXPECT(qgemm_sweep_noalloc(&full, 1, QGEMM_PATH_MFMA, nullptr) == QGEMM_OK);
  // an argument error is rejected as by qgemm_sweep_path
  std::vector<qgemm_job> jobs = make_jobs(QGEMM_PATH_AUTO);
  jobs[0].M = 0;
  const long before = g_launches;
  EXPECT(qgemm_sweep_noalloc(jobs.data(), (int)jobs.size(), QGEMM_PATH_AUTO, nullptr) == QGEMM_ERR_INVALID_ARG);
  EXPECT(g_launches == before);
}

// A launch of at least 4 GiB of weights (the stream kernel's big step
// shape): one or several large jobs, M within the stream classes.  Only the
// ends of each buffer are touched, so the allocations stay virtual.
void big_case() {
  const int M = (int)rnd(1, 16), path = rnd(0, 1) ? QGEMM_PATH_AUTO : QGEMM_PATH_MFMA;
  const int n = rnd(0, 1) ? 1 : (int)rnd(13, 16);
  std::vector<qgemm_job> jobs;
  int64_t bytes = 0;
  for (int i = 0; i < n; i++) {
    qgemm_job j;
    std::memset(&j, 0, sizeof(j));
    j.bits = kFmts[rnd(0, 3)];
    j.K = n == 1 ? 65536 : 16384;
    j.N = n == 1 ? rnd(140000, 200000) : rnd(40000, 50000);
    j.M = M;
    j.ldx = j.K;
    j.ldy = round_up(j.N, 4);
    const size_t pb = qgemm_packed_bytes(j.bits, j.N, j.K);
    bytes += (int64_t)pb;
    j.packed = alloc(pb);
    j.X = (const uint16_t*)alloc((size_t)((M - 1) * j.ldx + j.K) * 2);
    j.Y = (float*)alloc((size_t)((M - 1) * j.ldy + j.N) * 4);
    jobs.push_back(j);
  }
  EXPECT(bytes >= ((int64_t)4 << 30));
  const size_t wsb = qgemm_workspace_bytes(jobs.data(), n, path);
  void* ws = workspace(wsb);
  g_calls++;
  const long big0 = g_big_launches;
  EXPECT(qgemm_sweep_path(jobs.data(), n, path, ws, wsb, nullptr) == QGEMM_OK);
  EXPECT(g_big_launches == big0 + 1);
  EXPECT(qgemm_sweep_path(jobs.data(), n, path, ws, wsb - 256, nullptr) == QGEMM_ERR_INVALID_ARG);
}

qgemm_job make_head(int M) {
  qgemm_job h = make_job(M, true);
  if (rnd(0, 1)) h.Y = nullptr;  // outputs not written
  return h;
}

std::vector<qgemm_slot> make_slots(int M) {
  std::vector<qgemm_slot> s;
  int row = 0;
  while (row < M && (int)s.size() < 64) {
    const int nd = (int)rnd(0, std::min(15, M - row - 1));
    s.push_back({row, nd});
    row += nd + 1;
  }
  return s;
}

void verify_case() {
  const int M = (int)rnd(1, 64);
  qgemm_job h = make_head(M);
  std::vector<qgemm_slot> sl = make_slots(M);
  int32_t* drafts = (int32_t*)alloc((size_t)M * 4);
  int32_t* argmax = (int32_t*)alloc((size_t)M * 4);
  float* maxlogit = rnd(0, 1) ? (float*)alloc((size_t)M * 4) : nullptr;
  int32_t* acc = (int32_t*)alloc(sl.size() * 4);
  const size_t wsb = qgemm_verify_workspace_bytes(&h);
  void* ws = workspace(wsb);
  g_calls++;
  EXPECT(qgemm_verify_head(&h, drafts, sl.data(), (int)sl.size(), argmax, maxlogit, acc, ws, wsb, nullptr) ==
         QGEMM_OK);
  // a slot reaching past the last row, or too small a workspace: rejected
  const long before = g_launches;
  std::vector<qgemm_slot> bad = sl;
  bad.back().ndraft += 1;
  EXPECT(qgemm_verify_head(&h, drafts, bad.data(), (int)bad.size(), argmax, maxlogit, acc, ws, wsb, nullptr) ==
         QGEMM_ERR_INVALID_ARG);
  EXPECT(qgemm_verify_head(&h, drafts, sl.data(), (int)sl.size(), argmax, maxlogit, acc, ws, wsb - 8, nullptr) ==
         QGEMM_ERR_INVALID_ARG);
  EXPECT(g_launches == before);
}

void round_case() {
  const int ns = (int)rnd(0, 5);
  std::vector<std::vector<qgemm_job>> jobsets;
  std::vector<qgemm_round_sweep> sw;
  for (int i = 0; i < ns; i++) {
    const int path = (int)rnd(0, 2);
    jobsets.push_back(make_jobs(path));
    sw.push_back({nullptr, 0, path});
  }
  for (int i = 0; i < ns; i++) {
    sw[i].jobs = jobsets[i].data();
    sw[i].njobs = (int32_t)jobsets[i].size();
  }
  const bool with_head = ns == 0 || rnd(0, 1);
  const int M = (int)rnd(1, 64);
  qgemm_job h;
  std::vector<qgemm_slot> sl;
  int32_t *drafts = nullptr, *argmax = nullptr, *acc = nullptr;
  if (with_head) {
    h = make_head(M);
    sl = make_slots(M);
    drafts = (int32_t*)alloc((size_t)M * 4);
    argmax = (int32_t*)alloc((size_t)M * 4);
    acc = (int32_t*)alloc(sl.size() * 4);
  }
  const qgemm_job* hp = with_head ? &h : nullptr;
  const size_t wsb = qgemm_round_workspace_bytes(sw.data(), ns, hp);
  void* ws = workspace(wsb);
  qgemm_round* r = nullptr;
  g_calls++;
  EXPECT(qgemm_round_create(sw.data(), ns, hp, drafts, sl.data(), (int)sl.size(), argmax, nullptr, acc, ws, wsb,
                            nullptr, &r) == QGEMM_OK);
  EXPECT(r != nullptr);
  const long before = g_launches;
  for (int rep = 0; rep < 2; rep++) EXPECT(qgemm_round_launch(r, nullptr) == QGEMM_OK);
  EXPECT(g_launches == before);  // a replay records nothing new
  qgemm_round_destroy(r);
  qgemm_round* r2 = nullptr;
  if (wsb > 256)
    EXPECT(qgemm_round_create(sw.data(), ns, hp, drafts, sl.data(), (int)sl.size(), argmax, nullptr, acc, ws,
                              wsb - 256, nullptr, &r2) == QGEMM_ERR_INVALID_ARG &&
           r2 == nullptr);
}

// The round cache against a model of its LRU order: a few round
// descriptions (some with a head), a random sequence of runs, the hit flag,
// size and counters checked after every call; the cache owns and frees the
// workspaces (the sanitizers see a leak or a double free).
void round_cache_case() {
  const int nkeys = (int)rnd(1, 4), cap = (int)rnd(1, 3);
  std::vector<std::vector<std::vector<qgemm_job>>> jobsets(nkeys);
  std::vector<std::vector<qgemm_round_sweep>> sws(nkeys);
  std::vector<qgemm_job> heads(nkeys);
  std::vector<std::vector<qgemm_slot>> slots(nkeys);
  std::vector<int32_t*> drafts(nkeys), argmax(nkeys), acc(nkeys);
  for (int k = 0; k < nkeys; k++) {
    const int ns = (int)rnd(1, 3);
    std::vector<int> paths;
    for (int i = 0; i < ns; i++) {
      paths.push_back((int)rnd(0, 2));
      jobsets[k].push_back(make_jobs(paths.back()));
    }
    for (int i = 0; i < ns; i++)
      sws[k].push_back({jobsets[k][i].data(), (int32_t)jobsets[k][i].size(), (int32_t)paths[i]});
    if (rnd(0, 1)) {
      const int M = (int)rnd(1, 64);
      heads[k] = make_head(M);
      slots[k] = make_slots(M);
      drafts[k] = (int32_t*)alloc((size_t)M * 4);
      argmax[k] = (int32_t*)alloc((size_t)M * 4);
      acc[k] = (int32_t*)alloc(slots[k].size() * 4);
    }
  }
  qgemm_round_cache* c = nullptr;
  EXPECT(qgemm_round_cache_create(cap, &c) == QGEMM_OK && c != nullptr);
  std::list<int> model;  // front: most recent
  uint64_t hits = 0, misses = 0, evictions = 0;
  for (int t = 0; t < 10; t++) {
    const int k = (int)rnd(0, nkeys - 1);
    const bool hk = argmax[k] != nullptr;
    int hit = -1;
    g_calls++;
    EXPECT(qgemm_round_cache_run(c, sws[k].data(), (int)sws[k].size(), hk ? &heads[k] : nullptr, drafts[k],
                                 hk ? slots[k].data() : nullptr, hk ? (int)slots[k].size() : 0, argmax[k],
                                 nullptr, acc[k], nullptr, &hit) == QGEMM_OK);
    auto it = std::find(model.begin(), model.end(), k);
    const bool want = it != model.end();
    EXPECT(hit == (want ? 1 : 0));
    if (want) {
      model.erase(it);
      hits++;
    } else {
      misses++;
      if ((int)model.size() >= cap) {
        model.pop_back();
        evictions++;
      }
    }
    model.push_front(k);
    int size = -1;
    uint64_t h = 0, m = 0, e = 0;
    EXPECT(qgemm_round_cache_stats(c, &size, &h, &m, &e) == QGEMM_OK);
    EXPECT(size == (int)model.size() && h == hits && m == misses && e == evictions);
  }
  // an invalid miss changes nothing
  std::vector<qgemm_job> badj = jobsets[0][0];
  badj[0].K = 100;
  const qgemm_round_sweep bad = {badj.data(), (int32_t)badj.size(), 0};
  int hit = 7;
  EXPECT(qgemm_round_cache_run(c, &bad, 1, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                               &hit) == QGEMM_ERR_INVALID_ARG && hit == 0);
  int size = -1;
  EXPECT(qgemm_round_cache_stats(c, &size, nullptr, nullptr, nullptr) == QGEMM_OK && size == (int)model.size());
  qgemm_round_cache_destroy(c);
}

void attn_case() {
  const int n = (int)rnd(1, QGEMM_ATTN_MAX_SLOTS);
  const int kv = (int)rnd(0, 1);
  const size_t esz = kv == QGEMM_KV_FP8 ? 1 : 2;
  std::vector<qgemm_attn_slot> s(n);
  for (auto& x : s) {
    x.W = (int32_t)rnd(1, QGEMM_ATTN_MAX_W);
    x.L = (int32_t)(rnd(0, 5) == 0 ? rnd(x.W, 40000) : rnd(x.W, 3000));
    const size_t hq = QGEMM_ATTN_HKV * QGEMM_ATTN_GROUP;
    x.Q = (const uint16_t*)alloc((size_t)x.W * hq * QGEMM_ATTN_D * 2);
    x.K = alloc((size_t)x.L * QGEMM_ATTN_HKV * QGEMM_ATTN_D * esz);
    x.V = alloc((size_t)x.L * QGEMM_ATTN_HKV * QGEMM_ATTN_D * esz);
    x.O = (float*)alloc((size_t)x.W * hq * QGEMM_ATTN_D * 4);
  }
  const size_t wsb = qgemm_attn_workspace_bytes(s.data(), n, kv);
  EXPECT(wsb > 0);
  void* ws = alloc(wsb);
  g_calls++;
  EXPECT(qgemm_attn_verify(s.data(), n, kv, 0.0625f, ws, wsb, nullptr) == QGEMM_OK);
  const long before = g_launches;
  std::vector<qgemm_attn_slot> bad = s;
  qgemm_attn_slot& b = bad[rnd(0, n - 1)];
  switch (rnd(0, 5)) {
    case 0: b.W = 0; break;
    case 1: b.W = QGEMM_ATTN_MAX_W + 1; break;
    case 2: b.L = b.W - 1; break;
    case 3: b.O = (float*)b.K; break;
    case 4: b.Q = b.Q + 1; break;
    case 5: b.V = nullptr; break;
  }
  EXPECT(qgemm_attn_verify(bad.data(), n, kv, 0.0625f, ws, wsb, nullptr) == QGEMM_ERR_INVALID_ARG);
  EXPECT(qgemm_attn_verify(s.data(), n, kv, 0.0625f, ws, wsb - 256, nullptr) == QGEMM_ERR_INVALID_ARG);
  EXPECT(g_launches == before);
}

void pack_case() {
  const int bits = kFmts[rnd(0, 3)];
  const int g = bits == QGEMM_FMT_Q4_G64 ? 64 : 32;
  const int64_t N = rnd(1, 700), K = g * rnd(1, 40), ldw = K + rnd(0, 5);
  float* W = (float*)alloc((size_t)((N - 1) * ldw + K) * 4);
  const size_t pb = qgemm_packed_bytes(bits, N, K);
  EXPECT(pb > 0);
  void* packed = alloc(pb);
  g_calls++;
  EXPECT(qgemm_pack(W, ldw, N, K, bits, packed, nullptr) == QGEMM_OK);
  EXPECT(qgemm_packed_bytes(bits, N, K + 16) == 0 || g == 32);
  EXPECT(qgemm_pack(W, K - 1, N, K, bits, packed, nullptr) == QGEMM_ERR_INVALID_ARG);
}

}  // namespace

// The planning code's division by a job's k-tile count goes through
// div_magic: exact for every count 1 .. 2^17 and dividend 0 .. 2^31 - 1 --
// checked here at the dividends where an error would show first (around
// multiples of the divisor and at the top of the range) and at random ones.
void div_magic_check() {
  for (uint32_t d = 1; d <= (1u << 17); d++) {
    uint32_t m;
    int32_t sh;
    qg::div_magic(d, m, sh);
    auto q = [&](uint64_t x) { return (uint64_t)((x * m) >> sh); };
    const uint64_t top = (1ull << 31) - 1;
    for (uint64_t x : {(uint64_t)0, (uint64_t)1, (uint64_t)d - 1, (uint64_t)d, (uint64_t)d + 1, top, top - top % d,
                       top - top % d - 1, (uint64_t)rnd(0, (int64_t)top)}) {
      EXPECT(q(x) == x / d);
    }
    for (uint64_t k = 2; k <= 64 && k * d <= top; k *= 2) {
      EXPECT(q(k * d) == k && q(k * d - 1) == k - 1);
    }
  }
}

int main(int argc, char** argv) {
  if (argc != 3) {
    std::fprintf(stderr, "usage: fuzz_abi SEED ITERATIONS\n");
    return 2;
  }
  rng.seed(std::strtoull(argv[1], nullptr, 10));
  const long iters = std::strtol(argv[2], nullptr, 10);
  div_magic_check();
  for (g_iter = 0; g_iter < iters; g_iter++) {
    if (g_iter % 50 == 49) {
      big_case();
      free_all();
      continue;
    }
    switch (rnd(0, 7)) {
      case 0: case 1: sweep_case(); break;
      case 2: verify_case(); break;
      case 3: round_case(); break;
      case 4: attn_case(); break;
      case 5: pack_case(); break;
      case 6: noalloc_case(); break;
      case 7: round_cache_case(); break;
    }
    free_all();
  }
  std::printf("ok %ld\n", g_calls);
  return 0;
}
