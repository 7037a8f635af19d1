// Host side of the shared-KV attention verify: argument checks (host only,
// before any HIP call), the chunking of each slot's cache positions, the
// workspace layout of the per-chunk partials, and the two launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn_internal.h"
#include "qgemm.h"

namespace qa {
hipError_t launch_attn(const AttnArgs& a, bool fp8, int max_chunks, hipStream_t stream);
}

namespace {

constexpr int64_t kMaxL = (int64_t)1 << 24;
// partials of one (slot, KV head, chunk): kMaxRows rows of kD outputs, then
// kMaxRows (maximum, sum) pairs, in two arrays
constexpr size_t kPartO = (size_t)qa::kMaxRows * qa::kD * sizeof(float);
constexpr size_t kPartML = (size_t)qa::kMaxRows * 2 * sizeof(float);
// workgroups a launch aims at (every slot's positions cut into chunks of a
// common length, a multiple of the 32-position step, at least kMinChunk so
// that the partials stay small next to the cache bytes they summarize)
constexpr int64_t kTargetGroups = 256;
constexpr int64_t kMinChunk = 256;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

qgemm_status check(const qgemm_attn_slot* slots, int nslots, int kv) {
  if (!slots || nslots < 1 || nslots > qa::kMaxSlots) return QGEMM_ERR_INVALID_ARG;
  if (kv != QGEMM_KV_FP16 && kv != QGEMM_KV_FP8) return QGEMM_ERR_INVALID_ARG;
  const size_t esz = kv == QGEMM_KV_FP8 ? 1 : 2;
  for (int i = 0; i < nslots; i++) {
    const qgemm_attn_slot& s = slots[i];
    if (!s.Q || !s.K || !s.V || !s.O) return QGEMM_ERR_INVALID_ARG;
    if (!aligned(s.Q, 16) || !aligned(s.K, 16) || !aligned(s.V, 16) || !aligned(s.O, 16))
      return QGEMM_ERR_INVALID_ARG;
    if (s.W < 1 || s.W > qa::kMaxW || s.L < s.W || s.L > kMaxL) return QGEMM_ERR_INVALID_ARG;
  }
  // an output may not overlap any slot's inputs or another output
  for (int i = 0; i < nslots; i++) {
    const qgemm_attn_slot& s = slots[i];
    const size_t no = (size_t)s.W * qa::kHq * qa::kD * 4;
    for (int j = 0; j < nslots; j++) {
      const qgemm_attn_slot& t = slots[j];
      const size_t nq = (size_t)t.W * qa::kHq * qa::kD * 2;
      const size_t nkv = (size_t)t.L * qa::kHkv * qa::kD * esz;
      if (overlaps(s.O, no, t.Q, nq) || overlaps(s.O, no, t.K, nkv) || overlaps(s.O, no, t.V, nkv))
        return QGEMM_ERR_INVALID_ARG;
      if (j != i && overlaps(s.O, no, t.O, (size_t)t.W * qa::kHq * qa::kD * 4)) return QGEMM_ERR_INVALID_ARG;
    }
  }
  return QGEMM_OK;
}

// Chunk length and partial count of a launch (depends on the slots' L only).
void plan(const qgemm_attn_slot* slots, int nslots, int& chunk, int64_t& parts, int& max_chunks) {
  int64_t positions = 0;
  for (int i = 0; i < nslots; i++) positions += (int64_t)slots[i].L * qa::kHkv;
  const int64_t per = (positions + kTargetGroups - 1) / kTargetGroups;
  chunk = (int)std::max<int64_t>(kMinChunk, (per + qa::kBlk - 1) / qa::kBlk * qa::kBlk);
  parts = 0;
  max_chunks = 0;
  for (int i = 0; i < nslots; i++) {
    const int n = (int)((slots[i].L + chunk - 1) / chunk);
    parts += (int64_t)n * qa::kHkv;
    max_chunks = std::max(max_chunks, n);
  }
}

}  // namespace

extern "C" {

size_t qgemm_attn_workspace_bytes(const qgemm_attn_slot* slots, int nslots, int kv) {
  if (check(slots, nslots, kv) != QGEMM_OK) return 0;
  int chunk, max_chunks;
  int64_t parts;
  plan(slots, nslots, chunk, parts, max_chunks);
  return round_up((size_t)parts * kPartO, 256) + round_up((size_t)parts * kPartML, 256);
}

qgemm_status qgemm_attn_verify(const qgemm_attn_slot* slots, int nslots, int kv, float scale, void* workspace,
                               size_t ws_bytes, void* stream) {
  const qgemm_status st = check(slots, nslots, kv);
  if (st != QGEMM_OK) return st;
  if (!std::isfinite(scale) || !workspace || !aligned(workspace, 256)) return QGEMM_ERR_INVALID_ARG;
  int chunk, max_chunks;
  int64_t parts;
  plan(slots, nslots, chunk, parts, max_chunks);
  const size_t o_bytes = round_up((size_t)parts * kPartO, 256);
  if (ws_bytes < o_bytes + round_up((size_t)parts * kPartML, 256)) return QGEMM_ERR_INVALID_ARG;
  qa::AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.nslots = nslots;
  a.chunk = chunk;
  a.scale_log2e = (float)((double)scale * 1.4426950408889634);
  a.part_o = (float*)workspace;
  a.part_ml = (float*)((uint8_t*)workspace + o_bytes);
  int64_t part = 0;
  for (int i = 0; i < nslots; i++) {
    qa::AttnSlot& d = a.s[i];
    d.Q = slots[i].Q;
    d.K = (const uint8_t*)slots[i].K;
    d.V = (const uint8_t*)slots[i].V;
    d.O = slots[i].O;
    d.L = slots[i].L;
    d.W = slots[i].W;
    d.nchunks = (slots[i].L + chunk - 1) / chunk;
    d.part0 = (int32_t)part;
    part += (int64_t)d.nchunks * qa::kHkv;
  }
  return qa::launch_attn(a, kv == QGEMM_KV_FP8, max_chunks, (hipStream_t)stream) == hipSuccess ? QGEMM_OK
                                                                                              : QGEMM_ERR_HIP;
}

}  // extern "C"
