// Read ceiling of one sweep launch (a measurement kernel, not part of the
// sweep): the bytes a stream-kernel launch loads, loaded with the same
// geometry -- the same waves (four per workgroup, the stream kernels' count),
// the same partition of weight units over them, the same steps (four row
// blocks of 16 rows at one k tile), the same per-lane loads of codes, scales
// and high bits, the same X chunk per step and two steps in flight -- but no
// unpack, no contraction and no split-K exchange.  Its time is what one
// launch of the sweep's access pattern can stream; the sweep's time is
// judged against it beside the HBM peak (the EXL3-K5K6 model card,
// multi-GPU section, judges its GEMMs by a measured stream ceiling rather
// than the bandwidth the part is rated for).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "read_ceiling.h"

namespace {

typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

constexpr int kRows = 4;          // row blocks per step
constexpr int kDepth = 2;         // steps in flight per wave
constexpr int kWavesPerBlock = 4;

struct Job {
  const uint8_t* packed;
  const uint8_t* X;
  int64_t ldx_bytes;
  int32_t nrb, nkt, tb, wt;       // row blocks, k tiles, tile bytes, units per step
  int32_t steps, ubeg;            // steps (row groups x k tiles), first unit
};

struct Args {
  Job job[QGEMM_CEILING_MAX_JOBS];
  int32_t njobs, nwaves, total, xrows;
  uint32_t* sink;
};

struct Step {
  u4_t c[kRows];
  u2_t s[kRows];
  uint32_t h[kRows];
  u4_t x[4];
};

// the first step of job j whose first unit is >= u (units relative to the job)
__device__ __forceinline__ int first_step(int u, int wt) { return (u + wt - 1) / wt; }

template <bool kHi, int kXP>
__device__ __forceinline__ void load(Step& t, const Job& J, int s, int xrows, int lane) {
  const int rg = s / J.nkt, kt = s - rg * J.nkt;
  const uint32_t rstride = (uint32_t)(J.nkt * J.tb);
  const int left = J.nrb - 1 - rg * kRows;
  const uint8_t* wp = J.packed + ((int64_t)rg * kRows * J.nkt + kt) * J.tb;
#pragma unroll
  for (int r = 0; r < kRows; r++) {
    const uint8_t* tp = wp + (uint32_t)(r < left ? r : left) * rstride;
    t.c[r] = __builtin_nontemporal_load((const u4_t*)(tp + 16 * lane));
    t.s[r] = __builtin_nontemporal_load((const u2_t*)(tp + 1024 + 8 * (lane & 15)));
    if (kHi) t.h[r] = __builtin_nontemporal_load((const uint32_t*)(tp + 1152 + 4 * lane));
  }
#pragma unroll
  for (int p = 0; p < kXP; p++) {
    int row = 4 * p + (lane >> 4);
    row = row < xrows ? row : xrows - 1;  // rows past the panel read its last one, as the sweep does
    t.x[p] = *(const u4_t*)(J.X + (int64_t)row * J.ldx_bytes + 256 * kt + 16 * (lane & 15));
  }
}

template <bool kHi, int kXP>
__device__ __forceinline__ uint32_t fold(const Step& t) {
  uint32_t a = 0;
#pragma unroll
  for (int r = 0; r < kRows; r++) {
    a ^= t.c[r].x ^ t.c[r].y ^ t.c[r].z ^ t.c[r].w ^ t.s[r].x ^ t.s[r].y;
    if (kHi) a ^= t.h[r];
  }
#pragma unroll
  for (int p = 0; p < kXP; p++) a ^= t.x[p].x ^ t.x[p].w;
  return a;
}

// kHi: the launch holds 5-bit tiles (high-bit words read in every tile of a
// 5-bit job); kXP: 16-byte X pieces per lane and step (rows / 4)
template <bool kHi, int kXP>
__global__ void __launch_bounds__(64 * kWavesPerBlock) ceiling_kernel(Args a) {
  const int lane = threadIdx.x & 63;
  const int gw = (int)blockIdx.x * kWavesPerBlock + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (gw >= a.nwaves) return;
  // the wave's units [u0, u1): equal contiguous ranges
  const int q = a.total / a.nwaves, rem = a.total % a.nwaves;
  const int u0 = gw * q + (gw < rem ? gw : rem), u1 = u0 + q + (gw < rem ? 1 : 0);
  uint32_t acc = 0;
  for (int j = 0; j < a.njobs; j++) {
    const Job& J = a.job[j];
    const int lo = u0 > J.ubeg ? u0 - J.ubeg : 0;
    const int hi = u1 - J.ubeg;
    if (hi <= 0 || lo >= J.steps * J.wt) continue;
    const int s0 = first_step(lo, J.wt);
    int s1 = first_step(hi, J.wt);
    s1 = s1 < J.steps ? s1 : J.steps;
    if (s0 >= s1) continue;
    const bool hib = kHi && J.tb == 1408;
    Step buf[kDepth];
#pragma unroll
    for (int p = 0; p < kDepth; p++) {
      const int s = s0 + p < s1 ? s0 + p : s1 - 1;
      if (hib) load<true, kXP>(buf[p], J, s, a.xrows, lane);
      else load<false, kXP>(buf[p], J, s, a.xrows, lane);
    }
    for (int s = s0; s < s1; s += kDepth) {
#pragma unroll
      for (int p = 0; p < kDepth; p++) {
        if (s + p < s1) acc ^= hib ? fold<true, kXP>(buf[p]) : fold<false, kXP>(buf[p]);
        const int n = s + p + kDepth < s1 ? s + p + kDepth : s1 - 1;
        if (s + p + kDepth < s1) {
          if (hib) load<true, kXP>(buf[p], J, n, a.xrows, lane);
          else load<false, kXP>(buf[p], J, n, a.xrows, lane);
        }
      }
    }
  }
  // one word per wave keeps every load live
  acc = __builtin_amdgcn_readfirstlane(acc) ^ (uint32_t)__builtin_popcountll(__ballot(acc & 1));
  if (lane == 0) a.sink[gw] = acc;
}

}  // namespace

extern "C" int qgemm_read_ceiling(const qgemm_ceiling_job* jobs, int njobs, int nwaves, int xrows,
                                  uint32_t* sink, void* stream) {
  if (!jobs || njobs < 1 || njobs > QGEMM_CEILING_MAX_JOBS || !sink) return 1;
  if (nwaves < 1 || nwaves > QGEMM_CEILING_MAX_WAVES || xrows < 1 || xrows > 16) return 1;
  Args a = {};
  a.njobs = njobs;
  a.nwaves = nwaves;
  a.sink = sink;
  a.xrows = xrows;
  bool any5 = false;
  int64_t units = 0;
  for (int j = 0; j < njobs; j++) {
    const qgemm_ceiling_job& c = jobs[j];
    if (!c.packed || !c.X || (c.bits != 4 && c.bits != 5) || c.N < 1 || c.K < 128 || c.K % 128 != 0 ||
        c.ldx < c.K)
      return 1;
    Job& J = a.job[j];
    J.packed = (const uint8_t*)c.packed;
    J.X = (const uint8_t*)c.X;
    J.ldx_bytes = 2 * c.ldx;
    J.nrb = (int32_t)((c.N + 15) / 16);
    J.nkt = (int32_t)(c.K / 128);
    J.tb = c.bits == 5 ? 1408 : 1152;
    J.wt = c.bits == 5 ? 11 : 9;
    const int64_t steps = (int64_t)((J.nrb + kRows - 1) / kRows) * J.nkt;
    if (steps * J.wt + units >= ((int64_t)1 << 31)) return 1;
    J.steps = (int32_t)steps;
    J.ubeg = (int32_t)units;
    units += steps * J.wt;
    any5 = any5 || c.bits == 5;
  }
  if (units < (int64_t)nwaves * 11) return 1;  // every wave holds at least one step
  a.total = (int32_t)units;
  const int xp = (xrows + 3) / 4;
  const dim3 grid((unsigned)((nwaves + kWavesPerBlock - 1) / kWavesPerBlock)), block(64 * kWavesPerBlock);
  hipStream_t s = (hipStream_t)stream;
  // X pieces per lane: 1, 2 or 4 (rows 1-4, 5-8, 9-16)
  if (any5) {
    if (xp == 1) hipLaunchKernelGGL((ceiling_kernel<true, 1>), grid, block, 0, s, a);
    else if (xp == 2) hipLaunchKernelGGL((ceiling_kernel<true, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((ceiling_kernel<true, 4>), grid, block, 0, s, a);
  } else {
    if (xp == 1) hipLaunchKernelGGL((ceiling_kernel<false, 1>), grid, block, 0, s, a);
    else if (xp == 2) hipLaunchKernelGGL((ceiling_kernel<false, 2>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((ceiling_kernel<false, 4>), grid, block, 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
