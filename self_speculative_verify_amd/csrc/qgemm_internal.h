// Internal definitions shared by the host dispatcher and the gfx950 kernels of
// the quantized weight sweep.  Not part of the public boundary.
#pragma once

#include <stdint.h>

namespace qg {

constexpr int kTileRows = 16;        // rows n per tile
constexpr int kTileK = 128;          // k per tile (four groups of 32)
constexpr int kGroup = 32;           // k per scale group
constexpr int kScaleOff = 1024;      // 16 rows x 4 fp16 scales
constexpr int kHiOff = 1152;         // 5-bit: bit 4 of every code
constexpr int kTile4 = 1152;
constexpr int kTile5 = 1408;

constexpr int kMaxInline = 12;       // jobs passed by value in the kernel arguments
constexpr int kXRowBytes = 272;      // LDS row stride of a staged X chunk (256 + 16 pad)

// stream kernel (panels of at most 16 rows): waves per workgroup, and the
// range of waves in the grid (8 to 16 per CU of a 256-CU MI355X).  The count
// is chosen from the shapes alone -- never from the device or M -- so the K
// split of every row block, and with it every output bit, is reproducible.
constexpr int kStreamWavesPerBlock = 4;
constexpr int kStreamMinWaves = 2048;
constexpr int kStreamWaves = 4096;
// group kernel (17..64 rows): waves per workgroup, one 16-row block each
constexpr int kGroupWaves = 8;

inline __host__ __device__ int tile_bytes(int bits) { return bits == 4 ? kTile4 : kTile5; }

// One job as the kernels see it.  All sizes are derived on the host.
struct JobDesc {
  const uint8_t* packed;
  const uint16_t* X;
  float* Y;
  int64_t ldx;
  int64_t ldy;
  int64_t tile_begin;    // stream kernel: first flat tile of this job
  int64_t tile_end;
  int32_t N, K;
  int32_t M, bits;
  int32_t nkt;           // ceil(K / 128)
  int32_t ngroups;       // K / 32
  int32_t nrb;           // ceil(N / 16)
  int32_t rb_begin;      // stream kernel: first arrival counter of this job
  int32_t unit_begin;    // group kernel: first unit (row-block group) of this job
  int32_t unit_end;
};

struct SweepArgs {
  const JobDesc* table;  // device copy of all jobs (when njobs > kMaxInline), else null
  int* counters;         // stream kernel: arrival counter per row block (zero between calls)
  float* slots;          // stream kernel: two partial-sum slots per wave
  int64_t total;         // stream kernel: flat tiles; group kernel: units
  int32_t njobs;
  int32_t nwaves;        // stream kernel: waves in the grid (fixes the K split)
  int32_t slot_rows;     // stream kernel: rows per slot
  int32_t pad_;
  JobDesc inl[kMaxInline];
};

}  // namespace qg
