// Internal definitions shared by the host side and the gfx950 kernels of the
// shared-KV attention verify.  Not part of the public boundary.
#pragma once

#include <stdint.h>

namespace qa {

// Geometry of the full-attention layers: 4 KV heads of 256 dims, 6 query
// heads per KV head (24 query heads).
constexpr int kHkv = 4;
constexpr int kGroup = 6;
constexpr int kHq = kHkv * kGroup;
constexpr int kD = 256;

constexpr int kMaxW = 16;                  // verify positions per slot
constexpr int kMaxRows = kGroup * kMaxW;   // query rows per KV head: (position, head in group)
constexpr int kMb = kMaxRows / 16;         // 16-row blocks, one wave each
constexpr int kThreads = 64 * kMb;
constexpr int kBlk = 32;                   // cache positions per step
constexpr int kMaxSlots = 16;

struct AttnSlot {
  const uint16_t* Q;   // binary16 [W][kHq][kD]
  const uint8_t* K;    // [L][kHkv][kD] elements of 2 (fp16) or 1 (E4M3) bytes
  const uint8_t* V;
  float* O;            // fp32 [W][kHq][kD]
  int32_t L, W;
  int32_t nchunks;     // ceil(L / chunk)
  int32_t part0;       // partial of (slot, KV head g, chunk c): part0 + g * nchunks + c
};

struct AttnArgs {
  AttnSlot s[kMaxSlots];
  int32_t nslots;
  int32_t chunk;        // positions per workgroup, a multiple of kBlk
  float scale_log2e;    // softmax scale times log2(e): scores in base-2 units
  int32_t pad_;
  float* part_o;        // [part][kMaxRows][kD] unnormalized outputs
  float* part_ml;       // [part][kMaxRows][2]: running maximum (base 2), sum
};

}  // namespace qa
