// gfx950 kernels of the shared-KV attention verify.
//
// A verify round scores W positions per slot (the accepted token and its
// drafts, already appended to the slot's cache): query w at position
// L - W + w attends causally to positions 0 .. L - W + w.  The 6 query heads
// of a KV head at all W positions -- up to 96 query rows -- read that head's
// keys and values once ("shared-KV verify", Quasar/q27 wiki, intro bullets),
// as the weight sweep's panel rows share one weight read.
//
// attn_partial: one workgroup per (slot, KV head, chunk of positions), one
// wave per 16-row block of queries.  Per step of 32 positions the keys and
// the values go through LDS as they lie in the cache ([position][dim]),
// widened to binary16 when the cache is E4M3 (exactly, by the hardware
// conversion).  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_16x16x32_f16 (A = 16 positions x 32 dims of K, B = 32 dims x
// 16 query rows of Q), so lane l
// holds 8 scores of query row l % 16: positions 4c .. 4c + 3 and 16 + 4c ..
// 16 + 4c + 3 of the step (c = l / 16).  The online softmax keeps a running
// maximum per row (base-2 units) and a per-lane partial sum; the
// probabilities, rounded to binary16, are then exactly the B operand of the
// value product O^T += V^T P^T (A = 16 dims x those 8 positions of V, read
// transposed out of the row-major tile by gfx950's transposing LDS read,
// ds_read_b64_tr_b16), whose accumulator again holds row l % 16 in
// lane l, so the rescaling by exp2(m_old - m_new) is one multiply per value.
// Each chunk leaves its unnormalized output, maximum and sum in the
// workspace; attn_combine merges the chunks of every row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_internal.h"

namespace qa {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

// LDS rows padded so that the rows one fragment read touches fall on
// distinct banks.
constexpr int kKRow = kD + 8;                // halves per K row (528 bytes)
constexpr int kVRow = kD + 16;               // halves per V row (544 bytes: 4 rows step 8 banks)
constexpr int kKBytes = kBlk * kKRow * 2;
constexpr int kVBytes = kBlk * kVRow * 2;
constexpr int kBufBytes = kKBytes + kVBytes;   // one step's tiles; two buffers alternate

// Two E4M3 bytes of the word u (bytes 0-1, or 2-3 when kHi) -> two
// binary16 values: gfx950's scaled conversion with scale 1, exact for every
// code (E4M3 values are binary16 values; the attention tests compare the
// decoded rows with the format's definition for all 256 codes, NaN
// included).
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_h2(uint32_t u) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, kHi));
}

// Global pieces (16 bytes) of one step, for KV head g, in registers, read
// piece-fastest (a position's 512 or 256 bytes by consecutive lanes) and
// written to LDS row by row ([position][dim]) for K and V alike; the value
// product reads V transposed with gfx950's transposing LDS read.
template <bool kFp8>
struct Tile {
  // a piece is 8 cached elements: 16 bytes of binary16, or 8 E4M3 bytes
  // that widen to 16; either way one 16-byte LDS write per piece, and the
  // pieces of a position are consecutive lanes (no bank conflicts)
  static constexpr int kE = kFp8 ? 1 : 2;                 // bytes per cached element
  static constexpr int kPerPos = kD / 8;                  // pieces per position and head
  static constexpr int kPieces = kBlk * kPerPos;          // per tensor and step
  static constexpr int kIters = (kPieces + kThreads - 1) / kThreads;
  typedef typename std::conditional<kFp8, u2_t, u4_t>::type piece_t;
  piece_t k[kIters], v[kIters];

  // positions >= L read as zeros (they are masked; a zero keeps their
  // products zero)
  __device__ __forceinline__ void load(const uint8_t* K, const uint8_t* V, int g, int p0, int L, int tid) {
#pragma unroll
    for (int i = 0; i < kIters; i++) {
      const int q = tid + kThreads * i;
      k[i] = v[i] = piece_t{};
      if (q >= kPieces) continue;
      const int p = p0 + q / kPerPos, piece = q % kPerPos;
      if (p < L) {
        const size_t off = ((size_t)p * kHkv + g) * (kD * kE) + piece * 8 * kE;
        k[i] = __builtin_nontemporal_load((const piece_t*)(K + off));
        v[i] = __builtin_nontemporal_load((const piece_t*)(V + off));
      }
    }
  }

  static __device__ __forceinline__ u4_t widen(const piece_t& x) {
    if constexpr (kFp8)
      return u4_t{e4m3x2_to_h2<false>(x[0]), e4m3x2_to_h2<true>(x[0]), e4m3x2_to_h2<false>(x[1]),
                  e4m3x2_to_h2<true>(x[1])};
    else
      return x;
  }

  // Into LDS: K and V at [position][dim] (binary16).
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
    _Float16* ks = (_Float16*)lds;
    _Float16* vs = (_Float16*)(lds + kKBytes);
#pragma unroll
    for (int i = 0; i < kIters; i++) {
      const int q = tid + kThreads * i;
      if (q >= kPieces) continue;
      const int p = q / kPerPos, d0 = (q % kPerPos) * 8;
      *(u4_t*)(ks + p * kKRow + d0) = widen(k[i]);
      *(u4_t*)(vs + p * kVRow + d0) = widen(v[i]);
    }
  }
};

// Running softmax state of one lane's query row: maximum (base-2 units) and
// this lane's part of the sum.
struct Row {
  float m, l;
};

// One step of 32 positions from the LDS tiles: scores, online softmax, and
// the value product into acc.  kH splits the dims of the score product into
// kH independent accumulation chains per position block (more chains hide
// the MFMA dependency latency at the cost of registers).
template <int kH>
__device__ __forceinline__ void step(Row& st_, f4_t (&acc)[kD / 16], const h8_t (&qf)[kD / 32], const _Float16* ks,
                                     const _Float16* vt, int pb, int lim, int lane, float scale_log2e) {
  const int c = lane >> 4;
  // S^T for positions pb .. pb + 15 and pb + 16 .. pb + 31: 2 kH chains
  // (two position blocks x kH parts of the dims), interleaved, then the parts
  // added
  f4_t sh[2][kH];
#pragma unroll
  for (int sb = 0; sb < 2; sb++)
#pragma unroll
    for (int h = 0; h < kH; h++) sh[sb][h] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < kD / 32 / kH; s++)
#pragma unroll
    for (int h = 0; h < kH; h++)
#pragma unroll
      for (int sb = 0; sb < 2; sb++) {
        const int ds = h * (kD / 32 / kH) + s;
        const h8_t kf = *(const h8_t*)(ks + (16 * sb + (lane & 15)) * kKRow + 32 * ds + 8 * c);
        sh[sb][h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[ds], sh[sb][h], 0, 0, 0);
      }
  f4_t st[2] = {sh[0][0], sh[1][0]};
#pragma unroll
  for (int h = 1; h < kH; h++) {
    st[0] += sh[0][h];
    st[1] += sh[1][h];
  }
  // element j of this lane: position pb + (j < 4 ? 4c + j : 16 + 4c + j - 4)
  float x[8];
  float mx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int pos = pb + (j < 4 ? 4 * c + j : 16 + 4 * c + j - 4);
    x[j] = pos <= lim ? st[j >> 2][j & 3] * scale_log2e : -__builtin_inff();
    mx = fmaxf(mx, x[j]);
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(st_.m, mx);
  const float ms = m_new == -__builtin_inff() ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(st_.m - ms);
  // the sum takes the probabilities as rounded for the value product, so
  // the output is an exact average of V under those weights
  h8_t pf;
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    pf[j] = (_Float16)__builtin_amdgcn_exp2f(x[j] - ms);
    ps += (float)pf[j];
  }
  st_.l = st_.l * alpha + ps;
  st_.m = m_new;
  // the accumulators need rescaling only in a step that raised some row's
  // maximum (alpha < 1); once the maxima settle, most steps skip it
  if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < kD / 16; db++) acc[db] *= alpha;
  }
  // O^T[dims 16 db ..][rows] += V^T[dims][this lane's 8 positions] P^T.
  // The A fragment (lane l: dim 16 db + l % 16 at positions 4c .. 4c + 3
  // and 16 + 4c .. 16 + 4c + 3) comes from V at [position][dim] through
  // ds_read_b64_tr_b16: in each 16-lane group, output lane i element j is
  // element i % 4 of the 8 bytes that lane 4j + i / 4 addresses, so lane s
  // of group c points at position 4c + s / 4, dims 16 db + 4 (s % 4).
  const int s_ = lane & 15;
  const _Float16* vsrc = vt + (4 * c + (s_ >> 2)) * kVRow + 4 * (s_ & 3);
#pragma unroll
  for (int db = 0; db < kD / 16; db++) {
    typedef short s4_t __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s4_t lds_s4;
    const s4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vsrc + 16 * db));
    const s4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(vsrc + 16 * kVRow + 16 * db));
    const u2_t l2 = __builtin_bit_cast(u2_t, lo), h2 = __builtin_bit_cast(u2_t, hi);
    const u4_t va = {l2.x, l2.y, h2.x, h2.y};
    acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, va), pf, acc[db], 0, 0, 0);
  }
}

template <bool kFp8>
__global__ void __launch_bounds__(kThreads) attn_partial(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBufBytes];
  const int si = blockIdx.z, ci = blockIdx.x, g = blockIdx.y;
  if (si >= a.nslots) return;
  const AttnSlot S = a.s[si];
  if (ci >= S.nchunks) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = kGroup * S.W;                  // query rows of this KV head
  const bool active = 16 * wave < R;
  const int c = lane >> 4;
  const int row = 16 * wave + (lane & 15);     // query row held by this lane
  const int rr = row < R ? row : R - 1;        // rows past R repeat the last (never written)
  const int w = rr / kGroup;
  const int lim = S.L - S.W + w;               // last position this row sees
  const int p0 = ci * a.chunk;
  const int pend = min(S.L, p0 + a.chunk);
  const int nblk = (pend - p0 + kBlk - 1) / kBlk;

  // this lane's query fragments: row rr, dims 32 s + 8 c .. + 7
  h8_t qf[kD / 32];
  {
    const _Float16* qrow = (const _Float16*)S.Q + ((size_t)w * kHq + kGroup * g + rr % kGroup) * kD;
#pragma unroll
    for (int s = 0; s < kD / 32; s++) qf[s] = *(const h8_t*)(qrow + 32 * s + 8 * c);
  }
  f4_t acc[kD / 16];
#pragma unroll
  for (int db = 0; db < kD / 16; db++) acc[db] = f4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff(), l_run = 0.f;

  // Steps alternate between two LDS buffers, so one barrier per step: step
  // b + 1 is stored into the other buffer while step b is computed (the
  // barrier ending step b - 1 freed it).  Loads run two steps ahead in two
  // register sets: the set just stored is reloaded with step b + 3.
  // E4M3 tiles leave registers for four score chains; fp16 tiles measured
  // no better with four than with two
  constexpr int kChainParts = kFp8 ? 2 : 1;
  Tile<kFp8> t0, t1;
  t0.load(S.K, S.V, g, p0, S.L, tid);
  if (nblk > 1) t1.load(S.K, S.V, g, p0 + kBlk, S.L, tid);
  t0.store(lds, tid);
  if (nblk > 2) t0.load(S.K, S.V, g, p0 + 2 * kBlk, S.L, tid);
  __syncthreads();
  Row r_state{m_run, l_run};
  for (int b = 0; b < nblk; b += 2) {
    // step b from buffer 0; step b + 1 into buffer 1
    if (b + 1 < nblk) {
      t1.store(lds + kBufBytes, tid);
      if (b + 3 < nblk) t1.load(S.K, S.V, g, p0 + (b + 3) * kBlk, S.L, tid);
    }
    if (active)
      step<kChainParts>(r_state, acc, qf, (const _Float16*)lds, (const _Float16*)(lds + kKBytes), p0 + b * kBlk, lim, lane,
           a.scale_log2e);
    __syncthreads();
    if (b + 1 >= nblk) break;
    // step b + 1 from buffer 1; step b + 2 into buffer 0
    if (b + 2 < nblk) {
      t0.store(lds, tid);
      if (b + 4 < nblk) t0.load(S.K, S.V, g, p0 + (b + 4) * kBlk, S.L, tid);
    }
    if (active)
      step<kChainParts>(r_state, acc, qf, (const _Float16*)(lds + kBufBytes), (const _Float16*)(lds + kBufBytes + kKBytes),
           p0 + (b + 1) * kBlk, lim, lane, a.scale_log2e);
    __syncthreads();
  }
  m_run = r_state.m;
  l_run = r_state.l;
  if (!active) return;
  // row sums over the four lanes of a row; the maximum is already common
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (row < R) {
    const size_t part = (size_t)S.part0 + (size_t)g * S.nchunks + ci;
    float* o = a.part_o + (part * kMaxRows + row) * kD + 4 * c;
#pragma unroll
    // non-temporal: the partials are read once, by the combine kernel
    // (one slot over 32768 positions: a layer about 0.7 us faster)
    for (int db = 0; db < kD / 16; db++) __builtin_nontemporal_store(acc[db], (f4_t*)(o + 16 * db));
    if (c == 0) {
      __builtin_nontemporal_store(m_run, a.part_ml + (part * kMaxRows + row) * 2);
      __builtin_nontemporal_store(l_tot, a.part_ml + (part * kMaxRows + row) * 2 + 1);
    }
  }
}

// Sum and maximum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// One workgroup per (query row, KV head, slot), one thread per dim: the
// row's chunks merged with weights exp2(m_c - max m), divided by the merged
// sum.  Chunk 0 always holds position 0, so the maximum is finite.  With
// more than kFewChunks chunks the chunks' maxima, weights and sums are
// handled by the threads together (thread t takes chunks t, t + kD, ...), the
// weights shared through LDS, so each thread loads only its dim's partials,
// kBatch of them at a time: the loads, not the arithmetic, bound this kernel
// (one slot over 32768 positions, 64 chunks: a layer 38.1 -> 36.1 us with
// binary16 caches, 37.8 -> 35.5 us with E4M3; with 8 chunks the barriers
// cost more than they save, and every thread walks the chunks).
__global__ void __launch_bounds__(kD) attn_combine(AttnArgs a) {
  constexpr int kBatch = 32;
  constexpr int kWaves = kD / 64;
  constexpr int kFewChunks = 16;
  __shared__ float wbuf[kD];
  __shared__ float red[kWaves];
  const int r = blockIdx.x, g = blockIdx.y, si = blockIdx.z, d = threadIdx.x;
  if (si >= a.nslots) return;
  const AttnSlot S = a.s[si];
  if (r >= kGroup * S.W) return;
  const size_t row0 = ((size_t)S.part0 + (size_t)g * S.nchunks) * kMaxRows + r;
  const float* ml = a.part_ml + row0 * 2;
  const float* po = a.part_o + row0 * kD + d;
  const size_t mstep = (size_t)kMaxRows * 2, ostep = (size_t)kMaxRows * kD;
  const int nc = S.nchunks;
  float* const out = S.O + ((size_t)(r / kGroup) * kHq + kGroup * g + r % kGroup) * kD + d;
  if (nc <= kFewChunks) {
    // few chunks: every thread walks them all (no barriers)
    float M = -__builtin_inff();
#pragma unroll 8
    for (int c = 0; c < nc; c++) M = fmaxf(M, ml[c * mstep]);
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int c = 0; c < nc; c++) {
      const float wgt = __builtin_amdgcn_exp2f(ml[c * mstep] - M);
      den += wgt * ml[c * mstep + 1];
      num += wgt * po[c * ostep];
    }
    *out = num / den;
    return;
  }
  float M = -__builtin_inff();
  for (int c = d; c < nc; c += kD) M = fmaxf(M, ml[c * mstep]);
  M = wave_max(M);
  if ((d & 63) == 0) red[d >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) M = fmaxf(M, red[w]);
  __syncthreads();
  float num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kD) {
    const int n = nc - c0 < kD ? nc - c0 : kD;
    if (d < n) {
      const float wgt = __builtin_amdgcn_exp2f(ml[(c0 + d) * mstep] - M);
      wbuf[d] = wgt;
      den += wgt * ml[(c0 + d) * mstep + 1];
    }
    __syncthreads();
    int c = 0;
    for (; c + kBatch <= n; c += kBatch) {
      float v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; i++) v[i] = po[(size_t)(c0 + c + i) * ostep];
#pragma unroll
      for (int i = 0; i < kBatch; i++) num += wbuf[c + i] * v[i];
    }
    for (; c < n; c++) num += wbuf[c] * po[(size_t)(c0 + c) * ostep];
    __syncthreads();
  }
  den = wave_sum(den);
  if ((d & 63) == 0) red[d >> 6] = den;
  __syncthreads();
  den = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; w++) den += red[w];
  *out = num / den;
}

hipError_t launch_attn(const AttnArgs& a, bool fp8, int max_chunks, hipStream_t stream) {
  const dim3 grid((unsigned)max_chunks, kHkv, (unsigned)a.nslots);
  if (fp8)
    hipLaunchKernelGGL(attn_partial<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_partial<false>, grid, dim3(kThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  hipLaunchKernelGGL(attn_combine, dim3(kMaxRows, kHkv, (unsigned)a.nslots), dim3(kD), 0, stream, a);
  return hipGetLastError();
}

}  // namespace qa
