/*
 * qgemm -- fused quantized weight sweep for MI355X (gfx950).
 *
 * One decode step of a self-speculative decoder streams every quantized linear
 * weight once and multiplies it against a skinny activation panel of
 * M = slots x (1 + draft tokens) rows, so a single weight read verifies
 * several tokens (Quasar/q27 wiki: "decode physics" paragraph -- decode is
 * weight-read bound and each accepted position per weight read is the lever;
 * intro bullets -- concurrent slots share one fused weight sweep).  The
 * weights are 4- or 5-bit symmetric group-wise codes with one fp16 scale per
 * group, dequantized inside the product (Quasar wiki, engine-internals list,
 * "Weights" item; group size 32 here).
 *
 * This header is the whole boundary: plain C, device pointers and sizes.
 * The library allocates nothing that outlives a call; every buffer belongs to
 * the caller.  Its only global state is two small thread-safe caches of values
 * that depend on shapes and the device alone (kernel occupancy, and the wave
 * count chosen for a set of matrix shapes).
 *
 * ---------------------------------------------------------------------------
 * Quantizer (qgemm_pack).  W is logical [N][K] (N outputs, K inputs,
 * Y = X * W^T).  For every row n and group g of 32 consecutive k:
 *     amax = max |W[n,k]|                   (fp32)
 *     s    = fp16_RNE((double)amax / Qmax)  Qmax = 7 (4-bit) or 15 (5-bit)
 *     q    = 0 if s == 0, else clamp(RNE((double)W[n,k] / (double)s), +-Qmax)
 *     u    = q + 2^(bits-1)                 (stored offset-binary code)
 *
 * Packed layout "QG32 tiled v1".  Tiles of 16 rows x 128 k; tile (rb, kt) is
 * at byte (rb * NKT + kt) * TB, NKT = ceil(K/128), TB = 1152 (4-bit) or 1408
 * (5-bit).  For element (n, k) let r = n mod 16, j = (k mod 128) / 32,
 * c = (k mod 32) / 8, e = k mod 8:
 *     low 4 bits of u  -> little-endian 32-bit word at byte 16*(r + 16c) + 4j,
 *                         bit 4*(e >> 1) + 16*(e & 1)
 *     bit 4 of u       -> 32-bit word at byte 1152 + 4*(r + 16c),
 *                         bit (4 + 16*(e & 1) + 4*(e >> 1) + j) mod 32 (5-bit)
 *     s(n, 4kt + j)    -> IEEE binary16 at byte 1024 + 8r + 2j
 * Rows n >= N and groups beyond K/32 are padding (u = 2^(bits-1), s = +0).
 * Lane l = r + 16c of a 64-wide wave thus reads the 16 bytes at 16*l: chunk c
 * (8 consecutive k) of the four groups of row r, already in fp16-pair order.
 * Size: qgemm_packed_bytes(); 4.5 (4-bit) / 5.5 (5-bit) bits per weight.
 *
 * Format variants.  Wherever an argument or field is called `bits` it takes a
 * format code: 4 and 5 are the formats above; the variants keep the tile grid
 * and the code words and change the scale group or add zero points.
 *   QGEMM_FMT_Q4_G64: 4-bit symmetric, one scale per 64 weights (Quasar/q27
 *     wiki, "Batching & prefill notes": the group-64 format of 4.25 bits per
 *     weight).  Same quantizer with the amax over 64 consecutive k; K % 64 ==
 *     0.  Tiles of 1088 bytes: the codes, then s(n, 2kt + h) (h = (k mod 128)
 *     / 64) as binary16 at byte 1024 + 4r + 2h.  4.25 bits per weight.
 *   QGEMM_FMT_Q4_ZP: 4-bit group-32 asymmetric with a 4-bit zero point per
 *     group (the INT4 W4A16 group-32 asymmetric weights of the qwen38 model
 *     notes, "Path 1 -- vLLM" section).  Per row n and group g:
 *       lo = min(0, min W), hi = max(0, max W)        (fp32)
 *       s  = fp16_RNE(((double)hi - (double)lo) / 15)
 *       z  = 0 if s == 0, else clamp(RNE(-(double)lo / s), 0, 15)
 *       u  = z if s == 0, else clamp(RNE((double)W / s) + z, 0, 15)
 *     and W is taken as (u - z) * s.  u is stored in the code words (no
 *     offset), s at 1024 + 8r + 2j, and z of group j of row r in bits 4j ..
 *     4j + 3 of the little-endian 16-bit word at byte 1152 + 2r; tiles of
 *     1184 bytes (4.625 bits per weight).  Padding: u = 0, z = 0, s = +0.
 *
 * ---------------------------------------------------------------------------
 * Sweep (qgemm_sweep).  For each job: Y[m][n] = sum_k X[m][k] * q[n][k] *
 * s[n][k/32] for m < M, n < N.  X is fp16 (binary16 bits), Y is fp32 and is
 * overwritten.  Products q*x are exact in fp32 and every group's partial sum
 * is scaled by its fp32 scale; the result is within relative L2 1e-4 of the
 * exact product and, per row m, within 1e-3 * ||X[m,:]||_2 * max(s) of it.
 * Row m of Y depends only on row m of X and the matrices: for the same set of
 * matrices in a sweep it is bitwise the same for any other rows and any M of
 * one panel class -- GEMV M <= 8; MFMA M <= 16; MFMA 17 <= M <= 64 -- and
 * within the tolerance above across classes.  Repeated calls are bitwise equal.
 * A non-finite X entry makes its row's outputs non-finite (Inf or NaN is not
 * specified).  A sweep whose work exceeds the kernels' 32-bit ranges (about
 * 2^31 / 9 k tiles of 16-row blocks per launch) returns QGEMM_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------------
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QGEMM_OK = 0,
  QGEMM_ERR_INVALID_ARG = 1,  /* an argument fails the rules below; nothing enqueued */
  QGEMM_ERR_UNSUPPORTED = 2,  /* valid arguments the library cannot run (e.g. path) */
  QGEMM_ERR_NONFINITE = 3,    /* pack: NaN/Inf weight or a scale that overflows fp16 */
  QGEMM_ERR_HIP = 4           /* a HIP runtime call or launch failed */
} qgemm_status;

/* Which contraction a sweep uses.  AUTO takes MFMA at every M: on gfx950 it
 * is as fast as GEMV at M = 1 and faster above, and it keeps an M = 1 row
 * bitwise equal to the same row in any panel of up to 16 rows.  GEMV (per-lane
 * dot products) accepts M <= QGEMM_GEMV_MAX_M; MFMA accepts any M. */
typedef enum {
  QGEMM_PATH_AUTO = 0,
  QGEMM_PATH_GEMV = 1,
  QGEMM_PATH_MFMA = 2
} qgemm_path;

#define QGEMM_MAX_M 64
#define QGEMM_GEMV_MAX_M 8

/* Weight format codes (the `bits` argument and field). */
#define QGEMM_FMT_Q4 4
#define QGEMM_FMT_Q5 5
#define QGEMM_FMT_Q4_G64 0x104
#define QGEMM_FMT_Q4_ZP 0x204

/* One matrix of a sweep.  Pointers are device pointers.
 *   packed : tiled buffer from qgemm_pack, 256-byte aligned, read-only
 *   bits   : the format code it was packed with (QGEMM_FMT_*)
 *   N, K   : 1 <= N <= 2^30; 32 <= K <= 2^24 and K % 32 == 0 (64 for
 *            QGEMM_FMT_Q4_G64)
 *   X      : binary16 [M][ldx], 16-byte aligned, ldx % 8 == 0, K <= ldx <= 2^24
 *   Y      : fp32 [M][ldy], 16-byte aligned, ldy % 4 == 0, ldy >= N
 *   M      : 1 .. QGEMM_MAX_M
 * Y must not overlap any job's X, any packed buffer or another job's Y
 * (checked: QGEMM_ERR_INVALID_ARG); inputs may be shared between jobs. */
typedef struct {
  const void* packed;
  const uint16_t* X;
  float* Y;
  int64_t N;
  int64_t K;
  int64_t ldx;
  int64_t ldy;
  int32_t M;
  int32_t bits;
} qgemm_job;

/* Bytes of the packed buffer for an N x K matrix; 0 when the shape or bits
 * are invalid. */
size_t qgemm_packed_bytes(int bits, int64_t N, int64_t K);

/* Quantize and pack W (fp32 device buffer, row stride ldw >= K floats) into
 * `packed` (qgemm_packed_bytes() bytes, 256-byte aligned), padding included.
 * Enqueued on `stream` (a hipStream_t; NULL = default stream), then the call
 * synchronizes that stream once to report QGEMM_ERR_NONFINITE (the packed
 * contents are then unspecified).  Packing is an offline step: it may allocate
 * and free a 4-byte device flag inside the call. */
qgemm_status qgemm_pack(const float* W, int64_t ldw, int64_t N, int64_t K, int bits,
                        void* packed, void* stream);

/* Workspace bytes the sweep of these jobs on this path needs (a device buffer
 * the caller owns, 256-byte aligned); 0 when the jobs are invalid.  It holds
 * the job tables (launches of more than 12 jobs) and the split-K partial-sum
 * slots.  The buffer must be zero-filled before its first use (for instance
 * with qgemm_workspace_init); every completed sweep leaves its slots at zero
 * again, so the same set of jobs (same shapes and path) may sweep on it any
 * number of times.  Its layout depends on those shapes: before a
 * different set of jobs uses a workspace, zero-fill it again (or keep one
 * workspace per set of jobs, or record the sweeps as a round, below, whose
 * layout serves all of them).  A workspace serves one sweep at a time: sweeps
 * that overlap on one workspace race. */
size_t qgemm_workspace_bytes(const qgemm_job* jobs, int njobs, int path);

/* Zero-fill `ws_bytes` (a multiple of 4) of a workspace with a fill kernel on
 * `stream` (no memset node, so it may be captured in a graph). */
qgemm_status qgemm_workspace_init(void* workspace, size_t ws_bytes, void* stream);

/* Y = X * W^T for every job on `stream`: one kernel launch per kernel class
 * (jobs of equal panel height share one launch).  Asynchronous: argument
 * errors return before anything is enqueued; launch failures return
 * QGEMM_ERR_HIP; device faults surface at the caller's next synchronization.
 * The `jobs` array is host memory read during the call. */
qgemm_status qgemm_sweep(const qgemm_job* jobs, int njobs, void* workspace, size_t ws_bytes,
                         void* stream);

/* As qgemm_sweep with an explicit path (qgemm_path).  GEMV with any job's
 * M > QGEMM_GEMV_MAX_M is QGEMM_ERR_INVALID_ARG. */
qgemm_status qgemm_sweep_path(const qgemm_job* jobs, int njobs, int path, void* workspace,
                              size_t ws_bytes, void* stream);

/* Allocation-free sweep, for callers that cannot allocate device memory
 * (code that must not call hipMalloc: tight serving loops, harnesses that
 * forbid it).  As qgemm_sweep_path, with the library's own scratch in place of
 * the caller's workspace: one static device array of
 * QGEMM_NOALLOC_SCRATCH_BYTES, which every GPU the library runs on holds until
 * the process ends.  A job set whose qgemm_workspace_bytes exceeds that size
 * is QGEMM_ERR_INVALID_ARG, as are the argument errors of qgemm_sweep_path.
 * The call allocates no device memory; on `stream` it enqueues, in order: a
 * fill kernel when the scratch region this sweep's split-K slots need may
 * hold bytes an earlier call's job table left there, one copy per launch of
 * more than 12 jobs (its job table, from host memory read during the call),
 * and the sweep's launches.  Every call on one GPU shares that GPU's scratch:
 * calls that overlap on one GPU (unordered streams or threads) race.  The
 * outputs are bitwise those of qgemm_sweep_path for the same jobs and path. */
#define QGEMM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

qgemm_status qgemm_sweep_noalloc(const qgemm_job* jobs, int njobs, int path, void* stream);

/* ---------------------------------------------------------------------------
 * Verify head (greedy acceptance).  In a self-speculative decode round the
 * panel holds, per slot, the hidden states after the accepted context and
 * after each of its d drafted tokens (1 + d rows).  Greedy speculative
 * decoding must leave the greedy output unchanged (Quasar/q27 wiki, opening
 * notes: greedy spec decode by default, greedy output bitwise unchanged), so
 * draft i + 1 stands only if it equals the model's argmax at row i, and the
 * round yields the longest such prefix plus the argmax at the first row that
 * disagrees.  The per-round payoff is the accepted count per weight read
 * (same page, intro bullets).  The head is the lm_head-class matrix
 * (vocabulary rows N).  One call sweeps it with a per-row argmax epilogue
 * (the logits are reduced in the kernel, not written unless Y is given) and
 * then scores every slot.
 *
 *   head     : one job as for qgemm_sweep; head->Y may be NULL (no logits
 *              written) or a logits buffer obeying the sweep's rules
 *   drafts   : device int32 [M]; drafts[r] is the draft token that row r's
 *              argmax is checked against (unused for each slot's last row);
 *              may be NULL when no slot has drafts
 *   slots    : host array of nslots (1 .. 64) slots: rows row0 .. row0 + ndraft
 *              of the panel, ndraft >= 0, row0 + ndraft < M
 *   argmax   : device int32 [M]: per row, the column of the largest logit,
 *              the lowest column among equal values
 *   maxlogit : device fp32 [M] (may be NULL): that largest logit
 *   accepted : device int32 [nslots]: per slot, the number L of leading rows
 *              i < ndraft with argmax[row0 + i] == drafts[row0 + i]; the round
 *              emits drafts[row0 .. row0 + L - 1] and then argmax[row0 + L]
 * The logits (and so the argmax) are exactly those qgemm_sweep computes for
 * the same job.  Rows whose X is not finite get an unspecified column in
 * 0 .. N - 1.  The workspace (qgemm_verify_workspace_bytes, zero-filled
 * before first use like a sweep's) ends with the argmax keys, which the call leaves at
 * zero.  Two kernel launches on `stream`; asynchronous like qgemm_sweep. */
typedef struct {
  int32_t row0;
  int32_t ndraft;
} qgemm_slot;

size_t qgemm_verify_workspace_bytes(const qgemm_job* head);

qgemm_status qgemm_verify_head(const qgemm_job* head, const int32_t* drafts, const qgemm_slot* slots, int nslots,
                               int32_t* argmax, float* maxlogit, int32_t* accepted, void* workspace,
                               size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Round replay.  A decode round issues the same launches every step -- the
 * weight sweeps in dependency order (one per layer's matrix group, say), then
 * the verify head -- on the same buffers, and the host cost of issuing them
 * one call at a time adds up (Quasar/q27 wiki: "decode physics" paragraph, a
 * residual tail of about 140 launches per token; intro bullets, whole
 * fused-verify rounds replayed as shape-keyed graphs).  qgemm_round_create
 * records one round as a HIP graph; qgemm_round_launch replays it on any
 * stream with one call.  The graph holds kernel launches only (no copies or
 * memsets): job tables are uploaded into the workspace at creation.
 *
 *   sweeps    : host array of nsweeps (>= 0) sweeps, recorded in order; each
 *               as qgemm_sweep_path would run it (its jobs and path)
 *   head...   : an optional verify head (NULL: none, and then nsweeps >= 1) with
 *               the arguments of qgemm_verify_head, recorded last
 *   workspace : qgemm_round_workspace_bytes() bytes, 256-byte aligned,
 *               zero-filled before creation; it holds the tables of every
 *               sweep and one scratch region the sweeps share (they run in
 *               order) and must stay untouched while the round exists
 *   stream    : the tables are copied on it and it is synchronized once;
 *               recording itself uses a stream of the library's own
 *   out       : the new round (NULL on error)
 * Pointers and shapes are fixed at creation; buffer contents are read when
 * the round runs, so a caller refills X (and drafts) and replays.  The caller
 * keys rounds by shape and pointers and keeps as many as it likes.  Replays
 * on one workspace must not overlap.  Creation validates everything first
 * (QGEMM_ERR_INVALID_ARG before any HIP call) and may allocate host memory
 * and a HIP graph, freed by qgemm_round_destroy. */
typedef struct qgemm_round_s qgemm_round;

typedef struct {
  const qgemm_job* jobs;  /* host array of njobs jobs, read during creation only */
  int32_t njobs;
  int32_t path;           /* qgemm_path */
} qgemm_round_sweep;

size_t qgemm_round_workspace_bytes(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head);

qgemm_status qgemm_round_create(const qgemm_round_sweep* sweeps, int nsweeps, const qgemm_job* head,
                                const int32_t* drafts, const qgemm_slot* slots, int nslots, int32_t* argmax,
                                float* maxlogit, int32_t* accepted, void* workspace, size_t ws_bytes,
                                void* stream, qgemm_round** out);

/* Replay the round on `stream` (asynchronous, one graph launch). */
qgemm_status qgemm_round_launch(const qgemm_round* round, void* stream);

/* Kernel launches one replay makes (0 for NULL). */
int qgemm_round_kernels(const qgemm_round* round);

/* Free the round (NULL is a no-op).  Synchronize the streams of its replays
 * first. */
void qgemm_round_destroy(qgemm_round* round);

/* ---------------------------------------------------------------------------
 * Round cache.  Rounds keyed by everything a recording fixes, replayed on a
 * hit and recorded on a miss, least recently used evicted past the capacity
 * (Quasar/q27 wiki: intro bullets, fused-verify rounds replayed as
 * shape-keyed graphs; defaults paragraph, a graph-cache cap of 64; open
 * items, "graph-cache cap under churn", live traffic drawing 44+ keys).  A
 * key is the whole argument list of qgemm_round_create but the workspace:
 * every sweep's path and jobs (pointers, shapes, strides, M, bits), the
 * head's job, draft and output pointers and the slots' contents.  Buffers
 * that a caller allocates once per shape therefore give one key per shape.
 * The cache owns one workspace per round (device memory it allocates,
 * zero-fills on the caller's stream and frees on eviction).
 *
 *   capacity : rounds kept, 1 .. QGEMM_ROUND_CACHE_MAX
 *   hit      : set to 1 when the call replayed a cached round, 0 when it
 *              recorded one (or failed)
 * qgemm_round_cache_run validates a miss as qgemm_round_create does; an
 * eviction synchronizes the device (a replay of the evicted round may still
 * run), so a capacity that covers the live keys keeps the replay path free
 * of synchronization.  Calls on one cache are serialized (it is
 * thread-safe); replays share each round's workspace, so two replays of the
 * same round must not overlap (one stream per cache, as a decode loop has).
 * Destroy only after the streams of its replays are synchronized. */
#define QGEMM_ROUND_CACHE_MAX 4096
typedef struct qgemm_round_cache_s qgemm_round_cache;

qgemm_status qgemm_round_cache_create(int capacity, qgemm_round_cache** out);

qgemm_status qgemm_round_cache_run(qgemm_round_cache* cache, const qgemm_round_sweep* sweeps, int nsweeps,
                                   const qgemm_job* head, const int32_t* drafts, const qgemm_slot* slots,
                                   int nslots, int32_t* argmax, float* maxlogit, int32_t* accepted,
                                   void* stream, int* hit);

/* Rounds held, and the calls that hit, missed and evicted so far (any
 * pointer may be NULL). */
qgemm_status qgemm_round_cache_stats(const qgemm_round_cache* cache, int* size, uint64_t* hits, uint64_t* misses,
                                     uint64_t* evictions);

/* Free every round and workspace (NULL is a no-op).  When the cache holds
 * rounds it first synchronizes the device, since replays of them may still
 * run on any stream; a call must not overlap a qgemm_round_cache_run on the
 * same cache. */
void qgemm_round_cache_destroy(qgemm_round_cache* cache);

/* ---------------------------------------------------------------------------
 * Attention verify (shared KV).  The attention half of a verify round, per
 * full-attention layer: each slot's W verify positions (the accepted token
 * and its drafts, whose keys and values are already the last W of the slot's
 * L cached positions) attend causally over the slot's cache.  Query w sits
 * at position L - W + w and sees positions 0 .. L - W + w:
 *     O[w][h] = sum_j softmax_j(scale * Q[w][h] . K[j][h / 6]) V[j][h / 6]
 * Geometry of the Quasar/q27 wiki's full-attention layers: 4 KV heads of
 * head_dim 256 (long-context note on KV bytes per token) and 6 query heads
 * per KV head (fp8-KV note, GQA 6), so 24 query heads.  All W * 6 queries of
 * a KV head read its keys and values once (wiki intro bullets: one shared-KV
 * verify).  The cache is binary16, or OCP E4M3 bytes with no scale (the
 * wiki's KV-cache item: scale-free saturating fp8); E4M3 values are exact in
 * binary16 and the product runs in binary16 MFMA with fp32 accumulation.
 * Result: within relative L2 1e-3 of the exact attention over a slot's O and
 * max |O - exact| <= 2e-3 * max |V| (probabilities enter the value product
 * rounded to binary16).
 *
 *   Q     : binary16 [W][24][256], 16-byte aligned
 *   K, V  : [L][4][256] elements (binary16, or one E4M3 byte each), 16-byte
 *           aligned; NaN codes give unspecified outputs
 *   O     : fp32 [W][24][256], 16-byte aligned, overwritten; must not overlap
 *           Q, K, V or another slot's O
 *   W     : 1 .. QGEMM_ATTN_MAX_W;  L: W .. 2^24
 * Slots are independent; nslots 1 .. QGEMM_ATTN_MAX_SLOTS per call.  Two
 * launches on `stream`: chunks of positions in parallel, then their merge.
 * The workspace (qgemm_attn_workspace_bytes, 256-byte aligned, any contents)
 * holds the per-chunk partials; calls that overlap on one workspace race. */
#define QGEMM_KV_FP16 0
#define QGEMM_KV_FP8 1
#define QGEMM_ATTN_HKV 4
#define QGEMM_ATTN_GROUP 6
#define QGEMM_ATTN_D 256
#define QGEMM_ATTN_MAX_W 16
#define QGEMM_ATTN_MAX_SLOTS 16

typedef struct {
  const uint16_t* Q;
  const void* K;
  const void* V;
  float* O;
  int32_t L;
  int32_t W;
} qgemm_attn_slot;

size_t qgemm_attn_workspace_bytes(const qgemm_attn_slot* slots, int nslots, int kv);

qgemm_status qgemm_attn_verify(const qgemm_attn_slot* slots, int nslots, int kv, float scale, void* workspace,
                               size_t ws_bytes, void* stream);

/* The argument checks of qgemm_sweep_path alone (host only, no HIP call). */
qgemm_status qgemm_validate(const qgemm_job* jobs, int njobs, int path, void* workspace,
                            size_t ws_bytes);

/* The path AUTO takes for panel height M (QGEMM_PATH_GEMV or _MFMA), or -1. */
int qgemm_auto_path(int M);

/* Static description of a status code. */
const char* qgemm_status_string(qgemm_status s);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
