/* Read ceiling of one sweep launch: a measurement kernel, not part of the
 * sweep (libqgemm_ceiling.so, built beside libqgemm.so).
 *
 * It loads what a stream-kernel launch of the sweep (qgemm.h) loads for
 * panels of up to 16 rows -- every weight tile's codes, scales and (5-bit)
 * high bits, and one X chunk per step -- with the sweep's geometry: `nwaves`
 * waves, four per workgroup, each taking an equal contiguous range of the
 * launch's weight units (9 per 4-bit step, 11 per 5-bit step), steps of four
 * 16-row blocks at one 128-wide k tile, two steps in flight per wave.  It
 * computes nothing from the data beyond an XOR fold, and writes one 32-bit
 * word per wave to `sink` (so the loads stay live).  The time of one launch
 * is the streaming time a sweep launch of these shapes cannot beat; a
 * measured stream ceiling is the basis the EXL3-K5K6 model card (multi-GPU
 * section) judges its GEMMs against, beside the part's rated bandwidth.
 *
 *   jobs   : host array of njobs (1 .. QGEMM_CEILING_MAX_JOBS) matrices, each
 *            packed as for the sweep (QG32 tiles, bits 4 or 5, K a multiple
 *            of 128), with an fp16 panel X of xrows rows, row stride ldx
 *   nwaves : waves in the grid (1 .. QGEMM_CEILING_MAX_WAVES); the launch
 *            must hold at least 11 units per wave
 *   xrows  : panel rows (1 .. 16); rows past it are read as its last row
 *   sink   : device uint32 [nwaves], written
 * Returns 0 when launched on `stream` (a hipStream_t), 1 on an argument
 * error (nothing launched), 2 on a launch error.  Asynchronous. */
#ifndef QGEMM_READ_CEILING_H
#define QGEMM_READ_CEILING_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QGEMM_CEILING_MAX_JOBS 4
#define QGEMM_CEILING_MAX_WAVES 4096

typedef struct {
  const void* packed;
  const void* X;
  int64_t N, K, ldx;
  int32_t bits;
} qgemm_ceiling_job;

int qgemm_read_ceiling(const qgemm_ceiling_job* jobs, int njobs, int nwaves, int xrows, uint32_t* sink,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif
