/*
 * i8gs_peaks.h -- achievable-peak microbenchmarks for MI355X (gfx950), used by the
 * benchmark to report measured ceilings beside the vendor ones (HBM 8 TB/s, dense INT8
 * MFMA 5.0 POP/s).  Not part of the linear layer's ABI (include/i8gs.h).
 *
 * Both calls enqueue one kernel on `stream` (a hipStream_t) and return 0, 1 for
 * invalid arguments (nothing launched) or 5 if the launch failed.  Buffers are device
 * memory owned by the caller; sink must hold blocks * 256 ints.
 */
#ifndef I8GS_PEAKS_H
#define I8GS_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (a multiple of 16) of the 16-byte aligned device buffer src with
 * `blocks` workgroups of 256 threads (16-byte non-temporal loads, grid-stride), each
 * thread writing one fold of what it read to sink.  Bandwidth = bytes / kernel time. */
int i8gs_peak_stream_read(const void *src, size_t bytes, int *sink, int blocks, void *stream);

/* `blocks` workgroups of four waves, each wave issuing iters * 4 independent
 * v_mfma_i32_32x32x32_i8 (65536 ops each) on register operands.  Ops = blocks * 4 *
 * iters * 4 * 65536. */
int i8gs_peak_mfma_i8(int iters, int *sink, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* I8GS_PEAKS_H */
