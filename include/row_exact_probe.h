/*
 * row_exact_probe.h — measurement aid shipped with librow_exact_mv.so.
 *
 * Not part of the mat-vec itself.  A weight-streaming kernel cannot read HBM
 * faster than a kernel that does nothing but read, so the benchmark times
 * this plain read of the same number of bytes as the attainable read rate
 * for that size on the current device, next to the 8 TB/s HBM3E peak.
 */
#ifndef ROW_EXACT_PROBE_H
#define ROW_EXACT_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of launch shapes row_exact_stream_read accepts (shape 0 .. count-1). */
uint32_t row_exact_stream_read_shapes(void);

/* Enqueue one kernel that reads bytes [0, bytes) of the device buffer p with
 * 16-byte loads (lane L of a wave reads 16-byte chunk L of each 1 KiB the wave
 * visits) and folds them into a value it writes to *sink only in the
 * impossible-looking case that the fold equals a fixed constant (the write
 * keeps the loads alive).
 *  p     : device pointer, 16-byte aligned, caller-owned, only read.
 *  bytes : a multiple of 16, >= 16.
 *  sink  : device pointer to 4 writable bytes.
 *  shape : 0 .. row_exact_stream_read_shapes()-1, a (workgroups, loads in
 *          flight per lane) pair; the benchmark keeps the fastest.
 * Returns 0, ROW_EXACT_EARG (-1), ROW_EXACT_EALIGN (-2) or ROW_EXACT_EHIP
 * (-7); row_exact_last_error() describes a failure. */
int row_exact_stream_read(const void *p, uint64_t bytes, uint32_t *sink, uint32_t shape, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROW_EXACT_PROBE_H */
