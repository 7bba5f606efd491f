/*
 * pa_measure.h — HBM read ceilings (measurement only; not part of the attention path).
 *
 * The benchmark compares the decode kernels with what the device's HBM delivers for a
 * plain read: a contiguous stream (the best case) and a replay of the exact list of K/V
 * tiles a decode batch reads, with no attention arithmetic (the attainable rate of that
 * access pattern).  Both kernels only read; every loaded byte is folded into a value that
 * is stored to `sink` (one uint32 per workgroup) only in a case that practically never
 * happens, so no load can be dropped.  Device pointers, caller-owned memory, enqueued on
 * `stream`; errors as in pa.h.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Reads bytes (a multiple of 16) of buf, 16 KiB per wave at a time.  sink: one uint32 per
 * workgroup; workgroups of 256 threads, 0: two per CU. */
pa_status pa_measure_stream_read(const void* buf, size_t bytes, uint32_t* sink,
                                 int32_t workgroups, void* stream);

/* Reads num_tiles tiles of tile_bytes (a multiple of 1024) at base + tile_offsets[t] (int64
 * byte offsets, 16-byte aligned), the list split evenly over the waves of the grid in its
 * order, eight tiles in flight per wave.  sink: one uint32 per workgroup; workgroups of 256
 * threads, 0: two per CU. */
pa_status pa_measure_tile_read(const void* base, const int64_t* tile_offsets, int64_t num_tiles,
                               int32_t tile_bytes, uint32_t* sink, int32_t workgroups,
                               void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_MEASURE_H */
