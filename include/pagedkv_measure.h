/*
 * pagedkv_measure.h - measurement aid exported by libpagedkv (not part of the attention path).
 *
 * The pages report HBM read utilisation as a share of what the hardware can stream
 * ([BlockManager essay] §3: 78% at block size 16, 41% at 64). A share of the nominal peak
 * alone hides how much of it a read kernel can reach at all, so the library also measures
 * the achievable streaming-read rate on the device it runs on, with the access pattern of
 * the decode kernels.
 */
#ifndef PAGEDKV_MEASURE_H
#define PAGEDKV_MEASURE_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Enqueues one read of `bytes` bytes at `buf` (device memory, 16-byte aligned, bytes a
 * multiple of 16) with 16-byte non-temporal loads, 1 KiB per wave instruction and 8 loads in
 * flight per lane, on `num_workgroups` work-groups of 256 threads (8 per compute unit is the
 * usual choice). Nothing is written except, with negligible probability, one float per
 * work-group to `sink` (device memory of num_workgroups floats, caller-owned), which keeps the
 * loads from being optimised away. Time it with events on `stream`: bytes / time is the
 * streaming-read rate. Returns PA_ERR_INVALID_ARGUMENT for a null or misaligned pointer, a
 * size that is 0 or not a multiple of 16, or num_workgroups outside [1, 2^20];
 * PA_ERR_LAUNCH if the launch fails. Allocates nothing and does not synchronise.
 */
pa_status_t pa_measure_stream_read(const void* buf, size_t bytes, float* sink, int32_t num_workgroups,
                                   pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_MEASURE_H */
