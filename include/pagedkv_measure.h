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

/*
 * Enqueues the reads a split decode (pa_decode's VALU kernel, one work-group of 4 waves per
 * (sequence, kv head)) makes of a paged cache, and nothing else: each work-group reads the
 * sequence's context_len (tokens 0 .. L-1), stages its block_table row, and reads every K and
 * V row of its kv head below L, a wave load being 1 KiB of consecutive rows of one block.
 * The address translation ([BlockManager essay] §2) and the scattered blocks are those of the
 * decode; the attention arithmetic, the queries and the outputs are left out. Timed with
 * events on `stream`, the K+V bytes below the lengths over the time give the rate this
 * cache layout and decomposition allow, a ceiling for the decode on the same cache.
 * Arguments are pa_decode's (one partition per sequence): cache describes both pools; k_pool
 * and v_pool are device memory, 16-byte aligned; block_table is int32 [batch][max_blocks_per_seq];
 * context_lens int32 [batch]; sink is device memory of batch x num_kv_heads floats (written
 * only with negligible probability, to keep the loads alive). A sequence with a length
 * outside [1, max_context_len] or more than max_blocks_per_seq (or 4096) blocks is skipped;
 * ids outside the pool are not read. 8-bit pools: the codes only. Returns
 * PA_ERR_INVALID_ARGUMENT for null or misaligned pointers and bad sizes, PA_ERR_UNSUPPORTED
 * for a cache whose rows exceed 1 KiB or whose blocks hold less than 1 KiB per kv head
 * (or a cache pa_decode rejects), PA_ERR_LAUNCH if the launch fails. Allocates nothing
 * and does not synchronise.
 */
pa_status_t pa_measure_gather_read(const pa_cache_desc_t* cache, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                                   float* sink, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_MEASURE_H */
