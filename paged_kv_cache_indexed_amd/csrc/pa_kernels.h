// Internal interface between the C-ABI layer (pa_api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pagedkv.h"
#include "pa_device.h"

namespace pagedkv {

// Largest number of block-table entries one decode partition stages in LDS.
constexpr int kMaxIdsPerPartition = 1024;
// Beam groups: table entries staged per partition for all beams of a group together.
constexpr int kMaxBeamIds = 2048;
// Partition slots of one decode launch (the grid's z extent).
constexpr int kMaxPartitionSlots = 65535;

struct DecodeArgs {
    void* out;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const float* k_scale;  // 8-bit pools only: [num_blocks][num_kv_heads][block_size]
    const float* v_scale;
    const int32_t* block_table;
    const int32_t* context_lens;
    float* ws_o;   // [batch][num_q_heads][max_partitions][head_dim]
    float* ws_ml;  // [batch][num_q_heads][max_partitions][2] = (base-2 max, sum)
    int32_t* err_flag;
    int32_t num_blocks;
    int32_t log2_block_size;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t partition_size;
    int32_t max_partitions;
    int32_t window;    // > 0: attend to the last `window` tokens only; 0: the whole context
    float scale_log2;  // scale * log2(e): scores live in the base-2 exponent domain
    int64_t block_stride;  // bytes from one physical block to the next in k_pool / v_pool
    // multi-token attention only: query rows query_start[b] .. query_start[b+1]-1 belong to
    // sequence b; each workgroup covers one of col_tiles tiles of 16 (query, head) columns
    // fused append (pa_decode_append): the new token of sequence b, rows new_key/new_value
    // [batch][num_kv_heads][head_dim], goes to slot_mapping[b] before the decode reads it
    const void* new_key;
    const void* new_value;
    const int32_t* slot_mapping;
    // fused append with a reduce pass: the decode records sequence b's checked slot here (-1:
    // none) and the reduce kernel writes the rows, after every read of the pool
    int32_t* ws_slot;
    const int32_t* query_start;
    int32_t col_tiles;
    int32_t batch;
    int32_t num_q_tokens;  // rows of q and out
    // beam groups (pa_decode_beams): sequences g * beam_width .. + beam_width - 1 form group g,
    // whose blocks a workgroup reads once for all its beams where their tables agree
    int32_t beam_width;
};

struct CacheArgs {
    void* k_pool;
    void* v_pool;
    int32_t* err_flag;
    int32_t num_blocks;
    int32_t log2_block_size;
    int32_t num_kv_heads;
    int32_t row_vecs;      // 16-byte vectors per [head_dim] row
    int64_t block_stride;  // bytes from one physical block to the next in k_pool / v_pool
};

// VALU decode (every dtype and group size). kv_dtype is the pool's element type, dtype the
// type of q and out (equal unless the pool holds 8-bit floats).
hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream);
// The same over 8-bit float pools (dtype = type of q and out: fp16 or bf16; group <= 8).
hipError_t launch_decode_valu_fp8(const DecodeArgs& a, int dtype, int head_dim, int group, int batch,
                                  int num_kv_heads, hipStream_t stream);
// Matrix-core decode for grouped-query heads (fp16/bf16 or 8-bit pools, group 4/8/16,
// block_size >= 16, or 8 with head_dim <= 128); dtype is the type of q and out.
bool decode_mfma_supported(int kv_dtype, int head_dim, int group, int block_size);
hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream);
// 8-token blocks (head_dim 64 or 128): the same kernel with a block lookup per row.
hipError_t launch_decode_mfma_small_blocks(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group,
                                           int batch, int num_kv_heads, hipStream_t stream);
// Beam-group decode on the matrix cores (16-bit or 8-bit pools, head_dim 64/128, group 1-8,
// block_size >= 16 or 8, beam_width * group <= 16); `groups` = ceil(batch / beam_width).
bool decode_beams_supported(int kv_dtype, int head_dim, int group, int block_size, int beam_width);
hipError_t launch_decode_beams(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int groups,
                               int num_kv_heads, hipStream_t stream);
// 8-token blocks: the beam-group kernel with a block lookup per row.
hipError_t launch_decode_beams_small_blocks(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group,
                                            int groups, int num_kv_heads, hipStream_t stream);
// Multi-token attention on the matrix cores (16-bit or 8-bit pools, any group, block_size
// >= 16, or 8 up to head_dim 128) and its log-sum-exp combine per query row.
bool multi_token_supported(int kv_dtype, int head_dim, int group, int block_size);
hipError_t launch_multi_token(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream);
// 8-token blocks (head_dim 64 or 128): the 16-column kernel with a block lookup per row.
hipError_t launch_multi_token_small_blocks(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group,
                                           int batch, int num_kv_heads, hipStream_t stream);
hipError_t launch_reduce_multi(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
// Log-sum-exp combine of partition records (only when some sequence has > 1 partition).
hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_dim, int batch, hipStream_t stream);

hipError_t launch_reshape_and_cache(const CacheArgs& a, const void* key, const void* value,
                                    const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream);

// Copy-on-write. With 8-bit pools, k_scale/v_scale (non-null) are copied along with the codes.
hipError_t launch_copy_blocks(const CacheArgs& a, const int32_t* pairs, int32_t num_pairs, float* k_scale,
                              float* v_scale, hipStream_t stream);

// Re-blocking: every valid (token, kv head) row moves from the source layout to the
// destination layout (block size, stride and pool may differ; heads, dims and dtype agree).
struct ReblockArgs {
    const char* src_k;
    const char* src_v;
    const float* src_ks;  // 8-bit pools only
    const float* src_vs;
    const int32_t* src_table;
    char* dst_k;
    char* dst_v;
    float* dst_ks;
    float* dst_vs;
    const int32_t* dst_table;
    const int32_t* context_lens;
    int32_t* err_flag;
    int64_t src_stride;  // bytes between blocks
    int64_t dst_stride;
    int32_t src_num_blocks;
    int32_t dst_num_blocks;
    int32_t src_log2_bs;
    int32_t dst_log2_bs;
    int32_t src_mbs;  // table widths
    int32_t dst_mbs;
    int32_t num_kv_heads;
    int32_t row_vecs;  // 16-byte vectors per row
    int32_t max_context_len;
};
hipError_t launch_reblock(const ReblockArgs& a, int batch, hipStream_t stream);

// Measurement: the decode's K/V reads alone (pa_measure_gather_read): 4 waves per (kv head,
// sequence) read every token row of K and V below the length through the staged table, with
// the split decode's 1 KiB wave loads, and compute nothing.
struct GatherReadArgs {
    const char* k_pool;
    const char* v_pool;
    const int32_t* block_table;
    const int32_t* context_lens;
    float* sink;           // one float per work-group, written with negligible probability
    int64_t block_stride;  // bytes from one physical block to the next
    int32_t num_blocks;
    int32_t max_blocks_per_seq;
    int32_t max_context_len;
    int32_t log2_block_size;
    int32_t row_bytes;  // head_dim x element bytes: 64 .. 1024, a power of two
};
hipError_t launch_gather_read(const GatherReadArgs& a, int batch, int num_kv_heads, hipStream_t stream);

// Quantising append into 8-bit pools: src_dtype is the type of key/value rows.
hipError_t launch_reshape_and_cache_fp8(const CacheArgs& a, int src_dtype, int head_dim, const void* key,
                                        const void* value, float* k_scale, float* v_scale,
                                        const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream);

}  // namespace pagedkv
