// C ABI of libpagedkv: argument checks, launch-shape policy and kernel dispatch.
// No compute happens here; every step of the path runs in the HIP kernels.
#include <math.h>

#include <mutex>

#include "../../include/pagedkv_measure.h"
#include "pa_kernels.h"

using namespace pagedkv;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int log2_exact(int x) {
    if (x <= 0 || (x & (x - 1))) return -1;
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

int dtype_bytes(int dtype) {
    switch (dtype) {
        case PA_F32: return 4;
        case PA_F16:
        case PA_BF16: return 2;
        case PA_FP8_E4M3: return 1;
        default: return 0;
    }
}

int64_t dense_block_bytes(const pa_cache_desc_t* c) {
    return (int64_t)c->num_kv_heads * c->block_size * c->head_dim * dtype_bytes(c->dtype);
}

pa_status_t check_cache(const pa_cache_desc_t* c) {
    if (!c) return PA_ERR_INVALID_ARGUMENT;
    if (dtype_bytes(c->dtype) == 0) return PA_ERR_UNSUPPORTED;
    if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256) return PA_ERR_UNSUPPORTED;
    const int lbs = log2_exact(c->block_size);
    if (lbs < 3 || lbs > 9) return PA_ERR_UNSUPPORTED;  // 8 .. 512 tokens per block
    if (c->num_blocks <= 0 || c->num_kv_heads <= 0 || c->num_kv_heads > 65535) return PA_ERR_INVALID_ARGUMENT;
    // one pool must be addressable with the kernels' 64-bit byte offsets and 32-bit slots
    if ((int64_t)c->num_blocks * c->block_size > INT32_MAX) return PA_ERR_INVALID_ARGUMENT;
    if (c->block_stride != 0 && (c->block_stride % 16 != 0 || c->block_stride < dense_block_bytes(c)))
        return PA_ERR_INVALID_ARGUMENT;
    return PA_OK;
}

// Bytes from one physical block to the next (the dense size unless a stride is given).
int64_t block_stride(const pa_cache_desc_t* c) { return c->block_stride ? c->block_stride : dense_block_bytes(c); }

pa_status_t from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool is_fp8(const pa_cache_desc_t* c) { return c->dtype == PA_FP8_E4M3; }

// Tokens a sequence's partitions cover: everything without a window; with one, the window
// plus at most block_size - 1 tokens before it in the block where it starts.
int32_t window_span(const pa_cache_desc_t* c, int32_t max_context_len, int32_t window) {
    if (window <= 0) return max_context_len;
    const int64_t span = (int64_t)window + c->block_size - 1;
    return span < max_context_len ? (int32_t)span : max_context_len;
}

// The launch arguments every attention entry point shares. `rows` are the rows of q and out
// (sequences, or query tokens), which size the partition records; `need` is the workspace
// the call requires (records follow their outputs: o first, then the (max, sum) pairs).
DecodeArgs attention_args(const pa_cache_desc_t* c, void* out, const void* q, const void* k_pool, const void* v_pool,
                          const float* k_scale, const float* v_scale, const int32_t* block_table,
                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch, int64_t rows,
                          int32_t num_q_heads, int32_t max_context_len, float scale, int32_t P, int64_t parts,
                          void* workspace, size_t need, int32_t* err_flag) {
    DecodeArgs a{};
    a.out = out;
    a.q = q;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.context_lens = context_lens;
    a.ws_o = static_cast<float*>(workspace);
    a.ws_ml = need > 0 ? a.ws_o + (size_t)rows * num_q_heads * parts * c->head_dim : nullptr;
    a.err_flag = err_flag;
    a.num_blocks = c->num_blocks;
    a.log2_block_size = log2_exact(c->block_size);
    a.num_kv_heads = c->num_kv_heads;
    a.num_q_heads = num_q_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.max_context_len = max_context_len;
    a.partition_size = P;
    a.max_partitions = (int32_t)parts;
    a.scale_log2 = scale * 1.4426950408889634f;  // scores live in the base-2 exponent domain
    a.block_stride = block_stride(c);
    a.batch = batch;
    return a;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status_t s) {
    switch (s) {
        case PA_OK: return "PA_OK";
        case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT: bad pointer, size or workspace";
        case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype, head_dim, block_size or group not built";
        case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: the HIP runtime refused a kernel launch";
        case PA_ERR_SCRATCH_LIMIT:
            return "PA_ERR_SCRATCH_LIMIT: the call needs more workspace than the static scratch of "
                   "pa_decode_append_noalloc (PA_NOALLOC_SCRATCH_BYTES)";
        default: return "unknown pa_status_t";
    }
}

pa_status_t pa_reshape_and_cache(const pa_cache_desc_t* cache, const void* key, const void* value,
                                 void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                 int32_t num_tokens, int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARGUMENT;
    CacheArgs a{k_pool, v_pool, err_flag, cache->num_blocks, log2_exact(cache->block_size),
                cache->num_kv_heads, cache->head_dim * dtype_bytes(cache->dtype) / 16, block_stride(cache)};
    return from_hip(launch_reshape_and_cache(a, key, value, slot_mapping, num_tokens, (hipStream_t)stream));
}

pa_status_t pa_copy_blocks(const pa_cache_desc_t* cache, void* k_pool, void* v_pool, const int32_t* pairs,
                           int32_t num_pairs, int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    if (num_pairs < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_pairs == 0) return PA_OK;
    if (!k_pool || !v_pool || !pairs) return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARGUMENT;
    CacheArgs a{k_pool, v_pool, err_flag, cache->num_blocks, log2_exact(cache->block_size),
                cache->num_kv_heads, cache->head_dim * dtype_bytes(cache->dtype) / 16, block_stride(cache)};
    return from_hip(launch_copy_blocks(a, pairs, num_pairs, nullptr, nullptr, (hipStream_t)stream));
}

pa_status_t pa_reshape_and_cache_fp8(const pa_cache_desc_t* cache, int32_t src_dtype, const void* key,
                                     const void* value, void* k_pool, void* v_pool, float* k_scale,
                                     float* v_scale, const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (!is_fp8(cache)) return PA_ERR_INVALID_ARGUMENT;
    if (src_dtype != PA_F32 && src_dtype != PA_F16 && src_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
    if (num_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_tokens == 0) return PA_OK;
    if (!key || !value || !k_pool || !v_pool || !k_scale || !v_scale || !slot_mapping)
        return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned4(k_scale) ||
        !aligned4(v_scale))
        return PA_ERR_INVALID_ARGUMENT;
    CacheArgs a{k_pool, v_pool, err_flag, cache->num_blocks, log2_exact(cache->block_size),
                cache->num_kv_heads, cache->head_dim / 16, block_stride(cache)};
    return from_hip(launch_reshape_and_cache_fp8(a, src_dtype, cache->head_dim, key, value, k_scale, v_scale,
                                                 slot_mapping, num_tokens, (hipStream_t)stream));
}

pa_status_t pa_copy_blocks_fp8(const pa_cache_desc_t* cache, void* k_pool, void* v_pool, float* k_scale,
                               float* v_scale, const int32_t* pairs, int32_t num_pairs, int32_t* err_flag,
                               pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (!is_fp8(cache)) return PA_ERR_INVALID_ARGUMENT;
    if (num_pairs < 0) return PA_ERR_INVALID_ARGUMENT;
    if (num_pairs == 0) return PA_OK;
    if (!k_pool || !v_pool || !k_scale || !v_scale || !pairs) return PA_ERR_INVALID_ARGUMENT;
    // scale rows are copied as 16-byte vectors: block_size >= 8 makes each head's run 32+ bytes
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_scale) || !aligned16(v_scale))
        return PA_ERR_INVALID_ARGUMENT;
    CacheArgs a{k_pool, v_pool, err_flag, cache->num_blocks, log2_exact(cache->block_size),
                cache->num_kv_heads, cache->head_dim / 16, block_stride(cache)};
    return from_hip(launch_copy_blocks(a, pairs, num_pairs, k_scale, v_scale, (hipStream_t)stream));
}

pa_status_t pa_reblock(const pa_cache_desc_t* src, const void* src_k, const void* src_v, const float* src_k_scale,
                       const float* src_v_scale, const int32_t* src_table, int32_t src_max_blocks_per_seq,
                       const pa_cache_desc_t* dst, void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                       const int32_t* dst_table, int32_t dst_max_blocks_per_seq, const int32_t* context_lens,
                       int32_t batch, int32_t max_context_len, int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(src);
    if (st != PA_OK) return st;
    if ((st = check_cache(dst)) != PA_OK) return st;
    if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim || src->dtype != dst->dtype)
        return PA_ERR_INVALID_ARGUMENT;
    if (batch < 0 || batch > 65535 || max_context_len < 0) return PA_ERR_INVALID_ARGUMENT;
    if (batch == 0 || max_context_len == 0) return PA_OK;
    if (!src_k || !src_v || !src_table || !dst_k || !dst_v || !dst_table || !context_lens)
        return PA_ERR_INVALID_ARGUMENT;
    if (src_max_blocks_per_seq <= 0 || dst_max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v)) return PA_ERR_INVALID_ARGUMENT;
    const bool scaled = is_fp8(src);
    const bool any_scale = src_k_scale || src_v_scale || dst_k_scale || dst_v_scale;
    if (scaled) {
        if (!src_k_scale || !src_v_scale || !dst_k_scale || !dst_v_scale) return PA_ERR_INVALID_ARGUMENT;
        if (!aligned4(src_k_scale) || !aligned4(src_v_scale) || !aligned4(dst_k_scale) || !aligned4(dst_v_scale))
            return PA_ERR_INVALID_ARGUMENT;
    } else if (any_scale) {
        return PA_ERR_INVALID_ARGUMENT;
    }
    ReblockArgs a{static_cast<const char*>(src_k), static_cast<const char*>(src_v), src_k_scale, src_v_scale,
                  src_table, static_cast<char*>(dst_k), static_cast<char*>(dst_v), dst_k_scale, dst_v_scale,
                  dst_table, context_lens, err_flag, block_stride(src), block_stride(dst), src->num_blocks,
                  dst->num_blocks, log2_exact(src->block_size), log2_exact(dst->block_size), src_max_blocks_per_seq,
                  dst_max_blocks_per_seq, src->num_kv_heads, src->head_dim * dtype_bytes(src->dtype) / 16,
                  max_context_len};
    return from_hip(launch_reblock(a, batch, (hipStream_t)stream));
}

int32_t pa_decode_partition_size(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t requested) {
    if (check_cache(cache) != PA_OK || batch < 0 || max_context_len <= 0 || num_q_heads <= 0) return -1;
    const int bs = cache->block_size;
    const int64_t max_p = (int64_t)kMaxIdsPerPartition * bs;
    if (requested > 0) {
        if (requested % bs != 0 || requested > max_p) return -1;
        return requested;
    }
    // Defaults, from measurements on MI355X. Each workgroup pays a fixed prologue (length,
    // table and q loads) and epilogue, and splitting a sequence adds the reduce pass, so
    // partitions are as long as the launch shape allows.
    const int64_t wgs = (int64_t)batch * cache->num_kv_heads;
    const int64_t whole = ceil_div(max_context_len, bs) * bs;
    const int group = num_q_heads % cache->num_kv_heads == 0 ? num_q_heads / cache->num_kv_heads : 1;
    int64_t P;
    if (decode_mfma_supported(cache->dtype, cache->head_dim, group, bs)) {
        // Matrix-core path: one 4-wave workgroup per compute unit already streams at its
        // best; split only to reach 256 workgroups or to cap a partition at 4096 tokens.
        int64_t parts = wgs >= 256 ? 1 : ceil_div(256, wgs > 0 ? wgs : 1);
        if (parts < ceil_div(max_context_len, 4096)) parts = ceil_div(max_context_len, 4096);
        P = ceil_div(ceil_div(max_context_len, parts), bs) * bs;
    } else if (max_context_len <= (is_fp8(cache) ? 2048 : 1024) && wgs >= 128) {
        // VALU path, short contexts and at least half a workgroup per compute unit: no split
        // (the reduce launch costs more than the extra parallelism gains; equal lengths of
        // 600 tokens at 8 x 32 heads: 16.0 us whole against 18.6 us in 256-token partitions).
        // 8-bit rows stream in half the time, so contexts twice as long stay whole (256
        // sequences x 32 heads of long-tailed lengths, median 87, up to 1197 tokens: 85.7
        // against 90.8 us at P = 512; 16-bit pools there: 126.9 against 124.1 us).
        P = whole;
    } else {
        // VALU path: partitions of 256 tokens up to 2048-token contexts (a long-tailed batch
        // ends sooner when its longest sequences come in short pieces: that 256 x 32-head
        // batch was 1-2% faster per step at every block size than at 512), and
        // of 512 beyond (32K contexts: 7% slower at 256); shortened until the launch has about
        // 2048 workgroups (8 per compute unit).
        const int base_p = max_context_len <= 2048 ? 256 : 512;
        P = ceil_div(base_p > bs ? base_p : bs, bs) * bs;
        if (wgs * ceil_div(max_context_len, P) < 2048) {
            int64_t want = ceil_div((int64_t)max_context_len * wgs, 2048);
            // not below 256 tokens: shorter partitions lost 15-40% on small launches
            // (4 x 1000, 1 x 4096 and 8 x 600 tokens at 32 heads; 64 tokens against 256)
            const int64_t floor_p = bs > 256 ? bs : 256;
            if (want < floor_p) want = floor_p;
            P = ceil_div(want, bs) * bs;
        }
    }
    if (P > max_p) P = max_p;
    if (P > whole) P = whole;
    return (int32_t)P;
}

size_t pa_decode_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size) {
    const int32_t P = pa_decode_partition_size(cache, batch, num_q_heads, max_context_len, partition_size);
    if (P <= 0 || num_q_heads <= 0) return 0;
    const int64_t parts = ceil_div(max_context_len, P);
    if (parts <= 1) return 0;
    // partition records, then one slot per sequence for a fused append (pa_decode_append)
    return (size_t)batch * num_q_heads * parts * (cache->head_dim + 2) * sizeof(float) + (size_t)batch * sizeof(int32_t);
}

size_t pa_decode_sliding_window_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch,
                                                int32_t num_q_heads, int32_t max_context_len, int32_t window,
                                                int32_t partition_size) {
    if (check_cache(cache) != PA_OK || window <= 0 || max_context_len <= 0) return 0;
    return pa_decode_workspace_bytes(cache, batch, num_q_heads, window_span(cache, max_context_len, window),
                                     partition_size);
}

}  // extern "C"

namespace {

int32_t multi_partition_size(const pa_cache_desc_t* c, int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                             int32_t max_query_len, int32_t requested) {
    if (check_cache(c) != PA_OK || batch < 0 || max_context_len <= 0 || num_q_heads <= 0 || max_query_len <= 0)
        return -1;
    const int bs = c->block_size;
    const int64_t max_p = (int64_t)kMaxIdsPerPartition * bs;
    if (requested > 0) return (requested % bs != 0 || requested > max_p) ? -1 : requested;
    // As the grouped decode: one partition when the (sequence, kv head, column tile) grid
    // already holds 256 workgroups, else split towards 256; at most 4096 tokens each.
    const int group = num_q_heads % c->num_kv_heads == 0 ? num_q_heads / c->num_kv_heads : 1;
    const int64_t tiles = (int64_t)batch * c->num_kv_heads * ceil_div((int64_t)max_query_len * group, 16);
    int64_t parts = tiles >= 256 ? 1 : ceil_div(256, tiles > 0 ? tiles : 1);
    if (parts < ceil_div(max_context_len, 4096)) parts = ceil_div(max_context_len, 4096);
    int64_t P = ceil_div(ceil_div(max_context_len, parts), bs) * bs;
    if (P > max_p) P = max_p;
    return (int32_t)P;
}

}  // namespace

extern "C" {

size_t pa_multi_token_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_tokens,
                                      int32_t num_q_heads, int32_t max_context_len, int32_t max_query_len,
                                      int32_t partition_size) {
    const int32_t P = multi_partition_size(cache, batch, num_q_heads, max_context_len, max_query_len, partition_size);
    if (P <= 0 || num_q_tokens <= 0) return 0;
    const int64_t parts = ceil_div(max_context_len, P);
    if (parts <= 1) return 0;
    return (size_t)num_q_tokens * num_q_heads * parts * (cache->head_dim + 2) * sizeof(float);
}

pa_status_t pa_multi_token_attention(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                                     const void* k_pool, const void* v_pool, const float* k_scale,
                                     const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* query_start, int32_t batch,
                                     int32_t num_q_tokens, int32_t num_q_heads, int32_t max_context_len,
                                     int32_t max_query_len, float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (batch < 0 || batch > 65535 || num_q_tokens < 0) return PA_ERR_INVALID_ARGUMENT;
    if (batch == 0 || num_q_tokens == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens || !query_start)
        return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARGUMENT;
    if (is_fp8(cache)) {
        if (q_dtype != PA_F16 && q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
        if (!k_scale || !v_scale || !aligned4(k_scale) || !aligned4(v_scale)) return PA_ERR_INVALID_ARGUMENT;
    } else if (q_dtype != cache->dtype) {
        return PA_ERR_INVALID_ARGUMENT;
    }
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
    const int group = num_q_heads / cache->num_kv_heads;
    if (!multi_token_supported(cache->dtype, cache->head_dim, group, cache->block_size)) return PA_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || max_context_len <= 0 || max_query_len <= 0 || max_query_len > max_context_len)
        return PA_ERR_INVALID_ARGUMENT;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * cache->block_size) return PA_ERR_INVALID_ARGUMENT;
    if (!isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
    const int64_t col_tiles = ceil_div((int64_t)max_query_len * group, 16);
    if (col_tiles * batch > 65535) return PA_ERR_UNSUPPORTED;
    const int32_t P =
        multi_partition_size(cache, batch, num_q_heads, max_context_len, max_query_len, partition_size);
    if (P <= 0) return PA_ERR_INVALID_ARGUMENT;
    const int64_t parts = ceil_div(max_context_len, P);
    if (parts > kMaxPartitionSlots) return PA_ERR_UNSUPPORTED;
    const size_t need = pa_multi_token_workspace_bytes(cache, batch, num_q_tokens, num_q_heads, max_context_len,
                                                       max_query_len, partition_size);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PA_ERR_INVALID_ARGUMENT;

    DecodeArgs a = attention_args(cache, out, q, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks_per_seq,
                                  context_lens, batch, num_q_tokens, num_q_heads, max_context_len, scale, P, parts,
                                  workspace, need, err_flag);
    a.query_start = query_start;
    a.col_tiles = (int32_t)col_tiles;
    a.num_q_tokens = num_q_tokens;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_multi_token(a, cache->dtype, q_dtype, cache->head_dim, group, batch, cache->num_kv_heads, s);
    if (e == hipSuccess && parts > 1) e = launch_reduce_multi(a, q_dtype, cache->head_dim, s);
    return from_hip(e);
}

}  // extern "C"

namespace {

pa_status_t decode_impl(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                        const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                        const int32_t* block_table, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                        int32_t max_context_len, float scale, int32_t partition_size, int32_t window,
                        void* workspace, size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream,
                        const void* new_key = nullptr, const void* new_value = nullptr,
                        const int32_t* slot_mapping = nullptr) {
    if (window < 0) return PA_ERR_INVALID_ARGUMENT;
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (batch < 0 || batch > 65535) return PA_ERR_INVALID_ARGUMENT;
    if (batch == 0) return PA_OK;
    if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PA_ERR_INVALID_ARGUMENT;
    // a VALU wave load covers 1 KiB of consecutive token rows, which must lie in one block;
    // grouped heads that run on the matrix cores take smaller slabs too
    if ((int64_t)cache->head_dim * dtype_bytes(cache->dtype) * cache->block_size < 1024 &&
        !(num_q_heads % cache->num_kv_heads == 0 &&
          decode_mfma_supported(cache->dtype, cache->head_dim, num_q_heads / cache->num_kv_heads, cache->block_size)))
        return PA_ERR_UNSUPPORTED;
    if (is_fp8(cache)) {
        if (q_dtype != PA_F16 && q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
        // the VALU kernel takes at most 8 query heads per kv head over 8-bit pools
        const int g8 = num_q_heads / cache->num_kv_heads;
        if (g8 > 8 && !decode_mfma_supported(cache->dtype, cache->head_dim, g8, cache->block_size))
            return PA_ERR_UNSUPPORTED;
        if (!k_scale || !v_scale || !aligned4(k_scale) || !aligned4(v_scale)) return PA_ERR_INVALID_ARGUMENT;
    } else if (q_dtype != cache->dtype) {
        return PA_ERR_INVALID_ARGUMENT;
    }
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARGUMENT;
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
    const int group = num_q_heads / cache->num_kv_heads;
    if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16) return PA_ERR_UNSUPPORTED;
    if (group == 16 && cache->head_dim > 128) return PA_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARGUMENT;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * cache->block_size) return PA_ERR_INVALID_ARGUMENT;
    if (!isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
    // Partitions tile [start of the window's first block, L): at most `span` tokens.
    const int32_t span = window_span(cache, max_context_len, window);
    const int32_t P = pa_decode_partition_size(cache, batch, num_q_heads, span, partition_size);
    if (P <= 0) return PA_ERR_INVALID_ARGUMENT;
    const int64_t parts = ceil_div(span, P);
    if (parts > kMaxPartitionSlots) return PA_ERR_UNSUPPORTED;
    const size_t need = pa_decode_workspace_bytes(cache, batch, num_q_heads, span, partition_size);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PA_ERR_INVALID_ARGUMENT;

    DecodeArgs a = attention_args(cache, out, q, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks_per_seq,
                                  context_lens, batch, batch, num_q_heads, max_context_len, scale, P, parts, workspace,
                                  need, err_flag);
    a.window = window;
    a.new_key = new_key;
    a.new_value = new_value;
    a.slot_mapping = slot_mapping;
    // with a reduce pass, 16-bit rows are written by it, after the decode has read the pool
    // (8-bit rows are quantised by the decode and written by it)
    a.ws_slot = (slot_mapping && parts > 1 && !is_fp8(cache))
                    ? reinterpret_cast<int32_t*>(a.ws_ml + (size_t)batch * num_q_heads * parts * 2)
                    : nullptr;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = decode_mfma_supported(cache->dtype, cache->head_dim, group, cache->block_size)
                       ? launch_decode_mfma(a, cache->dtype, q_dtype, cache->head_dim, group, batch,
                                            cache->num_kv_heads, s)
                       : launch_decode_valu(a, cache->dtype, q_dtype, cache->head_dim, group, batch,
                                            cache->num_kv_heads, s);
    if (e == hipSuccess && parts > 1) e = launch_reduce(a, q_dtype, cache->head_dim, batch, s);
    return from_hip(e);
}

}  // namespace

extern "C" {

pa_status_t pa_decode(const pa_cache_desc_t* cache, void* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                      size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream) {
    if (cache && is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    return decode_impl(cache, cache ? cache->dtype : 0, out, q, k_pool, v_pool, nullptr, nullptr, block_table,
                       max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale, partition_size,
                       0, workspace, workspace_bytes, err_flag, stream);
}

pa_status_t pa_decode_sliding_window(const pa_cache_desc_t* cache, void* out, const void* q,
                                     const void* k_pool, const void* v_pool, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t max_context_len, float scale,
                                     int32_t window, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream) {
    if (window <= 0) return PA_ERR_INVALID_ARGUMENT;
    if (cache && is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    return decode_impl(cache, cache ? cache->dtype : 0, out, q, k_pool, v_pool, nullptr, nullptr, block_table,
                       max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale, partition_size,
                       window, workspace, workspace_bytes, err_flag, stream);
}

pa_status_t pa_decode_append(const pa_cache_desc_t* cache, void* out, const void* q, void* k_pool, void* v_pool,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                             const void* key, const void* value, const int32_t* slot_mapping,
                             int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                             pa_stream_t stream) {
    if (cache && is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    if (batch > 0 && (!key || !value || !slot_mapping || !aligned16(key) || !aligned16(value)))
        return PA_ERR_INVALID_ARGUMENT;
    return decode_impl(cache, cache ? cache->dtype : 0, out, q, k_pool, v_pool, nullptr, nullptr, block_table,
                       max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale, partition_size,
                       0, workspace, workspace_bytes, err_flag, stream, key, value, slot_mapping);
}

}  // extern "C"

namespace {

// Scratch of pa_decode_append_noalloc: the partition records and slot words that the other
// entry points take from the caller's workspace, in a static device array that every GPU the
// library runs on holds until the process ends. In host code `scratch` names a host-side
// stand-in, not device memory: kernels get the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in noalloc_scratch_ptr.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (set-up on the first call per device).
pa_status_t noalloc_scratch_ptr(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return PA_ERR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

extern "C" {

pa_status_t pa_decode_append_noalloc(const pa_cache_desc_t* cache, void* out, const void* q, void* k_pool,
                                     void* v_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                                     int32_t max_context_len, float scale, const void* key, const void* value,
                                     const int32_t* slot_mapping, int32_t partition_size, int32_t* err_flag,
                                     pa_stream_t stream) {
    if (cache && is_fp8(cache)) return PA_ERR_UNSUPPORTED;
    if (batch > 0 && (!key || !value || !slot_mapping || !aligned16(key) || !aligned16(value)))
        return PA_ERR_INVALID_ARGUMENT;
    // sizes first (no device call), so an oversized request is rejected before any set-up
    if (check_cache(cache) == PA_OK && batch > 0 && max_context_len > 0 &&
        pa_decode_workspace_bytes(cache, batch, num_q_heads, max_context_len, partition_size) >
            (size_t)PA_NOALLOC_SCRATCH_BYTES)
        return PA_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (batch > 0) {
        const pa_status_t st = noalloc_scratch_ptr(&ws);
        if (st != PA_OK) return st;
    }
    return decode_impl(cache, cache ? cache->dtype : 0, out, q, k_pool, v_pool, nullptr, nullptr, block_table,
                       max_blocks_per_seq, context_lens, batch, num_q_heads, max_context_len, scale, partition_size,
                       0, ws, ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, err_flag, stream, key, value, slot_mapping);
}

pa_status_t pa_decode_append_fp8(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                                 void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                 const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                                 const void* key, const void* value, const int32_t* slot_mapping,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                 pa_stream_t stream) {
    if (!cache || !is_fp8(cache)) return PA_ERR_INVALID_ARGUMENT;
    if (batch > 0 && (!key || !value || !slot_mapping || !aligned16(key) || !aligned16(value)))
        return PA_ERR_INVALID_ARGUMENT;
    return decode_impl(cache, q_dtype, out, q, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, max_context_len, scale, partition_size, 0, workspace,
                       workspace_bytes, err_flag, stream, key, value, slot_mapping);
}

pa_status_t pa_decode_fp8(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale, int32_t window,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                          pa_stream_t stream) {
    if (!cache || !is_fp8(cache)) return PA_ERR_INVALID_ARGUMENT;
    return decode_impl(cache, q_dtype, out, q, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks_per_seq,
                       context_lens, batch, num_q_heads, max_context_len, scale, partition_size, window, workspace,
                       workspace_bytes, err_flag, stream);
}

}  // extern "C"

namespace {

int32_t beams_partition_size(const pa_cache_desc_t* c, int32_t batch, int32_t beam_width, int32_t num_q_heads,
                             int32_t max_context_len, int32_t requested) {
    if (check_cache(c) != PA_OK || batch < 0 || beam_width <= 0 || max_context_len <= 0 || num_q_heads <= 0)
        return -1;
    const int bs = c->block_size;
    // every beam of a group stages its table slice: beam_width * P / bs entries
    const int64_t max_p = (int64_t)(kMaxBeamIds / beam_width) * bs;
    if (max_p < bs) return -1;
    if (requested > 0) return (requested % bs != 0 || requested > max_p) ? -1 : requested;
    // Measured defaults: 1024-token partitions (a block multiple; on 32K-token beams 512 and
    // 2048 were 8% and 4% slower, 256 30%), shortened while the launch has fewer than 1024
    // workgroups, never past one partition per context.
    const int64_t pairs = ceil_div(batch, beam_width) * (int64_t)c->num_kv_heads;
    int64_t P = ceil_div(1024 > bs ? 1024 : bs, bs) * bs;
    if (pairs * ceil_div(max_context_len, P) < 1024) {
        int64_t want = ceil_div((int64_t)max_context_len * pairs, 1024);
        if (want < 64) want = 64;
        P = ceil_div(want, bs) * bs;
    }
    const int64_t whole = ceil_div(max_context_len, bs) * bs;
    if (P > whole) P = whole;
    if (P > max_p) P = max_p;
    return (int32_t)P;
}

}  // namespace

extern "C" {

int32_t pa_decode_beams_partition_size(const pa_cache_desc_t* cache, int32_t batch, int32_t beam_width,
                                       int32_t num_q_heads, int32_t max_context_len, int32_t requested) {
    return beams_partition_size(cache, batch, beam_width, num_q_heads, max_context_len, requested);
}

size_t pa_decode_beams_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t beam_width,
                                       int32_t num_q_heads, int32_t max_context_len, int32_t partition_size) {
    const int32_t P = beams_partition_size(cache, batch, beam_width, num_q_heads, max_context_len, partition_size);
    if (P <= 0) return 0;
    const int64_t parts = ceil_div(max_context_len, P);
    if (parts <= 1) return 0;
    // the partition records of pa_decode (no slot words: the beam decode has no fused append)
    return (size_t)batch * num_q_heads * parts * (cache->head_dim + 2) * sizeof(float);
}

pa_status_t pa_decode_beams(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                            const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t batch, int32_t beam_width, int32_t num_q_heads, int32_t max_context_len,
                            float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                            int32_t* err_flag, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (batch < 0 || beam_width <= 0) return PA_ERR_INVALID_ARGUMENT;
    if (batch == 0) return PA_OK;
    if (ceil_div(batch, beam_width) > 65535) return PA_ERR_INVALID_ARGUMENT;
    if (!out || !q || !k_pool || !v_pool || !block_table || !context_lens) return PA_ERR_INVALID_ARGUMENT;
    if (is_fp8(cache)) {
        if (q_dtype != PA_F16 && q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
        if (!k_scale || !v_scale || !aligned4(k_scale) || !aligned4(v_scale)) return PA_ERR_INVALID_ARGUMENT;
    } else if (q_dtype != cache->dtype) {
        return PA_ERR_INVALID_ARGUMENT;
    }
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
        return PA_ERR_INVALID_ARGUMENT;
    if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads != 0) return PA_ERR_INVALID_ARGUMENT;
    const int group = num_q_heads / cache->num_kv_heads;
    if (!decode_beams_supported(cache->dtype, cache->head_dim, group, cache->block_size, beam_width))
        return PA_ERR_UNSUPPORTED;
    if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARGUMENT;
    if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * cache->block_size) return PA_ERR_INVALID_ARGUMENT;
    if (!isfinite(scale)) return PA_ERR_INVALID_ARGUMENT;
    const int32_t P = beams_partition_size(cache, batch, beam_width, num_q_heads, max_context_len, partition_size);
    if (P <= 0) return PA_ERR_INVALID_ARGUMENT;
    const int64_t parts = ceil_div(max_context_len, P);
    if (parts > kMaxPartitionSlots) return PA_ERR_UNSUPPORTED;
    const size_t need = pa_decode_beams_workspace_bytes(cache, batch, beam_width, num_q_heads, max_context_len, P);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace))) return PA_ERR_INVALID_ARGUMENT;

    DecodeArgs a = attention_args(cache, out, q, k_pool, v_pool, k_scale, v_scale, block_table, max_blocks_per_seq,
                                  context_lens, batch, batch, num_q_heads, max_context_len, scale, P, parts, workspace,
                                  need, err_flag);
    a.beam_width = beam_width;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_decode_beams(a, cache->dtype, q_dtype, cache->head_dim, group,
                                       (int)ceil_div(batch, beam_width), cache->num_kv_heads, s);
    if (e == hipSuccess && parts > 1) e = launch_reduce(a, q_dtype, cache->head_dim, batch, s);
    return from_hip(e);
}

pa_status_t pa_measure_gather_read(const pa_cache_desc_t* cache, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, int32_t max_blocks_per_seq,
                                   const int32_t* context_lens, int32_t batch, int32_t max_context_len,
                                   float* sink, pa_stream_t stream) {
    pa_status_t st = check_cache(cache);
    if (st != PA_OK) return st;
    if (batch < 0 || batch > 65535) return PA_ERR_INVALID_ARGUMENT;
    if (batch == 0) return PA_OK;
    if (!k_pool || !v_pool || !block_table || !context_lens || !sink) return PA_ERR_INVALID_ARGUMENT;
    if (!aligned16(k_pool) || !aligned16(v_pool)) return PA_ERR_INVALID_ARGUMENT;
    if (max_blocks_per_seq <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARGUMENT;
    // a wave load is 1 KiB of consecutive rows, which must lie in one block
    const int row_bytes = cache->head_dim * dtype_bytes(cache->dtype);
    if (row_bytes > 1024 || (int64_t)cache->block_size * row_bytes < 1024) return PA_ERR_UNSUPPORTED;
    GatherReadArgs a{static_cast<const char*>(k_pool), static_cast<const char*>(v_pool), block_table, context_lens,
                     sink, block_stride(cache), cache->num_blocks, max_blocks_per_seq, max_context_len,
                     log2_exact(cache->block_size), row_bytes};
    return from_hip(launch_gather_read(a, batch, cache->num_kv_heads, (hipStream_t)stream));
}

}  // extern "C"
