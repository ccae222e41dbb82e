/*
 * pagedkv.h - C ABI of libpagedkv: paged KV-cache decode attention for AMD MI355X (gfx950).
 *
 * Pages cited (by title and section):
 *   [BlockManager essay]  "KV Cache & BlockManager", dpshk.com/news/5906718
 *   [KV Block course]     vLLM memory-management course, ch. 3 "KV Block design"
 *   [Valid-length essay]  KV-cache valid length and padding-KV bug, dpshk.com/news/5937191
 *   [CANN paging article] "KV Cache paging optimisation in LLM inference", intelliparadigm.com
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is device memory owned by the caller (allocated, for
 *     instance, by torch). The library allocates nothing, keeps no state between calls
 *     and never synchronises: each call enqueues kernels on `stream` and returns.
 *   - Argument errors are found on the host before anything is launched and come back as
 *     a status other than PA_OK. A failed launch returns PA_ERR_LAUNCH.
 *   - Data errors that only the device can see (a bad block id, length or slot) never
 *     cause an out-of-bounds access: the affected item is skipped or its output set to
 *     NaN, and a bit (PA_FLAG_*) is OR-ed into *err_flag when err_flag is not NULL
 *     (reject, do not corrupt: [BlockManager essay] §4.1). The flag is never cleared by
 *     the library.
 *   - Layouts (row-major, contiguous):
 *       q, out             [batch][num_q_heads][head_dim]
 *       k_pool, v_pool     [num_blocks][num_kv_heads][block_size][head_dim]
 *                          (one block holds heads x block_size x head_dim for K and the
 *                          same for V: [BlockManager essay] §5.1, [KV Block course] §3.2)
 *       key, value         [num_tokens][num_kv_heads][head_dim]
 *       block_table        int32 [batch][max_blocks_per_seq], logical -> physical block
 *                          id, entries past the valid blocks are never read and may be -1
 *                          ([BlockManager essay] §2)
 *       context_lens       int32 [batch], number of valid tokens ([Valid-length essay] §4.1)
 *       slot_mapping       int32 [num_tokens], physical slot = block * block_size + offset
 *       pairs              int32 [num_pairs][2] = (src, dst) physical block ids
 *       k_scale, v_scale   float32 [num_blocks][num_kv_heads][block_size] (8-bit pools only)
 *   - q, out, key, value, k_pool and v_pool must be 16-byte aligned
 *     ([KV Block course] §3.7 on aligned block starts).
 *   - Supported: dtype f32/f16/bf16 (and 8-bit float pools, see PA_FP8_E4M3); head_dim
 *     64, 128, 256; block_size a power of two in [8, 512]; num_q_heads / num_kv_heads in
 *     {1, 2, 4, 8, 16}.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t; NULL is the default stream. */
typedef struct ihipStream_t* pa_stream_t;

typedef enum {
    PA_OK = 0,
    PA_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, workspace too small */
    PA_ERR_UNSUPPORTED = 2,      /* dtype, head_dim, block_size or group not built */
    PA_ERR_LAUNCH = 3,           /* the HIP runtime refused a launch */
    PA_ERR_SCRATCH_LIMIT = 4     /* pa_decode_append_noalloc: more workspace than its static scratch */
} pa_status_t;

/*
 * Element types. PA_FP8_E4M3 is a pool element type only: 8-bit floats in the OCP E4M3
 * format (sign, 4 exponent bits with bias 7, 3 mantissa bits; largest finite 448; S.1111.111
 * is NaN) with one float32 scale per (block, kv head, offset) row, so a row is worth
 * code * scale (the quantised blocks of [BlockManager essay] §3 and §6.3). Such pools are
 * written, copied and read only by the *_fp8 entry points; q, out, key and value stay
 * f16/bf16 (f32 too for key and value).
 */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype_t;

/* Device-side data error bits OR-ed into *err_flag. */
#define PA_FLAG_BAD_BLOCK_ID   1  /* a table entry inside the valid range is outside [0, num_blocks) */
#define PA_FLAG_BAD_LENGTH     2  /* context_len > max_context_len or > max_blocks_per_seq * block_size */
#define PA_FLAG_EMPTY_CONTEXT  4  /* context_len <= 0 */
#define PA_FLAG_BAD_SLOT       8  /* slot >= num_blocks * block_size */
#define PA_FLAG_BAD_COPY_PAIR 16  /* src or dst outside [0, num_blocks), or src == dst */

/*
 * Shape of one physical pool pair (K and V have the same shape).
 *
 * block_stride is the distance in bytes from block i to block i + 1 in k_pool and in
 * v_pool; 0 means dense (num_kv_heads * block_size * head_dim * element bytes). A larger
 * stride lets one allocation hold every layer's K and V, [num_blocks][2][num_layers]
 * [num_kv_heads][block_size][head_dim] ([BlockManager essay] §5.1): the pools of layer l
 * are then k_pool = base + (0 * num_layers + l) * dense bytes, v_pool = base + (1 *
 * num_layers + l) * dense bytes, and block_stride = 2 * num_layers * dense bytes. Inside a
 * block, heads, tokens and dims stay dense. block_stride must be 0 or a multiple of 16 that
 * is at least the dense size. Scale pools of 8-bit caches are always dense.
 */
typedef struct {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* pa_dtype_t */
    int64_t block_stride;
} pa_cache_desc_t;

/*
 * pa_reshape_and_cache - write new tokens' K and V into their pool slots.
 *
 * Token i's rows key[i] and value[i] ([num_kv_heads][head_dim]) are copied bit for bit to
 * block slot_mapping[i] / block_size, offset slot_mapping[i] % block_size, of every kv head,
 * so the physical order inside a block equals the logical order ([BlockManager essay] §4.4;
 * new K/V land at the valid length, [Valid-length essay] §4.1). A negative slot marks a
 * padding token and is skipped, so padding KV never enters the cache ([Valid-length essay]
 * §2.3). A slot >= num_blocks * block_size is skipped and sets PA_FLAG_BAD_SLOT.
 * num_tokens == 0 launches nothing. Two tokens with the same slot race (caller error).
 * An 8-bit pool returns PA_ERR_UNSUPPORTED (use pa_reshape_and_cache_fp8).
 */
pa_status_t pa_reshape_and_cache(const pa_cache_desc_t* cache, const void* key, const void* value,
                                 void* k_pool, void* v_pool, const int32_t* slot_mapping,
                                 int32_t num_tokens, int32_t* err_flag, pa_stream_t stream);

/*
 * pa_copy_blocks - copy-on-write of shared blocks.
 *
 * For every pair, physical block dst becomes a bitwise copy of block src, for K and V and
 * all kv heads. A block shared by several sequences (beams) is copied before one of them
 * writes into it ([BlockManager essay] §2, §4.2; [KV Block course] §3.4). Pairs run in
 * parallel: every dst must be distinct and no dst may be a src (a fresh block is always the
 * target of copy-on-write). A pair with an id outside [0, num_blocks) or src == dst is
 * skipped and sets PA_FLAG_BAD_COPY_PAIR. num_pairs == 0 launches nothing. An 8-bit pool
 * returns PA_ERR_UNSUPPORTED (use pa_copy_blocks_fp8, which moves the scales too).
 */
pa_status_t pa_copy_blocks(const pa_cache_desc_t* cache, void* k_pool, void* v_pool,
                           const int32_t* pairs, int32_t num_pairs, int32_t* err_flag,
                           pa_stream_t stream);

/*
 * pa_decode_append - pa_reshape_and_cache of one new token per sequence followed by
 * pa_decode, fused: the decode takes the new rows straight from key/value.
 *
 * key/value: [batch][num_kv_heads][head_dim] (the new token of each sequence, 16-byte
 * aligned); slot_mapping: int32 [batch]. context_lens are the lengths after the append, so
 * the new token is at position context_lens[b] - 1. For a sequence with slot_mapping[b] >= 0
 * the decode reads the token's K and V rows from key/value, never from the pool, and the
 * rows are written to the slot ([BlockManager essay] §4.4; [Valid-length essay] §4.1: the
 * write lands at the valid length) by the decode workgroup that owns that position, as its
 * last act, or, when the launch has a reduce pass (some sequence spans several partitions),
 * by the reduce kernel after the decode. Afterwards the pool equals that of the two separate
 * calls bit for bit, and the output equals pa_decode's up to the order of the fp32 sums
 * (bit for bit on the matrix-core path). slot_mapping[b] < 0 appends nothing for that
 * sequence. A slot that is not the slot of position context_lens[b] - 1 through block_table
 * is not written and sets PA_FLAG_BAD_SLOT. A sequence with an invalid length or block id
 * gets NaN outputs, as in pa_decode; its row is written only if its length is valid and
 * every block id of the partition holding the new position is valid. The appended
 * block must not be shared with another sequence (copy it first, pa_copy_blocks). 8-bit
 * pools return PA_ERR_UNSUPPORTED (use pa_decode_append_fp8).
 * Everything else is as pa_decode.
 */
pa_status_t pa_decode_append(const pa_cache_desc_t* cache, void* out, const void* q, void* k_pool, void* v_pool,
                             const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                             const void* key, const void* value, const int32_t* slot_mapping,
                             int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                             pa_stream_t stream);

/*
 * pa_decode_append_noalloc - pa_decode_append for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * The same arguments and results as pa_decode_append, without the workspace: the partition
 * records and slot words live in a static device array of PA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends. The caller still passes
 * every input and output. A call whose pa_decode_workspace_bytes(cache, batch, num_q_heads,
 * max_context_len, partition_size) exceeds PA_NOALLOC_SCRATCH_BYTES returns
 * PA_ERR_SCRATCH_LIMIT and launches nothing. The call allocates and frees nothing (the
 * first call on a device looks up the array's address there once). Nothing in the scratch
 * needs to start at zero: every record the reduce pass reads is written by the same call's
 * decode. All calls on one GPU share its array, so calls that can overlap on one GPU (on
 * different streams without ordering between them) race and give undefined results.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64 << 20)
pa_status_t pa_decode_append_noalloc(const pa_cache_desc_t* cache, void* out, const void* q, void* k_pool,
                                     void* v_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                                     int32_t max_context_len, float scale, const void* key, const void* value,
                                     const int32_t* slot_mapping, int32_t partition_size, int32_t* err_flag,
                                     pa_stream_t stream);

/*
 * pa_decode_partition_size - the context-partition length pa_decode will use.
 *
 * `requested` > 0 must be a multiple of block_size covering at most 1024 blocks (else
 * returns -1). 0 picks a default from the batch, head and length shape. A result >=
 * max_context_len means one partition per sequence (no reduce pass).
 */
int32_t pa_decode_partition_size(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t requested);

/*
 * pa_decode_workspace_bytes - bytes of device workspace pa_decode needs (0 if none).
 *
 * The workspace holds one (max, sum, normalised output) record per sequence, query head
 * and context partition, and one int32 per sequence (pa_decode_append), when some sequence
 * spans more than one partition.
 */
size_t pa_decode_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_heads,
                                 int32_t max_context_len, int32_t partition_size);

/*
 * pa_decode - one query per sequence attends over its paged K/V cache.
 *
 * out[b][h] = sum_t softmax_t(scale * q[b][h] . K_b[t]) V_b[t] over the context_lens[b]
 * valid tokens of sequence b, where token t of kv head g = h / (num_q_heads / num_kv_heads)
 * is read from physical block block_table[b][t / block_size] at offset t % block_size
 * ([BlockManager essay] §2, §5.2; [KV Block course] §3.3; [Valid-length essay] §3.1, §4.2;
 * [CANN paging article] §2.2). Tokens at or past context_len are never loaded.
 * Scores, the running max and sum, and the accumulators are fp32; out has the pool dtype.
 *
 * max_context_len bounds every context_lens[b] and sizes the launch; it must not exceed
 * max_blocks_per_seq * block_size. A sequence whose length is <= 0 or above either bound
 * gets NaN outputs and sets PA_FLAG_EMPTY_CONTEXT / PA_FLAG_BAD_LENGTH; a sequence with a
 * bad block id in its valid range gets NaN outputs and sets PA_FLAG_BAD_BLOCK_ID. Other
 * sequences are unaffected.
 *
 * partition_size: 0 = default, else as pa_decode_partition_size. When a sequence spans
 * several partitions, each writes (max, sum, output) to `workspace` and a second kernel
 * combines them with a log-sum-exp weighting; workspace_bytes must be at least
 * pa_decode_workspace_bytes(...) (the workspace may be NULL when that is 0). A launch
 * holds at most 65535 partitions per sequence (max_context_len / partition size, rounded
 * up); more returns PA_ERR_UNSUPPORTED. An 8-bit pool returns PA_ERR_UNSUPPORTED (use
 * pa_decode_fp8).
 */
pa_status_t pa_decode(const pa_cache_desc_t* cache, void* out, const void* q, const void* k_pool,
                      const void* v_pool, const int32_t* block_table, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t batch, int32_t num_q_heads,
                      int32_t max_context_len, float scale, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, int32_t* err_flag,
                      pa_stream_t stream);

/*
 * pa_decode_sliding_window - decode over the last `window` tokens only.
 *
 * As pa_decode, but sequence b attends to tokens [max(0, L - window), L) where L =
 * context_lens[b]: the sliding-window cache policy that keeps only the most recent tokens
 * ([Valid-length essay] §3.3, §5.3). Blocks that lie wholly before the window are never read
 * or checked, so their table entries may already be released (-1). window >= L gives the
 * same result as pa_decode, bit for bit. window must be > 0 (else PA_ERR_INVALID_ARGUMENT).
 *
 * Partitions of a sequence start at the block that holds its first attended token, so the
 * launch and the workspace scale with the window, not with max_context_len: they are those
 * of pa_decode with max_context_len replaced by span = min(max_context_len, window +
 * block_size - 1). partition_size = 0 picks pa_decode_partition_size(cache, batch,
 * num_q_heads, span, 0); the workspace must hold
 * pa_decode_sliding_window_workspace_bytes(...) bytes (0: none needed).
 */
pa_status_t pa_decode_sliding_window(const pa_cache_desc_t* cache, void* out, const void* q,
                                     const void* k_pool, const void* v_pool, const int32_t* block_table,
                                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t max_context_len, float scale,
                                     int32_t window, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream);

/*
 * pa_decode_sliding_window_workspace_bytes - workspace bytes pa_decode_sliding_window needs
 * for these sizes and this partition_size (0 = the default policy); 0 when it needs none or
 * when an argument is invalid (then the decode call itself reports the error).
 */
size_t pa_decode_sliding_window_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch,
                                                int32_t num_q_heads, int32_t max_context_len, int32_t window,
                                                int32_t partition_size);

/*
 * pa_reshape_and_cache_fp8 - quantise new tokens' K and V into an 8-bit float pool.
 *
 * As pa_reshape_and_cache (same slots, padding and error rules), but each (token, kv head)
 * row x of key/value (type src_dtype: PA_F32, PA_F16 or PA_BF16) is stored as codes with
 * its own scale: a = max |x| over the row, s = a / 448, code = the E4M3 value nearest
 * x / s clamped to [-448, 448], ties to the even mantissa; all arithmetic is float32 with
 * correctly rounded division. A row of zeros stores s = 0 and codes 0. Rows must be finite.
 * The cache dtype must be PA_FP8_E4M3; k_scale and v_scale must be 4-byte aligned.
 */
pa_status_t pa_reshape_and_cache_fp8(const pa_cache_desc_t* cache, int32_t src_dtype, const void* key,
                                     const void* value, void* k_pool, void* v_pool, float* k_scale,
                                     float* v_scale, const int32_t* slot_mapping, int32_t num_tokens,
                                     int32_t* err_flag, pa_stream_t stream);

/*
 * pa_copy_blocks_fp8 - copy-on-write of 8-bit float blocks: as pa_copy_blocks, and every
 * copied row keeps its scale (k_scale / v_scale rows move with the codes).
 */
pa_status_t pa_copy_blocks_fp8(const pa_cache_desc_t* cache, void* k_pool, void* v_pool, float* k_scale,
                               float* v_scale, const int32_t* pairs, int32_t num_pairs, int32_t* err_flag,
                               pa_stream_t stream);

/*
 * pa_decode_fp8 - decode over an 8-bit float cache.
 *
 * The result of pa_decode (window = 0) or pa_decode_sliding_window (window > 0) over the
 * dequantised rows code * scale: K row t contributes scale * (q . codes_t) * k_scale_t to the
 * score, V row t adds its softmax weight times v_scale_t times codes_t. Codes widen exactly;
 * scores and accumulators are fp32. q_dtype (PA_F16 or PA_BF16) is the type of q and out.
 * Launch shape, partitions, workspace (pa_decode_workspace_bytes, or
 * pa_decode_sliding_window_workspace_bytes for a window) and error rules are those of the
 * unquantised calls. The cache dtype must be PA_FP8_E4M3, num_q_heads / num_kv_heads at
 * most 8 (or 16 with head_dim 64 or 128), and block_size >= 16 when head_dim is 64 unless
 * 4, 8 or 16 query heads per kv head run on the matrix cores (else PA_ERR_UNSUPPORTED).
 */
pa_status_t pa_decode_fp8(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                          const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                          const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                          int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale, int32_t window,
                          int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                          pa_stream_t stream);

/*
 * pa_decode_append_fp8 - pa_reshape_and_cache_fp8 of one new token per sequence followed by
 * pa_decode_fp8 (no window), fused as pa_decode_append is.
 *
 * key/value: [batch][num_kv_heads][head_dim] in q_dtype (PA_F16 or PA_BF16), 16-byte
 * aligned. The decode work-group that owns position context_lens[b] - 1 quantises the
 * token's rows exactly as pa_reshape_and_cache_fp8 does (scale = max |x| / 448, codes nearest
 * to x / scale; [BlockManager essay] §3 on quantised blocks), uses the codes and scales like
 * every other row, and writes them, with the two scales, to the slot as its last act. The
 * pool and scale arrays afterwards equal those of the two separate calls bit for bit, and the
 * output equals pa_decode_fp8's up to the order of the fp32 sums (bit for bit on the
 * matrix-core path). Slot checks, skipped slots, errors, shapes and workspace are those of
 * pa_decode_append and pa_decode_fp8.
 */
pa_status_t pa_decode_append_fp8(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                                 void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                 const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                                 int32_t batch, int32_t num_q_heads, int32_t max_context_len, float scale,
                                 const void* key, const void* value, const int32_t* slot_mapping,
                                 int32_t partition_size, void* workspace, size_t workspace_bytes, int32_t* err_flag,
                                 pa_stream_t stream);

/*
 * pa_decode_beams - pa_decode (or pa_decode_fp8) for batches of beam groups.
 *
 * Sequences g * beam_width .. g * beam_width + beam_width - 1 form group g (the last group
 * may be smaller): beams or parallel samples forked from one prompt, whose block tables
 * reference the same physical blocks for their common prefix ([BlockManager essay] §4.2,
 * reference counts; copy-on-write, pa_copy_blocks, gives each its own blocks where they
 * diverge). The output is that of pa_decode / pa_decode_fp8 on the same arguments, for every
 * sequence and any tables: grouping changes only how blocks are read. One work-group per (kv
 * head, group, partition) compares the group's table slices for the partition; where every
 * beam that reaches the partition lists the same ids for the blocks it reads, each block is
 * read once for all of them, else once per beam.
 *
 * Arguments as pa_decode_fp8 (q_dtype; k_scale/v_scale for PA_FP8_E4M3 pools, ignored for
 * 16-bit ones, whose q_dtype must equal the pool's dtype), without a window, plus beam_width
 * >= 1. Runs on the matrix cores: head_dim 64 or 128, num_q_heads / num_kv_heads in {1, 2, 4,
 * 8} with beam_width * that group <= 16, block_size >= 16 or 8, else PA_ERR_UNSUPPORTED. Errors
 * (status codes, err_flag bits, NaN rows of the affected sequence only) are those of
 * pa_decode. The partition length is pa_decode_beams_partition_size(...) and the workspace
 * must hold pa_decode_beams_workspace_bytes(...) (NULL when that is 0).
 */
pa_status_t pa_decode_beams(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                            const void* k_pool, const void* v_pool, const float* k_scale, const float* v_scale,
                            const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t batch, int32_t beam_width, int32_t num_q_heads, int32_t max_context_len,
                            float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                            int32_t* err_flag, pa_stream_t stream);

/*
 * Partition length pa_decode_beams uses: `requested` > 0 must be a multiple of block_size
 * with beam_width * requested / block_size <= 2048 (else -1); 0 picks a default.
 */
int32_t pa_decode_beams_partition_size(const pa_cache_desc_t* cache, int32_t batch, int32_t beam_width,
                                       int32_t num_q_heads, int32_t max_context_len, int32_t requested);

/* Workspace bytes pa_decode_beams needs (0: none, or an invalid argument). */
size_t pa_decode_beams_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t beam_width,
                                       int32_t num_q_heads, int32_t max_context_len, int32_t partition_size);

/*
 * pa_reblock - migrate a paged cache to another block size.
 *
 * A new block size invalidates every block table, so the contents move to the new layout
 * ([CANN paging article] §4.1). For every sequence b and token t < context_lens[b], the K
 * and V rows of every kv head are copied bit for bit from block src_table[b][t /
 * src->block_size], offset t % src->block_size, of (src_k, src_v) to block dst_table[b][t /
 * dst->block_size], offset t % dst->block_size, of (dst_k, dst_v). With 8-bit pools the row
 * scales move too (all four scale pointers non-NULL; else they must be NULL). Other slots of
 * the destination are not written.
 *
 * Both descriptors must agree on num_kv_heads, head_dim and dtype; block sizes, pool sizes
 * and strides may differ. The two caches must not overlap, and no two tokens may share a
 * destination slot (caller error: they race). A sequence with context_len <= 0 moves
 * nothing; context_len > max_context_len or past either table's width skips the sequence
 * and sets PA_FLAG_BAD_LENGTH; an id outside its pool skips that token and sets
 * PA_FLAG_BAD_BLOCK_ID.
 */
pa_status_t pa_reblock(const pa_cache_desc_t* src, const void* src_k, const void* src_v, const float* src_k_scale,
                       const float* src_v_scale, const int32_t* src_table, int32_t src_max_blocks_per_seq,
                       const pa_cache_desc_t* dst, void* dst_k, void* dst_v, float* dst_k_scale, float* dst_v_scale,
                       const int32_t* dst_table, int32_t dst_max_blocks_per_seq, const int32_t* context_lens,
                       int32_t batch, int32_t max_context_len, int32_t* err_flag, pa_stream_t stream);

/*
 * pa_multi_token_attention - several new query tokens per sequence over the paged cache.
 *
 * Sequence b owns query rows query_start[b] .. query_start[b+1]-1 of q and out
 * ([num_q_tokens][num_q_heads][head_dim]): its n_b new tokens (a prefill chunk, a round of
 * a multi-round conversation, or speculative tokens), whose K and V were already appended
 * (pa_reshape_and_cache*) so that context_lens[b] includes them ([Valid-length essay] §2.2).
 * Query i sits at position p = context_lens[b] - n_b + i and attends to tokens 0 .. p only,
 * the causal mask inside the valid range ([Valid-length essay] §4.2):
 *   out[row][h] = sum_{t <= p} softmax_t(scale * q[row][h] . K_b[t]) V_b[t].
 * n_b = 1 is pa_decode. query_start is int32 [batch + 1], non-decreasing from 0, with
 * query_start[batch] <= num_q_tokens; rows outside every sequence are not written.
 *
 * Runs on the matrix cores: dtype f16/bf16 (q_dtype equal to it) or PA_FP8_E4M3 (q f16/bf16,
 * k_scale/v_scale as in pa_decode_fp8); block_size >= 16, or 8 with head_dim 64 or 128 (a
 * 16-row tile then spans two blocks and each row looks up its own); num_q_heads / num_kv_heads in
 * {1, 2, 4, 8, 16} (16 only with head_dim <= 128); else PA_ERR_UNSUPPORTED. max_query_len
 * bounds every n_b and sizes the launch (batch * ceil(max_query_len * group / 16) <= 65535).
 * A sequence with n_b > context_len, a bad length or n_b > max_query_len sets
 * PA_FLAG_BAD_LENGTH (its rows NaN where the launch covers them); a bad block id sets
 * PA_FLAG_BAD_BLOCK_ID and poisons that sequence's rows. Partitions and workspace work as
 * for pa_decode; the workspace must hold pa_multi_token_workspace_bytes(...).
 */
pa_status_t pa_multi_token_attention(const pa_cache_desc_t* cache, int32_t q_dtype, void* out, const void* q,
                                     const void* k_pool, const void* v_pool, const float* k_scale,
                                     const float* v_scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, const int32_t* query_start, int32_t batch,
                                     int32_t num_q_tokens, int32_t num_q_heads, int32_t max_context_len,
                                     int32_t max_query_len, float scale, int32_t partition_size, void* workspace,
                                     size_t workspace_bytes, int32_t* err_flag, pa_stream_t stream);

/* Workspace bytes pa_multi_token_attention needs (0: none, or an invalid argument). */
size_t pa_multi_token_workspace_bytes(const pa_cache_desc_t* cache, int32_t batch, int32_t num_q_tokens,
                                      int32_t num_q_heads, int32_t max_context_len, int32_t max_query_len,
                                      int32_t partition_size);

/* Human-readable text for a status code (static storage). */
const char* pa_status_string(pa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
