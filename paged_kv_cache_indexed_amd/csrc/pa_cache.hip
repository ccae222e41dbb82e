// Cache maintenance kernels: append through a slot mapping, and copy-on-write of blocks.
// The plain append and the copy move raw 16-byte vectors, so they are bit-exact for every
// dtype; the 8-bit append quantises each row on the way in.
#include "pa_kernels.h"

namespace pagedkv {

namespace {

constexpr int kThreads = 256;

// One thread per 16-byte vector of one (token, kv head) row. Token i's row for head h goes
// to block slot / bs, offset slot % bs: the physical order inside a block is the logical
// order ([BlockManager essay] §4.4). Negative slots are padding tokens and are skipped
// ([Valid-length essay] §2.3); slots past the pool set PA_FLAG_BAD_SLOT and are skipped.
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(CacheArgs a, const char* key,
                                                                     const char* value,
                                                                     const int32_t* slot_mapping,
                                                                     int32_t num_tokens) {
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t per_token = (size_t)a.num_kv_heads * a.row_vecs;
    if (i >= per_token * (size_t)num_tokens) return;
    const int token = (int)(i / per_token);
    const int rem = (int)(i - (size_t)token * per_token);
    const int h = rem / a.row_vecs;
    const int v = rem - h * a.row_vecs;
    const int slot = slot_mapping[token];
    if (slot < 0) return;
    const int blk = slot >> a.log2_block_size;
    if (blk >= a.num_blocks) {
        if (rem == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_SLOT);
        return;
    }
    const int off = slot & ((1 << a.log2_block_size) - 1);
    const size_t dst = (size_t)blk * a.block_stride +
                       (((((size_t)h) << a.log2_block_size) + off) * a.row_vecs + v) * 16;
    store16(static_cast<char*>(a.k_pool) + dst, load16(key + i * 16));
    store16(static_cast<char*>(a.v_pool) + dst, load16(value + i * 16));
}

// Quantising append into 8-bit float pools. LPR = head_dim / 16 lanes own one (token, kv
// head) row, 16 elements each: the row's largest magnitude is a max over the lane group,
// the scale s = max / 448, and each element becomes the E4M3 code nearest x / s (clamped to
// +-448), so every code and scale is a float32 decision made exactly as the format and
// IEEE division define it. Lanes past the last row take part in the group max with 0.
template <typename S, int D>
__global__ __launch_bounds__(kThreads) void reshape_and_cache_fp8_kernel(CacheArgs a, const char* key,
                                                                         const char* value, float* k_scale,
                                                                         float* v_scale, const int32_t* slot_mapping,
                                                                         int32_t num_tokens) {
    constexpr int LPR = D / 16;
    constexpr int kSrcVecs = 16 * S::kBytes / 16;  // 16-byte source vectors per lane
    constexpr int kSrcElems = VecInfo<S>::kElems;
    const size_t gid = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const size_t rid = gid / LPR;  // (token, kv head) row
    const int col = (int)(gid % LPR);
    const bool in_range = rid < (size_t)num_tokens * a.num_kv_heads;
    const int token = in_range ? (int)(rid / a.num_kv_heads) : 0;
    const int h = in_range ? (int)(rid % a.num_kv_heads) : 0;
    const int slot = in_range ? slot_mapping[token] : -1;
    const int blk = slot >> a.log2_block_size;
    if (in_range && slot >= 0 && blk >= a.num_blocks && col == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_SLOT);
    const bool write = in_range && slot >= 0 && blk < a.num_blocks;
    const int off = slot & ((1 << a.log2_block_size) - 1);
    const size_t srow = write ? ((((size_t)blk * a.num_kv_heads + h) << a.log2_block_size) + off) : 0;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const char* src = (which == 0 ? key : value) + (rid * D + (size_t)col * 16) * S::kBytes;
        float x[16];
        float amax = 0.f;
        if (in_range) {
#pragma unroll
            for (int v = 0; v < kSrcVecs; ++v) unpack(S{}, load16(src + 16 * v), x + v * kSrcElems);
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
        }
        amax = group_max<LPR>(amax);
        if (!write) continue;
        const float sc = __fdiv_rn(amax, 448.f);
        u32x4 codes = {0u, 0u, 0u, 0u};
        if (sc != 0.f) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const float qv = fminf(fmaxf(__fdiv_rn(x[e], sc), -448.f), 448.f);
                codes[e >> 2] |= e4m3_encode(qv) << (8 * (e & 3));
            }
        }
        char* pool = static_cast<char*>(which == 0 ? a.k_pool : a.v_pool);
        const size_t row_in_block = ((size_t)h << a.log2_block_size) + off;
        store16(pool + (size_t)blk * a.block_stride + row_in_block * D + (size_t)col * 16, codes);
        if (col == 0) (which == 0 ? k_scale : v_scale)[srow] = sc;
    }
}

// Grid (pairs, chunks): chunk c of pair p copies vectors [c * kChunk, (c + 1) * kChunk) of
// block src to block dst in both pools; with 8-bit pools the vectors past the codes are
// the block's scale rows (block_vecs1 of them in k_scale / v_scale).
constexpr int kCopyVecsPerThread = 4;
constexpr int kCopyChunk = kThreads * kCopyVecsPerThread;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CacheArgs a, const int32_t* pairs, char* k_scale,
                                                               char* v_scale, size_t block_vecs1) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks || src == dst) {
        if (blockIdx.y == 0 && threadIdx.x == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_COPY_PAIR);
        return;
    }
    const size_t block_vecs0 = ((size_t)a.num_kv_heads * a.row_vecs) << a.log2_block_size;
    const size_t begin = (size_t)blockIdx.y * kCopyChunk;
    const char* kp = static_cast<const char*>(a.k_pool);
    const char* vp = static_cast<const char*>(a.v_pool);
    u32x4 kbuf[kCopyVecsPerThread], vbuf[kCopyVecsPerThread];
    auto addr = [&](size_t idx, int blk) -> size_t {  // byte offset of vector idx
        return idx < block_vecs0 ? (size_t)blk * a.block_stride + idx * 16
                                 : ((size_t)blk * block_vecs1 + (idx - block_vecs0)) * 16;
    };
    const size_t total = block_vecs0 + block_vecs1;
#pragma unroll
    for (int r = 0; r < kCopyVecsPerThread; ++r) {
        const size_t idx = begin + (size_t)r * kThreads + threadIdx.x;
        if (idx < total) {
            const bool codes = idx < block_vecs0;
            kbuf[r] = load16((codes ? kp : k_scale) + addr(idx, src));
            vbuf[r] = load16((codes ? vp : v_scale) + addr(idx, src));
        }
    }
#pragma unroll
    for (int r = 0; r < kCopyVecsPerThread; ++r) {
        const size_t idx = begin + (size_t)r * kThreads + threadIdx.x;
        if (idx < total) {
            const bool codes = idx < block_vecs0;
            store16((codes ? static_cast<char*>(a.k_pool) : k_scale) + addr(idx, dst), kbuf[r]);
            store16((codes ? static_cast<char*>(a.v_pool) : v_scale) + addr(idx, dst), vbuf[r]);
        }
    }
}

// Re-blocking. Grid (row chunks, sequences): thread i of sequence b moves 16-byte vector
// i % row_vecs of kv head (i / row_vecs) % heads of token i / (heads * row_vecs), for K and
// V, looking the token's block up in both tables; with 8-bit pools the thread holding a
// row's first vector also moves its two scales.
__global__ __launch_bounds__(kThreads) void reblock_kernel(ReblockArgs a) {
    const int b = blockIdx.y;
    const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
    const int L = a.context_lens[b];
    if (L <= 0) return;
    if (L > a.max_context_len || ((L - 1) >> a.src_log2_bs) >= a.src_mbs || ((L - 1) >> a.dst_log2_bs) >= a.dst_mbs) {
        if (i == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_LENGTH);
        return;
    }
    const size_t per_token = (size_t)a.num_kv_heads * a.row_vecs;
    const int t = (int)(i / per_token);
    if (t >= L) return;
    const int rem = (int)(i - (size_t)t * per_token);
    const int h = rem / a.row_vecs;
    const int v = rem - h * a.row_vecs;
    const int sid = a.src_table[(size_t)b * a.src_mbs + (t >> a.src_log2_bs)];
    const int did = a.dst_table[(size_t)b * a.dst_mbs + (t >> a.dst_log2_bs)];
    if ((unsigned)sid >= (unsigned)a.src_num_blocks || (unsigned)did >= (unsigned)a.dst_num_blocks) {
        if (v == 0 && h == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_BLOCK_ID);
        return;
    }
    const int soff = t & ((1 << a.src_log2_bs) - 1);
    const int doff = t & ((1 << a.dst_log2_bs) - 1);
    const size_t srow = ((size_t)h << a.src_log2_bs) + soff;  // row inside the block
    const size_t drow = ((size_t)h << a.dst_log2_bs) + doff;
    const size_t so = (size_t)sid * a.src_stride + (srow * a.row_vecs + v) * 16;
    const size_t dof = (size_t)did * a.dst_stride + (drow * a.row_vecs + v) * 16;
    const u32x4 kv = load16(a.src_k + so);
    const u32x4 vv = load16(a.src_v + so);
    store16(a.dst_k + dof, kv);
    store16(a.dst_v + dof, vv);
    if (a.src_ks && v == 0) {
        const size_t ss = ((size_t)sid * a.num_kv_heads << a.src_log2_bs) + srow;
        const size_t ds = ((size_t)did * a.num_kv_heads << a.dst_log2_bs) + drow;
        a.dst_ks[ds] = a.src_ks[ss];
        a.dst_vs[ds] = a.src_vs[ss];
    }
}

template <typename S>
hipError_t launch_fp8_append_s(const CacheArgs& a, int head_dim, const void* key, const void* value, float* k_scale,
                               float* v_scale, const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream,
                               size_t blocks) {
    auto k = reshape_and_cache_fp8_kernel<S, 128>;
    switch (head_dim) {
        case 64: k = reshape_and_cache_fp8_kernel<S, 64>; break;
        case 128: break;
        case 256: k = reshape_and_cache_fp8_kernel<S, 256>; break;
        default: return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL(k, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a, static_cast<const char*>(key),
                       static_cast<const char*>(value), k_scale, v_scale, slot_mapping, num_tokens);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_and_cache(const CacheArgs& a, const void* key, const void* value,
                                    const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
    const size_t total = (size_t)num_tokens * a.num_kv_heads * a.row_vecs;
    const size_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a,
                       static_cast<const char*>(key), static_cast<const char*>(value), slot_mapping, num_tokens);
    return hipGetLastError();
}

hipError_t launch_copy_blocks(const CacheArgs& a, const int32_t* pairs, int32_t num_pairs, float* k_scale,
                              float* v_scale, hipStream_t stream) {
    const size_t block_vecs0 = ((size_t)a.num_kv_heads * a.row_vecs) << a.log2_block_size;
    // scale rows: num_kv_heads * block_size floats per block, block_size >= 8
    const size_t block_vecs1 = k_scale ? ((size_t)a.num_kv_heads << a.log2_block_size) / 4 : 0;
    const size_t chunks = (block_vecs0 + block_vecs1 + kCopyChunk - 1) / kCopyChunk;
    if (chunks > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, (unsigned)chunks), dim3(kThreads), 0, stream, a, pairs,
                       reinterpret_cast<char*>(k_scale), reinterpret_cast<char*>(v_scale), block_vecs1);
    return hipGetLastError();
}

hipError_t launch_reblock(const ReblockArgs& a, int batch, hipStream_t stream) {
    const size_t threads = (size_t)a.max_context_len * a.num_kv_heads * a.row_vecs;
    const size_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff || batch > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(reblock_kernel, dim3((unsigned)blocks, (unsigned)batch), dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const CacheArgs& a, int src_dtype, int head_dim, const void* key,
                                        const void* value, float* k_scale, float* v_scale,
                                        const int32_t* slot_mapping, int32_t num_tokens, hipStream_t stream) {
    const size_t threads = (size_t)num_tokens * a.num_kv_heads * (head_dim / 16);
    const size_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    switch (src_dtype) {
        case PA_F32:
            return launch_fp8_append_s<F32>(a, head_dim, key, value, k_scale, v_scale, slot_mapping, num_tokens,
                                            stream, blocks);
        case PA_F16:
            return launch_fp8_append_s<F16>(a, head_dim, key, value, k_scale, v_scale, slot_mapping, num_tokens,
                                            stream, blocks);
        case PA_BF16:
            return launch_fp8_append_s<BF16>(a, head_dim, key, value, k_scale, v_scale, slot_mapping, num_tokens,
                                             stream, blocks);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
