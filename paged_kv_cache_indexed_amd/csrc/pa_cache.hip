// Cache maintenance kernels: append through a slot mapping, and copy-on-write of blocks.
// Both move raw 16-byte vectors, so they are bit-exact for every dtype.
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
    const size_t dst = ((((size_t)blk * a.num_kv_heads + h) << a.log2_block_size) + off) * a.row_vecs + v;
    store16(static_cast<char*>(a.k_pool) + dst * 16, load16(key + i * 16));
    store16(static_cast<char*>(a.v_pool) + dst * 16, load16(value + i * 16));
}

// Grid (pairs, chunks): chunk c of pair p copies vectors [c * kChunk, (c + 1) * kChunk) of
// block src to block dst in both pools.
constexpr int kCopyVecsPerThread = 4;
constexpr int kCopyChunk = kThreads * kCopyVecsPerThread;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(CacheArgs a, const int32_t* pairs) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks || src == dst) {
        if (blockIdx.y == 0 && threadIdx.x == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_COPY_PAIR);
        return;
    }
    const size_t block_vecs = ((size_t)a.num_kv_heads * a.row_vecs) << a.log2_block_size;
    const size_t begin = (size_t)blockIdx.y * kCopyChunk;
    const char* ks = static_cast<const char*>(a.k_pool) + (size_t)src * block_vecs * 16;
    const char* vs = static_cast<const char*>(a.v_pool) + (size_t)src * block_vecs * 16;
    char* kd = static_cast<char*>(a.k_pool) + (size_t)dst * block_vecs * 16;
    char* vd = static_cast<char*>(a.v_pool) + (size_t)dst * block_vecs * 16;
    u32x4 kbuf[kCopyVecsPerThread], vbuf[kCopyVecsPerThread];
#pragma unroll
    for (int r = 0; r < kCopyVecsPerThread; ++r) {
        const size_t idx = begin + (size_t)r * kThreads + threadIdx.x;
        if (idx < block_vecs) {
            kbuf[r] = load16(ks + idx * 16);
            vbuf[r] = load16(vs + idx * 16);
        }
    }
#pragma unroll
    for (int r = 0; r < kCopyVecsPerThread; ++r) {
        const size_t idx = begin + (size_t)r * kThreads + threadIdx.x;
        if (idx < block_vecs) {
            store16(kd + idx * 16, kbuf[r]);
            store16(vd + idx * 16, vbuf[r]);
        }
    }
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

hipError_t launch_copy_blocks(const CacheArgs& a, const int32_t* pairs, int32_t num_pairs, hipStream_t stream) {
    const size_t block_vecs = ((size_t)a.num_kv_heads * a.row_vecs) << a.log2_block_size;
    const size_t chunks = (block_vecs + kCopyChunk - 1) / kCopyChunk;
    if (chunks > 65535) return hipErrorInvalidValue;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, (unsigned)chunks), dim3(kThreads), 0, stream, a, pairs);
    return hipGetLastError();
}

}  // namespace pagedkv
