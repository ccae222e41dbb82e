// Grouped-query paged decode on the gfx950 matrix cores for 8-token blocks: a 16-row operand
// tile then spans two blocks, so the kernel of pa_mfma_kernel.h looks up the block of each
// tile row. The block size trade-off (smaller blocks waste less memory,
// at more table lookups) is [BlockManager essay] §3.
#include "pa_mfma_lds.h"

namespace pagedkv {

namespace {

using mfma::decode_mfma_kernel;

constexpr int kSmallWaves = 4;

template <typename T, typename KV, int D, int G>
hipError_t launch_tdg(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    constexpr int NW = kSmallWaves;
    dim3 grid(num_kv_heads, batch, a.max_partitions);
    // 16-bit rows of 128 dims, up to 8 heads per kv head: the LDS path, whose load
    // instructions cover four rows of one block each
    if constexpr (std::is_same_v<KV, T> && D == 128 && G <= 8) return mfma::launch_decode_lds<T, G>(a, batch, num_kv_heads, stream);
    // 16-bit rows of 128 dims in a pool within 2 GiB: the tile's two blocks through one buffer
    // (mode 2), which keeps two waves per SIMD; per-lane row addresses (mode 1) need the
    // registers of a second wave there. Measured with 8 query heads per kv head (bf16): B = 128
    // at 2049 tokens 200 against 216 us, B = 256 at 257 tokens 82 against 111 us, B = 32 at
    // 2049 tokens 55 against 54 us.
    if constexpr (KV::kBytes == 2 && D == 128) {
        if (mfma::pool_within_2gib(a)) {
            hipLaunchKernelGGL((decode_mfma_kernel<T, KV, D, G, NW, true, false, false, 2>), grid, dim3(NW * 64), 0,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((decode_mfma_kernel<T, KV, D, G, NW, true, false, false, 1>), grid, dim3(NW * 64), 0, stream,
                       a);
    return hipGetLastError();
}

template <typename T, typename KV, int D>
hipError_t launch_td(const DecodeArgs& a, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (group) {
        case 4: return launch_tdg<T, KV, D, 4>(a, batch, num_kv_heads, s);
        case 8: return launch_tdg<T, KV, D, 8>(a, batch, num_kv_heads, s);
        case 16: return launch_tdg<T, KV, D, 16>(a, batch, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename KV>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_td<T, KV, 64>(a, group, batch, num_kv_heads, s);
        case 128: return launch_td<T, KV, 128>(a, group, batch, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_mfma_small_blocks(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group,
                                           int batch, int num_kv_heads, hipStream_t stream) {
    if (a.log2_block_size != 3) return hipErrorInvalidValue;
    if (kv_dtype == PA_FP8_E4M3) {
        switch (dtype) {
            case PA_F16: return launch_t<F16, FP8>(a, head_dim, group, batch, num_kv_heads, stream);
            case PA_BF16: return launch_t<BF16, FP8>(a, head_dim, group, batch, num_kv_heads, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (kv_dtype != dtype) return hipErrorInvalidValue;
    switch (dtype) {
        case PA_F16: return launch_t<F16, F16>(a, head_dim, group, batch, num_kv_heads, stream);
        case PA_BF16: return launch_t<BF16, BF16>(a, head_dim, group, batch, num_kv_heads, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
