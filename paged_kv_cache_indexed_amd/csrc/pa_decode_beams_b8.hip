// Beam-group decode over 8-token blocks: the beam-group kernel of pa_mfma_kernel.h with a
// block lookup per tile row (a 16-row tile spans two blocks). Beams share prefix blocks by
// reference counts ([BlockManager essay] §4.2); the block size trade-off is §3 there.
#include "pa_mfma_kernel.h"

namespace pagedkv {

namespace {

constexpr int kBeamWaves = 4;

template <typename T, typename KV, int D, int G>
hipError_t launch_tdg(const DecodeArgs& a, int groups, int num_kv_heads, hipStream_t stream) {
    constexpr int NW = kBeamWaves;
    dim3 grid(num_kv_heads, groups, a.max_partitions);
    // 16-bit rows of 128 dims in a pool within 2 GiB: one buffer over the tile's two blocks
    // (mode 2, two waves per SIMD); else per-lane row addresses (mode 1)
    if constexpr (KV::kBytes == 2 && D == 128) {
        if (mfma::pool_within_2gib(a)) {
            hipLaunchKernelGGL((mfma::decode_mfma_kernel<T, KV, D, G, NW, true, false, true, 2>), grid, dim3(NW * 64), 0,
                               stream, a);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((mfma::decode_mfma_kernel<T, KV, D, G, NW, true, false, true, 1>), grid, dim3(NW * 64), 0,
                       stream, a);
    return hipGetLastError();
}

template <typename T, typename KV, int D>
hipError_t launch_td(const DecodeArgs& a, int group, int groups, int num_kv_heads, hipStream_t s) {
    switch (group) {
        case 1: return launch_tdg<T, KV, D, 1>(a, groups, num_kv_heads, s);
        case 2: return launch_tdg<T, KV, D, 2>(a, groups, num_kv_heads, s);
        case 4: return launch_tdg<T, KV, D, 4>(a, groups, num_kv_heads, s);
        case 8: return launch_tdg<T, KV, D, 8>(a, groups, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename KV>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int group, int groups, int num_kv_heads, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_td<T, KV, 64>(a, group, groups, num_kv_heads, s);
        case 128: return launch_td<T, KV, 128>(a, group, groups, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_decode_beams_small_blocks(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group,
                                            int groups, int num_kv_heads, hipStream_t stream) {
    if (a.log2_block_size != 3) return hipErrorInvalidValue;
    if (kv_dtype == PA_FP8_E4M3) {
        switch (dtype) {
            case PA_F16: return launch_t<F16, FP8>(a, head_dim, group, groups, num_kv_heads, stream);
            case PA_BF16: return launch_t<BF16, FP8>(a, head_dim, group, groups, num_kv_heads, stream);
            default: return hipErrorInvalidValue;
        }
    }
    if (kv_dtype != dtype) return hipErrorInvalidValue;
    switch (dtype) {
        case PA_F16: return launch_t<F16, F16>(a, head_dim, group, groups, num_kv_heads, stream);
        case PA_BF16: return launch_t<BF16, BF16>(a, head_dim, group, groups, num_kv_heads, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
