// Beam-group decode on the gfx950 matrix cores: launchers of the kernel in pa_mfma_kernel.h
// with (beam, head) columns. Sequences forked from one prompt (beams, parallel samples)
// reference the same physical blocks for their common prefix ([BlockManager essay] §4.2);
// one workgroup per (kv head, group, partition) reads such a block once for every beam of the
// group instead of once per beam.
#include "pa_mfma_kernel.h"

namespace pagedkv {

namespace {

using mfma::decode_mfma_kernel;

constexpr int kBeamWaves = 4;

template <typename T, typename KV, int D, int G>
hipError_t launch_tdg(const DecodeArgs& a, int groups, int num_kv_heads, hipStream_t stream) {
    constexpr int NW = kBeamWaves;
    dim3 grid(num_kv_heads, groups, a.max_partitions);
    hipLaunchKernelGGL((decode_mfma_kernel<T, KV, D, G, NW, (D <= 128), false, true>), grid, dim3(NW * 64), 0,
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

bool decode_beams_supported(int kv_dtype, int head_dim, int group, int block_size, int beam_width) {
    return (kv_dtype == PA_F16 || kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) &&
           (head_dim == 64 || head_dim == 128) && (group == 1 || group == 2 || group == 4 || group == 8) &&
           (block_size >= 16 || (block_size == 8 && head_dim <= 128)) && beam_width >= 1 && beam_width * group <= 16;
}

hipError_t launch_decode_beams(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int groups,
                               int num_kv_heads, hipStream_t stream) {
    if (a.log2_block_size < 4)  // 8-token blocks: a block lookup per tile row
        return launch_decode_beams_small_blocks(a, kv_dtype, dtype, head_dim, group, groups, num_kv_heads, stream);
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
