// Grouped-query paged decode on the gfx950 matrix cores: launchers of the kernels in
// pa_mfma_kernel.h and pa_mfma_lds.h with one query per sequence (the columns are the
// group's heads).
#include "pa_mfma_lds.h"

namespace pagedkv {

namespace {

using mfma::decode_mfma_kernel;

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif

template <typename T, typename KV, int D, int G>
hipError_t launch_tdg(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    constexpr int NW = PA_MFMA_WAVES;
    dim3 grid(num_kv_heads, batch, a.max_partitions);
    // 16-bit rows of 128 dims and up to 8 heads per kv head: the LDS path (faster on every
    // shape measured, short contexts included)
    if constexpr (std::is_same_v<KV, T> && D == 128 && G <= 8) return mfma::launch_decode_lds<T, G>(a, batch, num_kv_heads, stream);
    hipLaunchKernelGGL((decode_mfma_kernel<T, KV, D, G, NW, (D <= 128)>), grid, dim3(NW * 64), 0, stream, a);
    return hipGetLastError();
}

template <typename T, typename KV, int D>
hipError_t launch_td(const DecodeArgs& a, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (group) {
        case 4: return launch_tdg<T, KV, D, 4>(a, batch, num_kv_heads, s);
        case 8: return launch_tdg<T, KV, D, 8>(a, batch, num_kv_heads, s);
        case 16:
            if constexpr (D <= 128) return launch_tdg<T, KV, D, 16>(a, batch, num_kv_heads, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename KV>
hipError_t launch_t(const DecodeArgs& a, int head_dim, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_td<T, KV, 64>(a, group, batch, num_kv_heads, s);
        case 128: return launch_td<T, KV, 128>(a, group, batch, num_kv_heads, s);
        case 256: return launch_td<T, KV, 256>(a, group, batch, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool decode_mfma_supported(int kv_dtype, int head_dim, int group, int block_size) {
    return (kv_dtype == PA_F16 || kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) &&
           (group == 4 || group == 8 || group == 16) && (block_size >= 16 || (block_size == 8 && head_dim <= 128)) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && !(group == 16 && head_dim == 256);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream) {
    if (a.log2_block_size < 4)
        return launch_decode_mfma_small_blocks(a, kv_dtype, dtype, head_dim, group, batch, num_kv_heads, stream);
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
