// Multi-token paged attention (several new queries per sequence, causal inside the valid
// range) on the matrix cores: launchers of the kernel in pa_mfma_kernel.h with (query, head)
// columns, and the log-sum-exp combine of its partition records per query row.
#include "pa_mfma_kernel.h"

namespace pagedkv {

namespace {

// out[row] = sum_p w_p o_p / sum_p w_p over the partitions p that hold tokens the row's query
// sees (those at or before its position); rows of sequences with one partition were written
// by the attention kernel itself.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_multi_kernel(DecodeArgs a) {
    const int tok = blockIdx.x;
    const int h = blockIdx.y;
    const int e = threadIdx.x;
    int lo = 0, hi = a.batch - 1;  // the last sequence whose rows start at or before tok
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.query_start[mid] <= tok) lo = mid;
        else hi = mid - 1;
    }
    const int b = lo;
    const int q0 = a.query_start[b];
    const int nq = a.query_start[b + 1] - q0;
    const int group = a.num_q_heads / a.num_kv_heads;
    if (tok < q0 || tok >= q0 + nq || q0 + nq > a.num_q_tokens || nq * group > 16 * a.col_tiles) return;
    const int L = a.context_lens[b];
    if (L <= 0 || L > a.max_context_len || ((L - 1) >> a.log2_block_size) >= a.max_blocks_per_seq || L < nq) return;
    const int P = a.partition_size;
    if ((L + P - 1) / P <= 1) return;
    const int nparts = (L - nq + (tok - q0)) / P + 1;
    const size_t rec0 = ((size_t)tok * a.num_q_heads + h) * a.max_partitions;
    const float o = lse_combine<D>(a.ws_ml + rec0 * 2, a.ws_o + rec0 * D, nparts, e);
    store_elem(T{}, a.out, ((size_t)tok * a.num_q_heads + h) * D + e, o);
}

#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif

template <typename T, typename KV, int D, int G>
hipError_t launch_tdg(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    constexpr int NW = PA_MFMA_WAVES;
    dim3 grid(num_kv_heads, batch * a.col_tiles, a.max_partitions);
    hipLaunchKernelGGL((mfma::decode_mfma_kernel<T, KV, D, G, NW, (D <= 128), true>), grid, dim3(NW * 64), 0, stream,
                       a);
    return hipGetLastError();
}

template <typename T, typename KV, int D>
hipError_t launch_td(const DecodeArgs& a, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (group) {
        case 1: return launch_tdg<T, KV, D, 1>(a, batch, num_kv_heads, s);
        case 2: return launch_tdg<T, KV, D, 2>(a, batch, num_kv_heads, s);
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

template <typename T, int D>
hipError_t launch_reduce_td(const DecodeArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((reduce_multi_kernel<T, D>), dim3(a.num_q_tokens, a.num_q_heads), dim3(D), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_t(const DecodeArgs& a, int head_dim, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_reduce_td<T, 64>(a, s);
        case 128: return launch_reduce_td<T, 128>(a, s);
        case 256: return launch_reduce_td<T, 256>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool multi_token_supported(int kv_dtype, int head_dim, int group, int block_size) {
    return (kv_dtype == PA_F16 || kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3) &&
           (group == 1 || group == 2 || group == 4 || group == 8 || group == 16) && block_size >= 16 &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && !(group == 16 && head_dim == 256);
}

hipError_t launch_multi_token(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream) {
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

hipError_t launch_reduce_multi(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream) {
    switch (dtype) {
        case PA_F16: return launch_reduce_t<F16>(a, head_dim, stream);
        case PA_BF16: return launch_reduce_t<BF16>(a, head_dim, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
