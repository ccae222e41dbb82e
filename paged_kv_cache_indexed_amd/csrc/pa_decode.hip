// Paged-KV decode entry points for 16/32-bit pools (VALU kernels from pa_decode_valu.h) and
// the log-sum-exp reduce kernel that combines context partitions.
#include <algorithm>

#include "pa_decode_valu.h"

namespace pagedkv {

namespace {

// Log-sum-exp combine (lse_combine) of the per-partition records. One work-group covers
// query heads [h0, h0 + hpw) of one sequence, hpw = ceil(num_q_heads / gridDim.x): the
// launch sizes gridDim.x so that the grid has about 1024 work-groups, since most of them
// only read a length and leave (sequences with one partition were finished by the decode).
//
// Fused append: the work-group also writes the new K and V rows of the kv heads whose first
// query head it covers to the slot the decode checked (a.ws_slot). Written here, in a short
// burst after the decode, they cost far less than as scattered stores among the decode's
// reads.
constexpr int kReduceThreads = 256;
constexpr int kReduceGroups = 1024;

template <typename T, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(DecodeArgs a) {
    const int b = blockIdx.y;
    const int hpw = (a.num_q_heads + (int)gridDim.x - 1) / (int)gridDim.x;
    const int h0 = blockIdx.x * hpw;
    const int h1 = min(h0 + hpw, a.num_q_heads);
    // the length is read with the slot and the first rows: read after the row stores (which
    // the compiler cannot prove leave it alone), it would wait for them to be acknowledged
    const int L = a.context_lens[b];
    if (a.ws_slot) {
        constexpr int kRowVecs = D * T::kBytes / 16;
        const int group = a.num_q_heads / a.num_kv_heads;
        const int kv0 = (h0 + group - 1) / group;
        const int nvec = ((h1 + group - 1) / group - kv0) * 2 * kRowVecs;
        const int lbs = a.log2_block_size;
        // vector i: kv head kv0 + i / (2 kRowVecs), K row then V row
        auto src = [&](int i) {
            return static_cast<const char*>(((i / kRowVecs) & 1) ? a.new_value : a.new_key) +
                   ((size_t)b * a.num_kv_heads + kv0 + i / (2 * kRowVecs)) * D * T::kBytes + 16 * (i % kRowVecs);
        };
        // the first pass of rows is read in the same round trip as the slot
        const int tid = threadIdx.x;
        const u32x4 first = tid < nvec ? load16(src(tid)) : u32x4{0, 0, 0, 0};
        const int slot = a.ws_slot[b];
        if (slot >= 0) {
            auto dst = [&](int i) {
                return static_cast<char*>(const_cast<void*>(((i / kRowVecs) & 1) ? a.v_pool : a.k_pool)) +
                       (size_t)(slot >> lbs) * a.block_stride +
                       (((((size_t)kv0 + i / (2 * kRowVecs)) << lbs) + (slot & ((1 << lbs) - 1))) * D) * T::kBytes +
                       16 * (i % kRowVecs);
            };
            if (tid < nvec) store16(dst(tid), first);
            for (int i = tid + kReduceThreads; i < nvec; i += kReduceThreads) store16(dst(i), load16(src(i)));
        }
    }
    if (L <= 0 || L > a.max_context_len || (L - 1) >> a.log2_block_size >= a.max_blocks_per_seq) return;
    const int nparts = (L - partition_base(a, L) + a.partition_size - 1) / a.partition_size;
    if (nparts <= 1) return;
    for (int i = threadIdx.x; i < (h1 - h0) * D; i += kReduceThreads) {
        const int h = h0 + i / D;
        const int e = i % D;
        const size_t row = (size_t)b * a.num_q_heads + h;
        const size_t rec0 = row * a.max_partitions;
        store_elem(T{}, a.out, row * D + e, lse_combine<D>(a.ws_ml + rec0 * 2, a.ws_o + rec0 * D, nparts, e));
    }
}

template <typename T, int D>
hipError_t launch_reduce_td(const DecodeArgs& a, int batch, hipStream_t stream) {
    const int groups = std::min(a.num_q_heads, std::max(1, (kReduceGroups + batch - 1) / batch));
    hipLaunchKernelGGL((reduce_kernel<T, D>), dim3(groups, batch), dim3(kReduceThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_reduce_t(const DecodeArgs& a, int head_dim, int batch, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_reduce_td<T, 64>(a, batch, s);
        case 128: return launch_reduce_td<T, 128>(a, batch, s);
        case 256: return launch_reduce_td<T, 256>(a, batch, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_reduce(const DecodeArgs& a, int dtype, int head_dim, int batch, hipStream_t stream) {
    switch (dtype) {
        case PA_F32: return launch_reduce_t<F32>(a, head_dim, batch, stream);
        case PA_F16: return launch_reduce_t<F16>(a, head_dim, batch, stream);
        case PA_BF16: return launch_reduce_t<BF16>(a, head_dim, batch, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_valu(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream) {
    if (kv_dtype == PA_FP8_E4M3) return launch_decode_valu_fp8(a, dtype, head_dim, group, batch, num_kv_heads, stream);
    if (kv_dtype != dtype) return hipErrorInvalidValue;
    switch (dtype) {
        case PA_F32: return valu::launch_decode_t<F32, F32>(a, head_dim, group, batch, num_kv_heads, stream);
        case PA_F16: return valu::launch_decode_t<F16, F16>(a, head_dim, group, batch, num_kv_heads, stream);
        case PA_BF16: return valu::launch_decode_t<BF16, BF16>(a, head_dim, group, batch, num_kv_heads, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
