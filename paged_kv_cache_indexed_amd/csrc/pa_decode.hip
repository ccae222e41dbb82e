// Paged-KV decode entry points for 16/32-bit pools (VALU kernels from pa_decode_valu.h) and
// the log-sum-exp reduce kernel that combines context partitions.
#include "pa_decode_valu.h"

namespace pagedkv {

namespace {

// Log-sum-exp combine of the per-partition records of one (sequence, query head):
//   out = sum_p w_p o_p / sum_p w_p,  w_p = l_p * 2^(m_p - max_p m_p),
// where o_p is the partition's normalised output and (m_p, l_p) its base-2 running max and
// sum. A NaN sum (bad block in that partition) makes the whole output NaN.
//
// Fused append: the work-group of the first query head of each kv head also writes that kv
// head's new K and V rows to the slot the decode checked (a.ws_slot). Written here, in a
// short burst after the decode, they cost far less than as scattered stores among the
// decode's reads.
template <typename T, int D>
__global__ __launch_bounds__(D) void reduce_kernel(DecodeArgs a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int e = threadIdx.x;
    if (a.ws_slot) {
        const int group = a.num_q_heads / a.num_kv_heads;
        const int slot = a.ws_slot[b];
        if (h % group == 0 && slot >= 0) {
            constexpr int kRowVecs = D * T::kBytes / 16;
            const int kvh = h / group;
            const int lbs = a.log2_block_size;
            for (int i = e; i < 2 * kRowVecs; i += D) {
                const int which = i / kRowVecs;
                const int v = i % kRowVecs;
                const size_t row = ((size_t)b * a.num_kv_heads + kvh) * D * T::kBytes + 16 * v;
                char* dst = static_cast<char*>(const_cast<void*>(which ? a.v_pool : a.k_pool)) +
                            (size_t)(slot >> lbs) * a.block_stride +
                            ((((size_t)kvh << lbs) + (slot & ((1 << lbs) - 1))) * D) * T::kBytes + 16 * v;
                store16(dst, load16(static_cast<const char*>(which ? a.new_value : a.new_key) + row));
            }
        }
    }
    const int L = a.context_lens[b];
    if (L <= 0 || L > a.max_context_len || (L - 1) >> a.log2_block_size >= a.max_blocks_per_seq) return;
    const int nparts = (L - partition_base(a, L) + a.partition_size - 1) / a.partition_size;
    if (nparts <= 1) return;
    const size_t rec0 = ((size_t)b * a.num_q_heads + h) * a.max_partitions;
    const float* ml = a.ws_ml + rec0 * 2;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
    float num = 0.f, den = 0.f;
    for (int p = 0; p < nparts; ++p) {
        const float w = ml[2 * p + 1] * fast_exp2(ml[2 * p] - M);
        den += w;
        num = fmaf(w, a.ws_o[(rec0 + p) * D + e], num);
    }
    store_elem(T{}, a.out, ((size_t)b * a.num_q_heads + h) * D + e, num / den);
}

template <typename T, int D>
hipError_t launch_reduce_td(const DecodeArgs& a, int batch, hipStream_t stream) {
    hipLaunchKernelGGL((reduce_kernel<T, D>), dim3(a.num_q_heads, batch), dim3(D), 0, stream, a);
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
