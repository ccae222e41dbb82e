// VALU paged-KV decode over 8-bit float (OCP E4M3) pools with a scale per row: the
// instantiations of pa_decode_valu.h for FP8 storage and fp16/bf16 queries.
#include "pa_decode_valu.h"

namespace pagedkv {

hipError_t launch_decode_valu_fp8(const DecodeArgs& a, int dtype, int head_dim, int group, int batch,
                                  int num_kv_heads, hipStream_t stream) {
    switch (dtype) {
        case PA_F16: return valu::launch_decode_t<F16, FP8>(a, head_dim, group, batch, num_kv_heads, stream);
        case PA_BF16: return valu::launch_decode_t<BF16, FP8>(a, head_dim, group, batch, num_kv_heads, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pagedkv
