// Measurement aid: the streaming-read rate this device actually sustains, reported beside the
// nominal HBM peak so that a decode kernel's bandwidth can be read against both. It reads a
// buffer the way the decode kernels read K and V (16-byte non-temporal loads, each wave
// instruction covering 1 KiB of consecutive memory, several loads in flight per lane) and
// does nothing else. Not part of the attention path.
#include "../../include/pagedkv_measure.h"
#include "pa_device.h"

namespace pagedkv {
namespace {

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;  // 16-byte loads in flight per lane

// Work-group w reads vectors [w * chunk, ...) in steps of the whole grid's chunk: every
// iteration issues kStreamUnroll loads per lane before using any of them. The XOR of what a
// lane read is stored only if it equals a value no real buffer is likely to produce, which
// keeps the loads alive without a reduction; the store is one float per work-group at most.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* buf, size_t n16, float* sink) {
    constexpr size_t kChunk = (size_t)kStreamThreads * kStreamUnroll;
    const size_t stride = (size_t)gridDim.x * kChunk;
    uint32_t x = 0;
    size_t i = (size_t)blockIdx.x * kChunk + threadIdx.x;
    for (; i + (kStreamUnroll - 1) * kStreamThreads < n16; i += stride) {
        u32x4 v[kStreamUnroll];
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(buf + i + (size_t)u * kStreamThreads);
#pragma unroll
        for (int u = 0; u < kStreamUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n16; i += kStreamThreads) {  // the last partial chunk of this work-group
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (x == 0x9e3779b9u) sink[blockIdx.x] = __uint_as_float(x);
}

}  // namespace
}  // namespace pagedkv

extern "C" pa_status_t pa_measure_stream_read(const void* buf, size_t bytes, float* sink, int32_t num_workgroups,
                                              pa_stream_t stream) {
    if (!buf || !sink || bytes == 0 || (bytes & 15) != 0 || num_workgroups <= 0 || num_workgroups > (1 << 20))
        return PA_ERR_INVALID_ARGUMENT;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) != 0) return PA_ERR_INVALID_ARGUMENT;
    hipLaunchKernelGGL(pagedkv::stream_read_kernel, dim3(num_workgroups), dim3(pagedkv::kStreamThreads), 0,
                       (hipStream_t)stream, static_cast<const pagedkv::u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
