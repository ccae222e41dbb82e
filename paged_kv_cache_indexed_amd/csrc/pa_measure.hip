// Measurement aids, not part of the attention path. The streaming-read rate this device
// actually sustains, reported beside the nominal HBM peak so that a decode kernel's bandwidth
// can be read against both: a buffer read the way the decode kernels read K and V (16-byte
// non-temporal loads, each wave instruction covering 1 KiB of consecutive memory, several
// loads in flight per lane) and nothing else. And the gather rate of a paged cache: the split
// decode's own reads of K and V through the block table, in its own decomposition, without
// the attention arithmetic.
#include "../../include/pagedkv_measure.h"
#include "pa_device.h"
#include "pa_kernels.h"

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

// The decode's reads without its arithmetic: work-group (kv head, sequence), 4 waves. It
// checks the length, stages the sequence's table row in LDS (ids outside the pool read
// nothing), and deals groups of rows to the waves round-robin as the split decode does: a
// wave load is 1 KiB of consecutive rows of one block (64 / (row_bytes / 16) rows), K and V
// through buffer resources over the (block, kv head) slab, rows past the length masked by
// an out-of-range offset. kGatherUnroll groups per wave are in flight at a time.
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;
constexpr int kGatherMaxIds = 4096;

__global__ __launch_bounds__(kGatherThreads) void gather_read_kernel(GatherReadArgs a) {
    __shared__ int s_ids[kGatherMaxIds];
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int L = a.context_lens[b];
    const int lbs = a.log2_block_size;
    const int bs = 1 << lbs;
    const int nids = L > 0 ? ((L - 1) >> lbs) + 1 : 0;
    if (L <= 0 || L > a.max_context_len || nids > a.max_blocks_per_seq || nids > kGatherMaxIds) return;
    for (int i = threadIdx.x; i < nids; i += kGatherThreads) {
        const int id = a.block_table[(size_t)b * a.max_blocks_per_seq + i];
        s_ids[i] = (unsigned)id < (unsigned)a.num_blocks ? id : -1;
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int lpr = a.row_bytes / 16;  // lanes per row
    const int rpl = 64 / lpr;          // rows per wave load
    const int row = lane / lpr;
    const int col = lane % lpr;
    const uint32_t slab = (uint32_t)bs * (uint32_t)a.row_bytes;
    const int ngroups = (L + rpl - 1) / rpl;
    uint32_t x = 0;
    for (int g = wave; g < ngroups; g += 4 * kGatherUnroll) {
        u32x4 kk[kGatherUnroll], vv[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const int gg = g + 4 * u;
            const int tok = gg * rpl;
            const int id = __builtin_amdgcn_readfirstlane(s_ids[(gg < ngroups ? tok : 0) >> lbs]);
            const size_t base = (size_t)(id < 0 ? 0 : id) * a.block_stride + (size_t)kvh * slab;
            const bool live = gg < ngroups && id >= 0 && tok + row < L;
            const uint32_t off = live ? (uint32_t)((((tok & (bs - 1)) + row) * a.row_bytes) + col * 16) : kOutOfRange;
            kk[u] = buffer_load16(make_rsrc(a.k_pool + base, slab), off);
            vv[u] = buffer_load16(make_rsrc(a.v_pool + base, slab), off);
        }
        // every dword of every load feeds x: with some unused the compiler narrows the loads
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u)
            x ^= kk[u][0] ^ kk[u][1] ^ kk[u][2] ^ kk[u][3] ^ vv[u][0] ^ vv[u][1] ^ vv[u][2] ^ vv[u][3];
    }
    if (x == 0x9e3779b9u) a.sink[(size_t)b * gridDim.x + kvh] = __uint_as_float(x);
}

}  // namespace

hipError_t launch_gather_read(const GatherReadArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    hipLaunchKernelGGL(gather_read_kernel, dim3(num_kv_heads, batch), dim3(kGatherThreads), 0, stream, a);
    return hipGetLastError();
}

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
