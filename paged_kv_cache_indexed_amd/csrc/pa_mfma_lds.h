#pragma once
// Grouped-query paged decode (one query per sequence, 16-bit pools, head_dim 128, G <= 8 query
// heads per kv head) with K/V tiles brought to LDS by direct-to-LDS buffer loads.
//
// The matrix-core decode of pa_mfma_kernel.h loads its tiles straight into the MFMA operand
// layout: each load instruction covers a 64-byte strip of 16 rows, which the L1 serves one
// lane at a time. Here each wave stages one 16-token tile at a time in LDS, filled by
// buffer_load_dwordx4 ... lds: every load instruction reads four whole rows (1 KiB of
// consecutive memory) and needs no registers, and the other waves of the compute unit (two
// to four per SIMD) keep loads in flight while a wave computes. Per tile and wave:
//   * Loads. Instruction i of the K tile gives lane l row r = 4i + l / 16; the hardware
//     writes lane l's 16 bytes to position l % 16 of the row in LDS, so the lane fetches the
//     row's 16-byte chunk (l % 16) ^ r: chunk j of row r sits at position j ^ r. (XOR keeps each
//     quad of lanes inside one aligned 64-byte segment, so the loads stay coalesced.) V rows
//     put chunk j at j ^ (2r mod 16). Each instruction's four rows lie in one block (blocks
//     hold a multiple of 8 tokens) and it takes that block's id. A row outside the attended
//     range gets an out-of-range offset: no memory access, and the hardware writes zeros to
//     its LDS slot.
//   * Scores. S^T = K Q^T with v_mfma_f32_16x16x32: lane (n, g) reads chunk 4c + g of row n
//     (dims 32c + 8g .. +7) as the A operand of k-block c, from position (4c + g) ^ n: the 16
//     rows of a lane group hit distinct banks. Q is the B operand with the same dims.
//   * P V with v_mfma_f32_16x16x16: lane (n, g) holds the weights of head n at tokens
//     4g .. 4g+3, which is its A operand (k-slots 4g .. 4g+3), split into rounded high and low
//     parts as in the other matrix-core paths. The B operand (dim 16s + n at tokens 4g..4g+3)
//     comes from one ds_read_b64_tr_b16 per 16-dim slice: in each 16-lane group, lane i
//     receives element i % 4 of the 8-byte pieces that lanes i / 4 + 4k (k = 0..3) address, so
//     lane n addresses row 4g + n / 4, dims 16s + 4 (n % 4) .. +3.
//   * After the last tile the work-group meets at a barrier and the waves' softmax states are
//     merged through the tile buffers' memory: 8 KiB of LDS per wave in all (plus the table
//     slice), so two 8-wave or four 4-wave work-groups fit a compute unit.
// Measured against the direct-load kernel (bf16, 8 kv heads of 8 query heads, decode launch):
// B = 32 at 2049 tokens 45.2 against 48.7-54.3 us, B = 128 at 2049 173.8 against 186.5, B = 8
// at 32769 194.5 against 210.2, B = 256 at 129 tokens (4 waves) 32.6 against 48.2 us. Keeping
// two or four tiles per wave in flight instead (a ring of distinct LDS arrays, one work-group
// per compute unit) measured 46.9-48.4 us at B = 32, 2049 tokens: more bytes in flight per
// wave, fewer waves, slower.
// Everything else (length and table checks in the prologue, the base-2 online softmax with
// the lazy rescale, the wave merge and the records for the log-sum-exp reduce, the fused
// append) is the decode's.
#include "pa_mfma_kernel.h"

namespace pagedkv {
namespace mfma {

constexpr int kLdsTileVecs = 2 * 16 * 16;  // 16-byte vectors per tile buffer: 16 K rows, 16 V rows

#define PA_LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Byte address in LDS of a pointer to a __shared__ object (the low half of its flat address).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)reinterpret_cast<uintptr_t>(p); }

// Registers for four waves per SIMD (at most 128 per lane): two 8-wave or four 4-wave
// work-groups per compute unit, as many as the LDS allows.
template <typename T, int G, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(4))) void decode_mfma_lds_kernel(DecodeArgs a) {
    static_assert(T::kBytes == 2 && G >= 1 && G <= 8, "16-bit pools, at most 8 heads per kv head");
    constexpr int D = 128;
    constexpr int NC = D / 32;  // k-blocks of the score contraction
    constexpr int NS = D / 16;  // 16-dim output slices
    constexpr int kRowBytes = D * 2;
    using M = Mma<T>;

    __shared__ u32x4 s_tile[NW][kLdsTileVecs];
    __shared__ int s_ids[kMaxIdsPerPartition];
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    // the waves' weighted sums, merged after the loop, in the tile buffers' memory
    static_assert(sizeof(float) * G * D <= sizeof(u32x4) * kLdsTileVecs, "one wave's sums fit its tile");
    float (*const s_acc)[G][D] = reinterpret_cast<float (*)[G][D]>(&s_tile[0][0]);
    __shared__ __align__(16) char s_new[NewRec<T, D>::kBytes];

    const int p = grid_partition();
    const int kvh = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int lbs = a.log2_block_size;
    const int bs = 1 << lbs;

    if (partition_is_dead(a, p, b)) return;
    // Q as the B operand (zero beyond G): k-block c of lane group g holds dims 32c + 8g .. +7
    const bool col_valid = n < G;
    u32x4 qb[NC];
    {
        const char* qrow = static_cast<const char*>(a.q) + ((size_t)b * a.num_q_heads + kvh * G + (col_valid ? n : 0)) * D * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) qb[c] = col_valid ? load16(qrow + 2 * (32 * c + 8 * g)) : u32x4{0, 0, 0, 0};
    }
    Partition part;
    if (!partition_prologue<T, D, G, NW * 64>(a, p, kvh, b, s_ids, part, s_new)) return;
    const int ntok = part.ntok;
    const int rel_lo = part.rel_lo;
    const int npos = part.npos;
    const int tile0 = rel_lo >> 4;                    // first tile holding an attended token
    const int ntiles = ((ntok + 15) >> 4) - tile0;    // tiles of the partition from there
    const int nt = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;  // this wave's: tile0 + wave + NW k

    const size_t head_bytes = (size_t)bs * kRowBytes;
    const char* kpool = static_cast<const char*>(a.k_pool);
    const char* vpool = static_cast<const char*>(a.v_pool);
    auto vswz = [](int r) { return (2 * r) & 15; };

    // Loads of this wave's tile k into buf. Instruction i reads
    // rows 4i .. 4i+3 of the tile, which lie in one block: its id is looked up for the
    // instruction (clamped to the last attended row, so the entry is one the prologue staged).
    auto issue = [&](int k, u32x4* buf) {
        const int rel = (tile0 + wave + NW * k) << 4;  // wave-uniform
        const int pos = lane & 15;
        // attended rows of the tile: [lo, lo + span) relative to rel (one unsigned compare per
        // row and selects rather than branches: a load under a lane branch would leave the
        // compiler's wait counts unsure of what is outstanding)
        const int lo = rel_lo - rel;
        const uint32_t span = (uint32_t)(ntok - rel_lo);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int id = __builtin_amdgcn_readfirstlane(s_ids[min(rel + 4 * i, ntok - 1) >> lbs]);
            const size_t slab = (size_t)id * a.block_stride + (size_t)kvh * head_bytes;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + slab, (uint32_t)head_bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vpool + slab, (uint32_t)head_bytes);
            const int r = 4 * i + (lane >> 4);
            const bool live = (uint32_t)(r - lo) < span;
            const uint32_t row = (uint32_t)((((rel + 4 * i) & (bs - 1)) + (lane >> 4)) * kRowBytes);
            const uint32_t ok = live ? row + 16u * (uint32_t)(pos ^ r) : kOutOfRange;
            const uint32_t ov = live ? row + 16u * (uint32_t)(pos ^ vswz(r)) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, PA_LDS_PTR(buf + 64 * i), 16, ok, 0, 0, PA_KV_LOAD_POLICY);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, PA_LDS_PTR(buf + 256 + 64 * i), 16, ov, 0, 0,
                                                     PA_KV_LOAD_POLICY);
        }
    };

    float m = -INFINITY;  // running base-2 max of head n (same in all four lane groups)
    float l = 0.f;        // this lane's part of head n's running sum
    f32x4 acc[NS];        // acc[s][i] = O[head 4g + i][dim 16s + n]
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int k, u32x4* buf) {
        const int rel0 = (tile0 + wave + NW * k) << 4;
        if (npos >= 0) {  // fused append: the new token's rows replace its slot's (wave-uniform test)
            const int d = npos - rel0;
            if (d >= 0 && d < 16 && lane < 16) {
                buf[16 * d + (lane ^ d)] = *reinterpret_cast<const u32x4*>(s_new + 16 * lane);
                buf[256 + 16 * d + (lane ^ vswz(d))] = *reinterpret_cast<const u32x4*>(s_new + kRowBytes + 16 * lane);
            }
        }
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) st = M::k32(buf[16 * n + ((4 * c + g) ^ n)], qb[c], st);
        float sc[4];
        if (rel0 >= rel_lo && rel0 + 16 <= ntok) {  // the whole tile is attended (wave-uniform)
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = st[i] * a.scale_log2;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = rel0 + 4 * g + i;
                sc[i] = (tok < ntok && tok >= rel_lo) ? st[i] * a.scale_log2 : -INFINITY;
            }
        }
        float cm = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
        cm = fmaxf(cm, shfl_xor(cm, 16));
        cm = fmaxf(cm, shfl_xor(cm, 32));
        // the reference max moves only when a column's tile max exceeds it by more than 2^8
        const bool grow = cm > m + 8.f;
        if (__any(grow)) {
            const float mn = grow ? cm : m;
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai =
                    __int_as_float(__builtin_amdgcn_ds_bpermute((4 * g + i) << 2, __float_as_int(alpha)));
#pragma unroll
                for (int s = 0; s < NS; ++s) acc[s][i] *= ai;
            }
        }
        const float ms = (m == -INFINITY) ? 0.f : m;
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = fast_exp2(sc[i] - ms);
            l += pr[i];
        }
        u32x2 phi, plo;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const uint32_t h = M::pack_round(pr[2 * w], pr[2 * w + 1]);
            phi[w] = h;
            plo[w] = M::pack_round(pr[2 * w] - M::lo(h), pr[2 * w + 1] - M::hi(h));
        }
        // B operands of the 8 slices: the transpose reads of the V tile, all issued before any
        // is used, and waited for inside the same block. (The tile's loads are complete: the
        // K reads above waited for them, K and V having been issued together. Written as
        // builtins, these reads would carry no alias information, and the compiler would wait
        // for every tile in flight before them.)
        const int vr = 4 * g + (n >> 2);  // the V row this lane addresses
        uint32_t va[NS];
#pragma unroll
        for (int s = 0; s < NS; ++s)
            va[s] = lds_addr(reinterpret_cast<const char*>(buf + 256 + 16 * vr + ((2 * s + ((n & 3) >> 1)) ^ vswz(vr))) +
                             8 * (n & 1));
        u32x2 vb[NS];
        asm volatile(
            "ds_read_b64_tr_b16 %0, %8\n\t"
            "ds_read_b64_tr_b16 %1, %9\n\t"
            "ds_read_b64_tr_b16 %2, %10\n\t"
            "ds_read_b64_tr_b16 %3, %11\n\t"
            "ds_read_b64_tr_b16 %4, %12\n\t"
            "ds_read_b64_tr_b16 %5, %13\n\t"
            "ds_read_b64_tr_b16 %6, %14\n\t"
            "ds_read_b64_tr_b16 %7, %15\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(vb[0]), "=&v"(vb[1]), "=&v"(vb[2]), "=&v"(vb[3]), "=&v"(vb[4]), "=&v"(vb[5]), "=&v"(vb[6]),
              "=&v"(vb[7])
            : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "v"(va[4]), "v"(va[5]), "v"(va[6]), "v"(va[7])
            : "memory");
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            acc[s] = M::k16(phi, vb[s], acc[s]);
            acc[s] = M::k16(plo, vb[s], acc[s]);
        }
    };

    u32x4* const buf = s_tile[wave];
    for (int k = 0; k < nt; ++k) {
        issue(k, buf);
        compute(k, buf);
    }
    // every wave done with its tiles before the sums take their memory
    __syncthreads();

    // column n's sum over the four lane groups
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (g == 0 && n < G) {
        s_m[wave][n] = m;
        s_l[wave][n] = l;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i < G) s_acc[wave][4 * g + i][16 * s + n] = acc[s][i];
    __syncthreads();
    partition_epilogue<T, D, G, NW>(a, p, kvh, b, part, s_m, s_l, s_acc);
    if (part.npos >= 0 && !a.ws_slot) store_new_rows<T, D, NW * 64>(a, part.slot, kvh, 1, s_new);
}

#undef PA_LDS_PTR

// Launch of the LDS path: 8 waves per work-group (two work-groups per compute unit, two waves
// per SIMD), or 4 for partitions of up to 512 tokens in a grid of 1024 or more work-groups,
// where four work-groups per unit hide each one's prologue (B = 256 at 129 tokens: 32.6
// against 40.2 us; B = 32 at 2049 tokens, one 4-wave work-group per unit: 52.2 against 45.2).
template <typename T, int G>
hipError_t launch_decode_lds(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    const dim3 grid(num_kv_heads, batch, a.max_partitions);
    if (a.partition_size <= 512 && (int64_t)num_kv_heads * batch * a.max_partitions >= 1024)
        hipLaunchKernelGGL((decode_mfma_lds_kernel<T, G, 4>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((decode_mfma_lds_kernel<T, G, 8>), grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mfma
}  // namespace pagedkv
