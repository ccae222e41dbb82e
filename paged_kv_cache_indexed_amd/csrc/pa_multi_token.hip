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

// ---- Long query chunks: 64 (query, head) rows per work-group ---------------------------------
//
// When a sequence brings more than 16 (query, head) rows per kv head (chunked prefill, long
// speculative runs), the kernel above re-reads every K/V tile for each 16-column tile and
// transposes V once per tile and wave. This one gives a work-group 64 rows (16 per wave) of
// one kv head and streams the partition's K/V once for all of them:
//   * 32-token tiles are loaded by the whole work-group with whole-row loads (1 KiB
//     contiguous per wave instruction) into LDS, double-buffered, one barrier per tile. K and
//     V are stored row-major as loaded (16-byte unit u of token r at u ^ (r & 7) for K, so
//     the operand reads below hit distinct banks; at u ^ vsw(r) for V, so the transpose reads
//     do).
//   * Each wave computes S^T = K Q^T for its 16 rows (K tile rows from LDS as the A operand,
//     Q^T in registers as B), runs the same base-2 online softmax as the decode (P stays in
//     the lanes that computed it, split into rounded high and low parts), and accumulates
//     O = P V with the B operand read from the V tile by ds_read_b64_tr_b16, which transposes
//     4 x 16 pieces across each 16-lane group: lane (n, g) receives dim n of the slice at
//     tokens 4g..4g+3 and 16+4g..16+4g+3, the tokens its k-slots stand for. (A transposed
//     [dim][token] copy written with 16-bit stores was 1-7% slower and took more registers.)
//   * Rows belong to one wave from start to end, so there is no cross-wave merge: each wave
//     writes its rows' outputs, or their partition records for the log-sum-exp reduce.
// 16-bit pools, head_dim 64 or 128; the group size is a run-time value.
namespace prefill {


using mfma::f32x4;
using mfma::u32x2;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 16 * kWaves;  // (query, head) rows per work-group
constexpr int kTile = 32;           // tokens per K/V tile

// NaN sink: the rows of row tile rt of sequence b (query-major (query, head) rows).
template <typename T, int D>
struct RowTileNanSink {
    const DecodeArgs& a;
    int q0, nq, kvh, rt, G;
    __device__ bool valid(int r) const { return kRows * rt + r < nq * G; }
    __device__ size_t row(int r) const {
        const int x = kRows * rt + r;
        return (size_t)(q0 + x / G) * a.num_q_heads + kvh * G + x % G;
    }
    __device__ void nan_outputs() const {
        for (int i = threadIdx.x; i < kRows * D; i += kThreads)
            if (valid(i / D)) store_elem(T{}, a.out, row(i / D) * D + i % D, __builtin_nanf(""));
    }
    __device__ void nan_records(int p) const {
        for (int i = threadIdx.x; i < kRows * (D + 2); i += kThreads) {
            const int r = i / (D + 2), e = i % (D + 2);
            if (!valid(r)) continue;
            const size_t rec = row(r) * a.max_partitions + p;
            if (e < D) a.ws_o[rec * D + e] = __builtin_nanf("");
            else a.ws_ml[rec * 2 + (e - D)] = (e == D) ? -INFINITY : __builtin_nanf("");
        }
    }
};

// 8-byte buffer load (8 E4M3 codes).
__device__ __forceinline__ u32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)offset, 0, 0));
}

// T: type of q, out and the tiles in LDS; KV: the pool's storage (T, or FP8 codes that widen
// exactly to T when parked, with the tile's K and V scales beside them in LDS).
template <typename T, typename KV, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void prefill_kernel(DecodeArgs a) {
    static_assert(T::kBytes == 2 && (D == 64 || D == 128), "16-bit rows of 64 or 128 elements");
    constexpr bool kFp8 = std::is_same_v<KV, FP8>;
    using M = mfma::Mma<T>;
    constexpr int U = D / 8;                   // 16-byte units per 16-bit row (8 elements each)
    constexpr int NC = D / 32;                 // k-blocks of the score contraction
    constexpr int NS = D / 16;                 // 16-dim output slices
    // Units of 8 elements per thread per tile, for K and for V (16 bytes each from 16-bit
    // pools, 8 codes from 8-bit ones).
    constexpr int kLoads = kTile * U / kThreads;
    static_assert(kLoads >= 1 && kLoads * kThreads == kTile * U, "tile split");
    __shared__ int s_ids[kMaxIdsPerPartition];
    __shared__ u32x4 s_k[2][kTile * U];
    __shared__ u32x4 s_v[2][kTile * U];
    // V rows as loaded; unit u of token r at u ^ vsw(r), so that the transpose reads (4 rows,
    // 2 units per 16-lane group) and the row writes spread over the banks
    auto vsw = [](int r) { return (r * (U / 8)) & (U - 1); };
    __shared__ float s_ks[kFp8 ? 2 : 1][kFp8 ? kTile : 1];  // 8-bit pools: the tile's K and V row scales
    __shared__ float s_vs[kFp8 ? 2 : 1][kFp8 ? kTile : 1];

    const int G = a.num_q_heads / a.num_kv_heads;
    const int row_tiles = (a.col_tiles + 3) / 4;
    const int p = grid_partition();
    const int kvh = blockIdx.x;
    const int b = (int)blockIdx.y / row_tiles;
    const int rt = (int)blockIdx.y - b * row_tiles;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int lbs = a.log2_block_size;
    const int bs = 1 << lbs;

    const int q0 = a.query_start[b];
    const int nq = a.query_start[b + 1] - q0;
    if (q0 < 0 || nq < 0 || q0 + nq > a.num_q_tokens || nq * G > 16 * a.col_tiles) {
        if (p == 0 && kvh == 0 && rt == 0 && tid == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_LENGTH);
        return;
    }
    if (kRows * rt >= nq * G) return;  // no row of this sequence in this tile (uniform)
    const int r_tile = 16 * wave + n;   // this lane's row inside the tile (column n of S^T)
    const int x = kRows * rt + r_tile;  // row index in the sequence
    const bool row_valid = x < nq * G;
    const int qi = x / G;

    // Q^T as the B operand: k-block c of lane group g holds dims 32c + 8g .. +7 of the row
    u32x4 qb[NC];
    {
        const char* qrow = static_cast<const char*>(a.q) +
                           ((size_t)(q0 + (row_valid ? qi : 0)) * a.num_q_heads + kvh * G + (row_valid ? x % G : 0)) * D * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) qb[c] = row_valid ? load16(qrow + 2 * (32 * c + 8 * g)) : u32x4{0, 0, 0, 0};
    }
    Partition part;
    if (!partition_prologue_sink<T, D, kThreads>(a, p, b, max(nq, 1), RowTileNanSink<T, D>{a, q0, nq, kvh, rt, G},
                                                 s_ids, part))
        return;
    const int first_pos = part.len - nq;  // position of query 0
    const int last_q = min(kRows * rt + kRows - 1, nq * G - 1) / G;
    const int tile_end = first_pos + last_q + 1 - part.t0;  // tokens the tile's last query sees
    if (tile_end <= 0) return;  // the whole partition is after this tile's queries (uniform)
    const int ntok = min(part.ntok, tile_end);
    const int rel_lo = part.rel_lo;
    const int lim = row_valid ? min(ntok, first_pos + qi + 1 - part.t0) : 0;  // this row sees [rel_lo, lim)
    const int k0 = rel_lo / kTile;
    const int ntiles = (ntok + kTile - 1) / kTile - k0;
    // Tokens every row of this wave sees: rows are query-major, so the wave's first row has the
    // smallest limit when all 16 rows are valid (a partial wave takes the masked path).
    const int xw = kRows * rt + 16 * wave;
    const int lim_wave = xw + 15 < nq * G ? min(ntok, first_pos + xw / G + 1 - part.t0) : 0;

    const size_t head_bytes = (size_t)bs * D * KV::kBytes;
    const char* kpool = static_cast<const char*>(a.k_pool);
    const char* vpool = static_cast<const char*>(a.v_pool);

    // Load i of thread tid covers 16-byte unit u of tile token t, unit kThreads i + tid of the
    // tile in row order: a wave instruction reads 4 (head_dim 128) or 8 (head_dim 64) whole
    // consecutive rows, which lie in one aligned group of 8 tokens, so in one block: the id is
    // wave-uniform.
    auto slot_of = [&](int i, int& t, int& u) {
        t = (kThreads * i + tid) / U;
        u = (kThreads * i + tid) % U;
    };
    auto issue = [&](int k, u32x4* kr, u32x4* vr) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            int t, u;
            slot_of(i, t, u);
            const int rel = (k0 + k) * kTile + t;
            const int tw = (kThreads * i + 64 * wave) / U;
            const int rel_w = (k0 + k) * kTile + tw;  // the wave's first token
            const int id = __builtin_amdgcn_readfirstlane(s_ids[(rel_w < ntok ? rel_w : 0) >> lbs]);
            const size_t slab = (size_t)id * a.block_stride + (size_t)kvh * head_bytes;
            const uint32_t off = (rel < ntok && rel >= rel_lo) ? (uint32_t)((((rel & (bs - 1)) * U) + u) * 16)
                                                                : kOutOfRange;
            kr[i] = buffer_load16<0>(make_rsrc(kpool + slab, (uint32_t)head_bytes), off);
            vr[i] = buffer_load16<0>(make_rsrc(vpool + slab, (uint32_t)head_bytes), off);
        }
    };
    auto park = [&](int buf, const u32x4* kr, const u32x4* vr) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            int t, u;
            slot_of(i, t, u);
            s_k[buf][t * U + (u ^ (t & 7))] = kr[i];
            s_v[buf][t * U + (u ^ vsw(t))] = vr[i];
        }
    };

    // 8-bit pools: the same (token, unit) slots, each an 8-byte load of 8 codes; threads 0-31
    // and 32-63 also load the K and V scales of the 32 tile tokens (whose blocks may differ
    // from lane to lane).
    float scale8 = 0.f;
    auto issue8 = [&](int k, u32x2* kr, u32x2* vr) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            int t, u;
            slot_of(i, t, u);
            const int rel = (k0 + k) * kTile + t;
            const int tw = (kThreads * i + 64 * wave) / U;
            const int rel_w = (k0 + k) * kTile + tw;  // the wave's first token
            const int id = __builtin_amdgcn_readfirstlane(s_ids[(rel_w < ntok ? rel_w : 0) >> lbs]);
            const size_t slab = (size_t)id * a.block_stride + (size_t)kvh * head_bytes;
            const uint32_t off = (rel < ntok && rel >= rel_lo) ? (uint32_t)((rel & (bs - 1)) * D + 8 * u) : kOutOfRange;
            kr[i] = buffer_load8(make_rsrc(kpool + slab, (uint32_t)head_bytes), off);
            vr[i] = buffer_load8(make_rsrc(vpool + slab, (uint32_t)head_bytes), off);
        }
        if (tid < 2 * kTile) {
            const int rel = (k0 + k) * kTile + (tid & (kTile - 1));
            scale8 = 0.f;
            if (rel < ntok && rel >= rel_lo) {
                const size_t srow = (((size_t)s_ids[rel >> lbs] * a.num_kv_heads + kvh) << lbs) + (rel & (bs - 1));
                scale8 = (tid < kTile ? a.k_scale : a.v_scale)[srow];
            }
        }
    };
    auto park8 = [&](int buf, const u32x2* kr, const u32x2* vr) {
        u32x4 kw[kLoads], vw[kLoads];
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {  // the codes widen exactly to T
            kw[i] = mfma::widen8(T{}, kr[i].x, kr[i].y);
            vw[i] = mfma::widen8(T{}, vr[i].x, vr[i].y);
        }
        park(buf, kw, vw);
        if (tid < kTile) s_ks[buf][tid] = scale8;
        else if (tid < 2 * kTile) s_vs[buf][tid - kTile] = scale8;
    };

    float m = -INFINITY;  // running base-2 max of row n (same in the four lane groups)
    float l = 0.f;        // this lane's part of row n's running sum
    f32x4 acc[NS];        // acc[s][i] = O[row 4g + i][dim 16s + n]
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int k, int buf) {
        const int rel0 = (k0 + k) * kTile;
        const bool full = rel0 >= rel_lo && rel0 + kTile <= lim_wave;
        float sc[8];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            const int r = 16 * t + n;
#pragma unroll
            for (int c = 0; c < NC; ++c) st = M::k32(s_k[buf][r * U + ((4 * c + g) ^ (r & 7))], qb[c], st);
            if constexpr (kFp8) {  // the K row scales multiply the scores
#pragma unroll
                for (int i = 0; i < 4; ++i) st[i] *= s_ks[buf][16 * t + 4 * g + i];
            }
            if (full) {  // every row of the wave sees the whole tile (wave-uniform)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[4 * t + i] = st[i] * a.scale_log2;
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = rel0 + 16 * t + 4 * g + i;
                    sc[4 * t + i] = (tok < lim && tok >= rel_lo) ? st[i] * a.scale_log2 : -INFINITY;
                }
            }
        }
        float cm = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
        cm = fmaxf(cm, shfl_xor(cm, 16));
        cm = fmaxf(cm, shfl_xor(cm, 32));
        // The reference max m moves only when a row's tile max exceeds it by more than 2^8
        // (weights then stay below 256, far inside fp32 and the split into high and low
        // parts), so most tiles skip rescaling the accumulators; m and l stay a consistent
        // pair for the normalisation and the partition records whichever reference is used.
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
        float pr[8];
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            pr[j] = fast_exp2(sc[j] - ms);
            psum += pr[j];
        }
        l += psum;
        if constexpr (kFp8) {  // the V row scales multiply the weights (not the running sum)
#pragma unroll
            for (int j = 0; j < 8; ++j) pr[j] *= s_vs[buf][16 * (j >> 2) + 4 * g + (j & 3)];
        }
        u32x4 phi, plo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t h = M::pack_round(pr[2 * w], pr[2 * w + 1]);
            phi[w] = h;
            plo[w] = M::pack_round(pr[2 * w] - M::lo(h), pr[2 * w + 1] - M::hi(h));
        }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            // lane n addresses row 4g + n / 4 (of each 16-token half), dims 16s + 4 (n % 4) .. +3;
            // the transpose read hands it dim 16s + n of rows 4g .. 4g+3
            u32x4 vb;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = 16 * h + 4 * g + (n >> 2);
                const int uu = 2 * s + ((n & 3) >> 1);
                const char* piece = reinterpret_cast<const char*>(&s_v[buf][r * U + (uu ^ vsw(r))]) + 8 * (n & 1);
                const u32x2 y = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) mfma::mf_s16x4*)(const_cast<char*>(piece))));
                vb[2 * h] = y.x;
                vb[2 * h + 1] = y.y;
            }
            acc[s] = M::k32(phi, vb, acc[s]);
            acc[s] = M::k32(plo, vb, acc[s]);
        }
    };

    if constexpr (kFp8) {
        if (ntiles > 0) {
            u32x2 kr[kLoads], vr[kLoads];
            issue8(0, kr, vr);
            park8(0, kr, vr);
            __syncthreads();
            if (ntiles > 1) issue8(1, kr, vr);
            for (int k = 0; k < ntiles; ++k) {
                compute(k, k & 1);
                if (k + 1 < ntiles) park8((k + 1) & 1, kr, vr);
                __syncthreads();
                if (k + 2 < ntiles) issue8(k + 2, kr, vr);
            }
        }
    } else if (ntiles > 0) {
        u32x4 kr[kLoads], vr[kLoads];
        issue(0, kr, vr);
        park(0, kr, vr);
        __syncthreads();
        if (ntiles > 1) issue(1, kr, vr);
        for (int k = 0; k < ntiles; ++k) {
            compute(k, k & 1);
            if (k + 1 < ntiles) park((k + 1) & 1, kr, vr);
            __syncthreads();
            if (k + 2 < ntiles) issue(k + 2, kr, vr);
        }
    }

    // row n's totals, then each lane's four rows 4g + i from their lanes
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    const int xr0 = kRows * rt + 16 * wave;  // row index of this wave's row 0
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int rr = 4 * g + i;
        const float li = __int_as_float(__builtin_amdgcn_ds_bpermute(rr << 2, __float_as_int(l)));
        const int xi = xr0 + rr;
        if (xi >= nq * G) continue;
        const size_t orow = (size_t)(q0 + xi / G) * a.num_q_heads + kvh * G + xi % G;
        const float inv = 1.f / li;
        if (part.nparts == 1) {
#pragma unroll
            for (int s = 0; s < NS; ++s) store_elem(T{}, a.out, orow * D + 16 * s + n, acc[s][i] * inv);
        } else {
            const size_t rec = orow * a.max_partitions + p;
#pragma unroll
            for (int s = 0; s < NS; ++s) a.ws_o[rec * D + 16 * s + n] = acc[s][i] * inv;
        }
    }
    if (part.nparts > 1 && g == 0 && row_valid) {
        const size_t rec = ((size_t)(q0 + qi) * a.num_q_heads + kvh * G + x % G) * a.max_partitions + p;
        a.ws_ml[rec * 2] = m;
        a.ws_ml[rec * 2 + 1] = l;
    }
}

template <typename T, typename KV, int D>
hipError_t launch_prefill_td(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    const int row_tiles = (a.col_tiles + 3) / 4;
    dim3 grid(num_kv_heads, batch * row_tiles, a.max_partitions);
    hipLaunchKernelGGL((prefill_kernel<T, KV, D>), grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace prefill

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
           (group == 1 || group == 2 || group == 4 || group == 8 || group == 16) &&
           (block_size >= 16 || (block_size == 8 && head_dim <= 128)) &&
           (head_dim == 64 || head_dim == 128 || head_dim == 256) && !(group == 16 && head_dim == 256);
}

hipError_t launch_multi_token(const DecodeArgs& a, int kv_dtype, int dtype, int head_dim, int group, int batch,
                              int num_kv_heads, hipStream_t stream) {
    // 64 or more (query, head) rows per kv head: the 64-row kernel (with fewer rows its tiles
    // run mostly empty: 2 column tiles measured 30% slower there)
    if (a.col_tiles >= 4 && (head_dim == 64 || head_dim == 128) && (kv_dtype == dtype || kv_dtype == PA_FP8_E4M3)) {
        const bool f8 = kv_dtype == PA_FP8_E4M3;
        if (dtype == PA_F16) {
            if (f8) return head_dim == 64 ? prefill::launch_prefill_td<F16, FP8, 64>(a, batch, num_kv_heads, stream)
                                          : prefill::launch_prefill_td<F16, FP8, 128>(a, batch, num_kv_heads, stream);
            return head_dim == 64 ? prefill::launch_prefill_td<F16, F16, 64>(a, batch, num_kv_heads, stream)
                                  : prefill::launch_prefill_td<F16, F16, 128>(a, batch, num_kv_heads, stream);
        }
        if (dtype == PA_BF16) {
            if (f8) return head_dim == 64 ? prefill::launch_prefill_td<BF16, FP8, 64>(a, batch, num_kv_heads, stream)
                                          : prefill::launch_prefill_td<BF16, FP8, 128>(a, batch, num_kv_heads, stream);
            return head_dim == 64 ? prefill::launch_prefill_td<BF16, BF16, 64>(a, batch, num_kv_heads, stream)
                                  : prefill::launch_prefill_td<BF16, BF16, 128>(a, batch, num_kv_heads, stream);
        }
    }
    // 8-token blocks, fewer rows: the 16-column kernel with a block lookup per row (the 64-row
    // kernel's wave loads stay inside an aligned group of 8 tokens, so it takes any block size)
    if (a.log2_block_size < 4)
        return launch_multi_token_small_blocks(a, kv_dtype, dtype, head_dim, group, batch, num_kv_heads, stream);
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
