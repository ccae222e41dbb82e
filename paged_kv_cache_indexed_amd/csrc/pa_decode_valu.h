#pragma once
// VALU paged-KV decode for gfx950 (templates; instantiated by pa_decode.hip for 16/32-bit
// pools and by pa_decode_fp8.hip for 8-bit float pools).
//
// Work decomposition (VALU path, used for every group size):
//   * A workgroup is 4 wave64s. It owns the tokens [p*P, min(L, (p+1)*P)) of one kv head of
//     one sequence and the G = Hq/Hkv query heads that read that kv head.
//   * The partition's slice of the block table is staged in LDS once and checked, so the
//     per-load address translation is an LDS broadcast read plus scalar arithmetic
//     ([BlockManager essay] §2 on caching the mapping table on chip).
//   * A K or V row of one token is head_dim * bytes long and is covered by LPR lanes with
//     one 16-byte load each; a wave load covers RPL = 64 / LPR consecutive tokens of one
//     block, 1 KiB of contiguous memory. Token groups of RPL rows are dealt round-robin to
//     the 4 waves, so the waves of a workgroup stream adjacent KiB of the same block.
//   * Each group of LPR lanes runs its own online softmax (running max and sum in fp32,
//     base-2 exponent with the scale folded into q . k) over the tokens it loads, so the
//     inner loop needs no cross-row traffic; rows are merged with lane shuffles and waves
//     through LDS at the end.
//   * Tokens at or past the valid length are never loaded ([Valid-length essay] §4.1-4.2):
//     K/V are read with buffer loads whose resource spans one (block, kv head) slab, and a
//     masked lane's offset is out of range, so the hardware returns zeros without a memory
//     access; the lane's score is -inf and its weight exp2(-inf) = 0.
//   * Two register buffers of UNROLL groups are kept loading: while one is consumed the
//     other's loads are in flight, so each lane has 2 * UNROLL K+V loads outstanding.
#include <type_traits>

#include "pa_decode_common.h"

namespace pagedkv {
namespace valu {


constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = kDecodeThreads;

// Lazy rescaling of the online softmax (8-bit pools): the running reference moves only when a
// score exceeds it by more than this (base-2 exponent), so weights stay below 2^8 in fp32.
constexpr float kLazyRescale = 8.f;

// KV is the pool's element type: a lane's 16-byte load holds E elements of a token row.
template <typename KV, int D>
struct RowShape {
    static constexpr int E = VecInfo<KV>::kElems;  // elements per 16-byte vector
    static constexpr int LPR = D / E;              // lanes per token row
    static constexpr int RPL = 64 / LPR;           // token rows per wave load
    static_assert(LPR >= 1 && LPR <= 64 && RPL * LPR == 64, "row shape");
};

// A lane's slice of one query head: the E elements matching its K vector, in q's type T.
template <typename T, typename KV>
struct QFrag {
    static constexpr int kVecs = VecInfo<KV>::kElems * T::kBytes / 16;
    u32x4 v[kVecs];
};

template <typename T, typename KV>
__device__ __forceinline__ float dot_frag(const QFrag<T, KV>& q, u32x4 k) {
    if constexpr (std::is_same_v<KV, FP8>) return dot16_fp8(T{}, q.v, k);
    else return dot16(T{}, q.v[0], k);
}

// Streams this lane's share of a partition of kv head `kvh` and leaves the wave's merged
// online-softmax state of the G query heads in every lane (m, l, and the E accumulators of
// the lane's column). Row groups of RPL tokens are taken in the order
// slot, slot + STRIDE, slot + 2 STRIDE, ...: STRIDE waves cooperate on one head, or one
// wave (STRIDE = 1) owns it. All lanes must be active.
//
// With 8-bit pools each token row also has a float32 scale (k_scale / v_scale, one per
// (block, kv head, offset)): the K scale multiplies the row's score, the V scale its softmax
// weight in the weighted sum (not in the running sum, which normalises the weights).
//
// Fused append: the row at position part.npos (if >= 0) is taken from s_new (K row, then V
// row, of this wave's kv head, in the pool's storage) instead of the pool. Over an 8-bit pool
// the wave that folds the token in first quantises the staged rows s_raw (q's type) into
// s_new, while its first loads are in flight.
template <typename T, typename KV, int D, int G, int UNROLL, int STRIDE>
__device__ __forceinline__ void stream_partition(const DecodeArgs& a, const int* s_ids, const Partition& part,
                                                 int kvh, int slot, const QFrag<T, KV>* qv, float* m, float* l,
                                                 float (*acc)[RowShape<KV, D>::E], char* s_new = nullptr,
                                                 const char* s_raw = nullptr) {
    constexpr bool kScaled = std::is_same_v<KV, FP8>;
    constexpr int E = RowShape<KV, D>::E;
    constexpr int LPR = RowShape<KV, D>::LPR;
    constexpr int RPL = RowShape<KV, D>::RPL;
    const int lane = threadIdx.x & 63;
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int lbs = a.log2_block_size;
    const int bs = 1 << lbs;
    const int ntok = part.ntok;
    const int rel_lo = part.rel_lo;
    const int g0 = rel_lo / RPL;  // first row group holding an attended token
    const int npos = part.npos;   // fused append: this row comes from s_new, after the loop

    const size_t head_bytes = (size_t)bs * D * KV::kBytes;
    const size_t block_bytes = (size_t)a.block_stride;
    const char* kpool = static_cast<const char*>(a.k_pool);
    const char* vpool = static_cast<const char*>(a.v_pool);
    constexpr int kTokPerIter = UNROLL * STRIDE * RPL;
    const int niters = (ntok - g0 * RPL + kTokPerIter - 1) / kTokPerIter;

#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
    }

    // Branch-free loads: every lane issues its loads; a lane whose token is at or past the
    // partition end gets an out-of-range offset and reads zeros without a memory access.
    // The buffer resource spans only this (block, kv head) slab.
    const uint32_t slab_bytes = (uint32_t)head_bytes;
    const uint32_t lane_bytes = (uint32_t)(((size_t)row * D + col * E) * KV::kBytes);
    auto issue = [&](int it, u32x4* kk, u32x4* vv, float* ksc, float* vsc) {
        int idv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int rel = (g0 + (it * UNROLL + u) * STRIDE + slot) * RPL;  // wave-uniform
            idv[u] = s_ids[(rel < ntok ? rel : 0) >> lbs];  // partitions start on a block
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int rel = (g0 + (it * UNROLL + u) * STRIDE + slot) * RPL;
            const int id = __builtin_amdgcn_readfirstlane(idv[u]);
            const size_t slab = (size_t)id * block_bytes + (size_t)kvh * head_bytes;
            const bool live = rel + row < ntok && rel + row >= rel_lo && rel + row != npos;
            const uint32_t off = live ? (uint32_t)((rel & (bs - 1)) * D * KV::kBytes) + lane_bytes : kOutOfRange;
            kk[u] = buffer_load16(make_rsrc(kpool + slab, slab_bytes), off);
            vv[u] = buffer_load16(make_rsrc(vpool + slab, slab_bytes), off);
            if constexpr (kScaled) {
                // cached, unlike the streamed codes: with 16-token blocks two kv heads' scales
                // share a 128-byte line (2-3% faster than streamed loads on 64 x 32 heads of
                // 450-520 tokens and on 256 x 32 heads of long-tailed lengths)
                const size_t srow = ((size_t)id * a.num_kv_heads + kvh) << lbs;  // this slab's scales
                const uint32_t soff = live ? (uint32_t)(((rel & (bs - 1)) + row) * 4) : kOutOfRange;
                ksc[u] = buffer_load_f32<0>(make_rsrc(a.k_scale + srow, (uint32_t)bs * 4), soff);
                vsc[u] = buffer_load_f32<0>(make_rsrc(a.v_scale + srow, (uint32_t)bs * 4), soff);
            }
        }
    };

    auto compute = [&](int it, const u32x4* kk, const u32x4* vv, const float* ksc, const float* vsc) {
        float s[G][UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int rel = (g0 + (it * UNROLL + u) * STRIDE + slot) * RPL + row;
            const bool valid = rel < ntok && rel >= rel_lo && rel != npos;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = group_sum<LPR>(dot_frag(qv[g], kk[u]));
                if constexpr (kScaled) d *= ksc[u];
                s[g][u] = valid ? d * a.scale_log2 : -INFINITY;
            }
        }
        if constexpr (kScaled) {
            // 8-bit pools: m[g] is a reference the state is scaled to, moved only when a score
            // passes it by more than kLazyRescale (base 2), so every weight 2^(s - m) stays
            // below 2^kLazyRescale and the 16 accumulators of a lane are rescaled rarely, not
            // once per row group. The rows are then folded in one at a time, each V row
            // widened just before its FMAs (16 values a row: widening all UNROLL rows first
            // would hold UNROLL x 16 more registers).
            float ms[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float cm = s[g][0];
#pragma unroll
                for (int u = 1; u < UNROLL; ++u) cm = fmaxf(cm, s[g][u]);
                if (cm > m[g] + kLazyRescale) {  // -inf + k is -inf: the first finite score moves it
                    const float alpha = fast_exp2(m[g] - cm);
                    m[g] = cm;
                    l[g] *= alpha;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
                }
                ms[g] = (m[g] == -INFINITY) ? 0.f : m[g];
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float wv[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float pr = fast_exp2(s[g][u] - ms[g]);
                    l[g] += pr;
                    wv[g] = pr * vsc[u];
                }
                // two codes at a time: each widened pair feeds its FMAs at once
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vv[u][w], 1.f, false);
                    const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vv[u][w], 1.f, true);
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        acc[g][4 * w] = fmaf(wv[g], lo.x, acc[g][4 * w]);
                        acc[g][4 * w + 1] = fmaf(wv[g], lo.y, acc[g][4 * w + 1]);
                        acc[g][4 * w + 2] = fmaf(wv[g], hi.x, acc[g][4 * w + 2]);
                        acc[g][4 * w + 3] = fmaf(wv[g], hi.y, acc[g][4 * w + 3]);
                    }
                }
            }
        } else {
            float vf[UNROLL][E];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) unpack(KV{}, vv[u], vf[u]);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float cm = s[g][0];
#pragma unroll
                for (int u = 1; u < UNROLL; ++u) cm = fmaxf(cm, s[g][u]);
                const float mn = fmaxf(m[g], cm);
                const float ms = (mn == -INFINITY) ? 0.f : mn;
                const float alpha = fast_exp2(m[g] - ms);
                m[g] = mn;
                l[g] *= alpha;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
#pragma unroll
                for (int u = 0; u < UNROLL; ++u) {
                    const float pr = fast_exp2(s[g][u] - ms);
                    l[g] += pr;
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[g][e] = fmaf(pr, vf[u][e], acc[g][e]);
                }
            }
        }
    };

    // Two register buffers, each refilled right after it is consumed, so two groups of
    // loads are in flight at all times and every wait before a compute covers only the older
    // group. Refills past the last group get out-of-range offsets: they return zeros and move
    // no data. The scheduling barriers keep the compiler from sinking a refill below the next
    // compute, which would drain the load queue.
    u32x4 ka[UNROLL], va[UNROLL], kb[UNROLL], vb[UNROLL];
    float ksa[UNROLL], vsa[UNROLL], ksb[UNROLL], vsb[UNROLL];  // row scales (8-bit pools only)
    issue(0, ka, va, ksa, vsa);
    issue(1, kb, vb, ksb, vsb);
    if constexpr (kScaled) {
        if (npos >= 0 && slot == 0) quantize_new_rows<T, D>(s_raw, s_new);  // wave-uniform
    }
    int it = 0;
    for (; it + 1 < niters; it += 2) {  // one latch: the wait state is the same on every entry
        __builtin_amdgcn_sched_barrier(0);
        compute(it, ka, va, ksa, vsa);
        __builtin_amdgcn_sched_barrier(0);
        issue(it + 2, ka, va, ksa, vsa);
        __builtin_amdgcn_sched_barrier(0);
        compute(it + 1, kb, vb, ksb, vsb);
        __builtin_amdgcn_sched_barrier(0);
        issue(it + 3, kb, vb, ksb, vsb);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (it < niters) compute(it, ka, va, ksa, vsa);

    // Fused append: the new token (masked in the loop above) joins the row-0 stream of the
    // first wave that owns this head, its K and V rows (and scales) read from s_new.
    if (npos >= 0 && slot == 0) {
        using R = NewRec<KV, D>;
        const u32x4 kx = *reinterpret_cast<const u32x4*>(s_new + 16 * col);
        float vx[E];
        unpack(KV{}, *reinterpret_cast<const u32x4*>(s_new + R::kRowBytes + 16 * col), vx);
        float kscale = 1.f, vscale = 1.f;
        if constexpr (kScaled) {
            kscale = reinterpret_cast<const float*>(s_new + 2 * R::kRowBytes)[0];
            vscale = reinterpret_cast<const float*>(s_new + 2 * R::kRowBytes)[1];
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = group_sum<LPR>(dot_frag(qv[g], kx));
            if constexpr (kScaled) d *= kscale;
            const float sc = (row == 0) ? d * a.scale_log2 : -INFINITY;
            const float mn = fmaxf(m[g], sc);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = fast_exp2(m[g] - ms);
            const float pr = fast_exp2(sc - ms);
            m[g] = mn;
            l[g] = l[g] * alpha + pr;
            float wv = pr;
            if constexpr (kScaled) wv *= vscale;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] = fmaf(wv, vx[e], acc[g][e] * alpha);
        }
    }

    // ---- merge the RPL row streams of this wave ----
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float mo = shfl_xor(m[g], off);
            const float lo = shfl_xor(l[g], off);
            const float mn = fmaxf(m[g], mo);
            const float ms = (mn == -INFINITY) ? 0.f : mn;
            const float fa = fast_exp2(m[g] - ms);
            const float fb = fast_exp2(mo - ms);
            l[g] = l[g] * fa + lo * fb;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[g][e] = acc[g][e] * fa + shfl_xor(acc[g][e], off) * fb;
            m[g] = mn;
        }
    }
}

template <typename T, typename KV, int D, int G>
__device__ __forceinline__ void load_q(const DecodeArgs& a, int b, int h0, QFrag<T, KV>* qv) {
    constexpr int E = RowShape<KV, D>::E;
    const int col = (threadIdx.x & 63) % RowShape<KV, D>::LPR;
    const char* qbase = static_cast<const char*>(a.q) + (((size_t)b * a.num_q_heads + h0) * D + col * E) * T::kBytes;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < QFrag<T, KV>::kVecs; ++j) qv[g].v[j] = load16(qbase + (size_t)g * D * T::kBytes + 16 * j);
}

// One (partition, kv head, sequence) item of split mode: the NW waves of the workgroup share
// the partition (groups of RPL rows dealt round-robin), merge their states through LDS and
// write the item's output or partition record. All threads call it.
template <typename T, typename KV, int D, int G, int UNROLL, int NW>
__device__ __forceinline__ void split_item(const DecodeArgs& a, int p, int kvh, int b, int* s_ids,
                                           float (*s_m)[G], float (*s_l)[G], float (*s_acc)[G][D],
                                           char* s_new) {
    constexpr int E = RowShape<KV, D>::E;
    constexpr int LPR = RowShape<KV, D>::LPR;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPR;
    const int col = lane % LPR;

    if (partition_is_dead(a, p, b)) return;
    // q before the prologue, so its load overlaps the length and table round trip
    QFrag<T, KV> qv[G];
    load_q<T, KV, D, G>(a, b, kvh * G, qv);
    Partition part;
    if (!partition_prologue<T, D, G, NW * 64>(a, p, kvh, b, s_ids, part, s_new)) return;
    // the rows in the pool's storage: the staged rows themselves, or after them the 8-bit
    // record the folding wave quantises them into
    char* s_rec = s_new + (std::is_same_v<KV, FP8> ? NewRec<T, D>::kBytes : 0);

    float m[G], l[G], acc[G][E];
    stream_partition<T, KV, D, G, UNROLL, NW>(a, s_ids, part, kvh, wave, qv, m, l, acc, s_rec, s_new);
    if (row == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[wave][g][col * E + e] = acc[g][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            s_m[wave][g] = m[g];
            s_l[wave][g] = l[g];
        }
    }
    __syncthreads();
    partition_epilogue<T, D, G, NW>(a, p, kvh, b, part, s_m, s_l, s_acc);
    if (part.npos >= 0 && !a.ws_slot) store_new_rows<KV, D, NW * 64>(a, part.slot, kvh, 1, s_rec);
}

// Split mode: the NW waves of a workgroup share one kv head's partition. One workgroup per
// grid cell.
template <typename T, typename KV, int D, int G, int UNROLL, int NW>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(DecodeArgs a) {
    __shared__ int s_ids[kMaxIdsPerPartition];
    __shared__ float s_m[NW][G];
    __shared__ float s_l[NW][G];
    __shared__ float s_acc[NW][G][D];
    // the new token's K and V rows as read, and their 8-bit record (fused append)
    __shared__ __align__(16) char s_new[NewRec<T, D>::kBytes + (std::is_same_v<KV, FP8> ? NewRec<KV, D>::kBytes : 0)];
    split_item<T, KV, D, G, UNROLL, NW>(a, grid_partition(), blockIdx.x, blockIdx.y, s_ids, s_m, s_l, s_acc, s_new);
}

// Head mode, for short partitions: a workgroup owns one (partition, sequence) and 4
// consecutive kv heads that share the staged table slice; wave w streams kv head
// 4 * blockIdx.y + w alone and writes its result without any cross-wave merge.
template <typename T, typename KV, int D, int G, int UNROLL>
__global__ __launch_bounds__(kThreads) void decode_valu_heads_kernel(DecodeArgs a) {
    constexpr int E = RowShape<KV, D>::E;
    constexpr int LPR = RowShape<KV, D>::LPR;
    __shared__ int s_ids[kMaxIdsPerPartition];

    const int p = grid_partition();
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = lane / LPR;
    const int col = lane % LPR;
    const int kvh0 = blockIdx.x * kWaves;
    const int nkv = min(kWaves, a.num_kv_heads - kvh0);
    const bool active = wave < nkv;
    const int kvh = active ? kvh0 + wave : kvh0;
    const int h0 = kvh * G;

    // the new token's K and V rows of the workgroup's kv heads as read, and for an 8-bit pool
    // each wave's record of its own kv head (fused append)
    using R = NewRec<KV, D>;
    constexpr int kRaw = NewRec<T, D>::kBytes;
    constexpr bool kRec8 = std::is_same_v<KV, FP8>;
    __shared__ __align__(16) char s_new[kWaves * kRaw + (kRec8 ? kWaves * R::kBytes : 0)];
    if (partition_is_dead(a, p, b)) return;
    QFrag<T, KV> qv[G];
    load_q<T, KV, D, G>(a, b, h0, qv);
    Partition part;
    if (!partition_prologue_heads<T, D, kThreads, kWaves>(a, p, kvh0 * G, nkv * G, b, s_ids, part, s_new))
        return;
    if (!active) return;  // no barrier follows

    float m[G], l[G], acc[G][E];
    char* s_rec = kRec8 ? s_new + kWaves * kRaw + wave * R::kBytes : s_new + wave * kRaw;
    stream_partition<T, KV, D, G, UNROLL, 1>(a, s_ids, part, kvh, 0, qv, m, l, acc, s_rec, s_new + wave * kRaw);
    if (row == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const size_t hrow = (size_t)b * a.num_q_heads + h0 + g;
            const float inv = 1.f / l[g];
            if (part.nparts == 1) {
#pragma unroll
                for (int e = 0; e < E; ++e) store_elem(T{}, a.out, hrow * D + col * E + e, acc[g][e] * inv);
            } else {
                const size_t rec = hrow * a.max_partitions + p;
#pragma unroll
                for (int e = 0; e < E; ++e) a.ws_o[rec * D + col * E + e] = acc[g][e] * inv;
                if (col == 0) {
                    a.ws_ml[rec * 2] = m[g];
                    a.ws_ml[rec * 2 + 1] = l[g];
                }
            }
        }
    }
    // each wave stores its own kv head's new rows (nothing to do when not appending)
    if (part.npos >= 0 && !a.ws_slot) {
        constexpr int kVecs = 2 * R::kRowBytes / 16;
        const int lbs = a.log2_block_size;
        const int slot = part.slot;
        const int off = slot & ((1 << lbs) - 1);
        char* base[2] = {static_cast<char*>(const_cast<void*>(a.k_pool)),
                         static_cast<char*>(const_cast<void*>(a.v_pool))};
        for (int i = lane; i < kVecs; i += 64) {
            const int which = i / (R::kRowBytes / 16);
            const int v = i % (R::kRowBytes / 16);
            char* dst = base[which] + (size_t)(slot >> lbs) * a.block_stride +
                        ((((size_t)kvh << lbs) + off) * R::kRowBytes) + 16 * v;
            store16(dst, load16(s_rec + 16 * i));
        }
        if constexpr (R::kScaled) {
            if (lane < 2) {
                const size_t srow = (((size_t)(slot >> lbs) * a.num_kv_heads + kvh) << lbs) + off;
                const_cast<float*>(lane ? a.v_scale : a.k_scale)[srow] =
                    reinterpret_cast<const float*>(s_rec + 2 * R::kRowBytes)[lane];
            }
        }
    }
}

// Partitions of at most this many tokens run in head mode.
#ifndef PA_HEAD_MODE_MAX_P
#define PA_HEAD_MODE_MAX_P 128
#endif
// Waves per split-mode workgroup.
#ifndef PA_SPLIT_WAVES
#define PA_SPLIT_WAVES 4
#endif

template <typename T, typename KV, int D, int G, int UNROLL>
hipError_t launch_decode_tgdu(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    if (a.partition_size <= PA_HEAD_MODE_MAX_P) {
        dim3 grid((num_kv_heads + kWaves - 1) / kWaves, batch, a.max_partitions);
        hipLaunchKernelGGL((decode_valu_heads_kernel<T, KV, D, G, UNROLL>), grid, dim3(kThreads), 0, stream, a);
    } else {
        constexpr int NW = PA_SPLIT_WAVES;
        dim3 grid(num_kv_heads, batch, a.max_partitions);
        hipLaunchKernelGGL((decode_valu_kernel<T, KV, D, G, UNROLL, NW>), grid, dim3(NW * 64), 0, stream, a);
    }
    return hipGetLastError();
}

// Groups per iteration per wave: 4 for long partitions (and for head mode, where one wave
// streams a whole partition); 2 for short split-mode partitions (<= 384 tokens), where a
// 4-deep iteration would leave most lanes idle and the smaller register footprint lets 8
// waves share a SIMD. Grouped-query heads multiply the registers per group. 8-bit pools
// take 1 everywhere: a lane's 16-byte load is 16 codes (1 KiB per wave load is 8 rows, as
// many tokens as 2 groups of 16-bit rows), and at 72 VGPRs 7 waves share a SIMD, against
// 3 with 4 groups (145 VGPRs). Measured with lazy rescaling on 256 sequences x 32 heads of
// long-tailed lengths: median 87, 83 against 115 us; median 23, 42 against 56 us; on 64 x 32
// heads of 450-520 tokens, 50 against 58 us.
template <typename T, typename KV, int D, int G>
hipError_t launch_decode_tgd(const DecodeArgs& a, int batch, int num_kv_heads, hipStream_t stream) {
    if constexpr (G <= 2 && std::is_same_v<KV, FP8>) {
        return launch_decode_tgdu<T, KV, D, G, 1>(a, batch, num_kv_heads, stream);
    } else if constexpr (G <= 2) {
        if (a.partition_size > PA_HEAD_MODE_MAX_P && a.partition_size <= 384)
            return launch_decode_tgdu<T, KV, D, G, 2>(a, batch, num_kv_heads, stream);
        return launch_decode_tgdu<T, KV, D, G, 4>(a, batch, num_kv_heads, stream);
    } else {
        return launch_decode_tgdu<T, KV, D, G, (G <= 4 ? 2 : 1)>(a, batch, num_kv_heads, stream);
    }
}

template <typename T, typename KV, int D>
hipError_t launch_decode_td(const DecodeArgs& a, int group, int batch, int num_kv_heads, hipStream_t s) {
    switch (group) {
        case 1: return launch_decode_tgd<T, KV, D, 1>(a, batch, num_kv_heads, s);
        case 2: return launch_decode_tgd<T, KV, D, 2>(a, batch, num_kv_heads, s);
        case 4: return launch_decode_tgd<T, KV, D, 4>(a, batch, num_kv_heads, s);
        case 8: return launch_decode_tgd<T, KV, D, 8>(a, batch, num_kv_heads, s);
        case 16:
            // 16 heads of 16-element lanes would spill: 8-bit pools take at most 8 per kv head here
            if constexpr (D <= 128 && !std::is_same_v<KV, FP8>)
                return launch_decode_tgd<T, KV, D, 16>(a, batch, num_kv_heads, s);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

template <typename T, typename KV>
hipError_t launch_decode_t(const DecodeArgs& a, int head_dim, int group, int batch, int num_kv_heads,
                           hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_decode_td<T, KV, 64>(a, group, batch, num_kv_heads, s);
        case 128: return launch_decode_td<T, KV, 128>(a, group, batch, num_kv_heads, s);
        case 256: return launch_decode_td<T, KV, 256>(a, group, batch, num_kv_heads, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace valu
}  // namespace pagedkv
