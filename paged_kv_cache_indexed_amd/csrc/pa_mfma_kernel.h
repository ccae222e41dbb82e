#pragma once
// Paged attention on the gfx950 matrix cores (fp16 / bf16 operands): the kernel template shared
// by the grouped-query decode (pa_decode_mfma.hip) and multi-token attention (pa_multi_token.hip).
//
// When G = Hq / Hkv query heads share one kv head, scores and the value sum are small dense
// contractions: S = Q K^T over head_dim and O = P V over tokens. One workgroup still owns
// one (context partition, kv head, sequence); each of its 4 waves walks 32-token chunks
// (two 16-token tiles) of the partition with its own online softmax.
//
// Per chunk and wave (16 x 16 MFMA tiles; lane l has n = l % 16 and lane group g = l / 16):
//   * Scores, transposed: S^T[token][head] = K[token][:] . Q[head][:] with
//     v_mfma_f32_16x16x32. The K tile is the A operand straight from memory: for k-block c,
//     lane l loads dims 32c + 8g .. +7 of token row n (one load instruction covers 64
//     contiguous bytes of 16 rows). Q (B operand, heads as columns, zero beyond G) uses the
//     same dim-to-k-slot assignment, so the contraction is exact whatever order the
//     hardware sums k in. Lane l receives S^T for head n at tokens
//     4g..4g+3 of each tile.
//   * Those 8 values per lane are exactly an A operand of the P V product with tokens on the
//     contraction axis (k-slot (g, j) <-> token 16 * (j / 4) + 4g + j % 4), so P never moves
//     between lanes. P is split into a rounded high part and the rounded remainder; two
//     MFMAs (hi and lo) keep ~16 mantissa bits in the weights.
//   * V has tokens on rows and dims contiguous, but the B operand needs tokens along k. Each
//     16-token x 16-dim slice is transposed by one v_mfma_f32_16x16x16 against an identity
//     B operand (exact: products with 1 and sums with 0); its fp32 output (4 tokens of one
//     dim per lane) packs back to 16-bit without rounding and is the B operand of
//     v_mfma_f32_16x16x32 for O += P V. Where 16-bit tiles pass through LDS anyway (several
//     queries, beam groups) the B operand is read from there with transpose reads instead.
//   * Everything else (length checks, block ids staged and checked in LDS, masked loads
//     that never touch padding, base-2 online softmax in fp32, wave and partition merge) is
//     shared with the VALU path. A row outside the attended range gets an out-of-range
//     buffer offset, or in the per-lane-address mode for 8-token blocks no load under its
//     lane mask, and is zero.
//
// 8-bit float pools (OCP E4M3 codes, a float32 scale per (token, kv head) row): a lane's
// 16-byte load holds 16 codes, dims 64c' + 16g .. +15 of token row n (still 64 contiguous
// bytes of 16 rows per instruction). They widen exactly to q's 16-bit type as the A operands
// of k-blocks 2c' (dims +0..7) and 2c' + 1 (dims +8..15); Q's B operand follows the same
// assignment. Lane (n, g) holds the scores of tokens 4g .. 4g+3 of each tile, which are also
// its P entries, so one aligned 16-byte load per tile brings the four K scales (they multiply
// the scores) and one the four V scales (they multiply P before the split into hi and lo).
#include <type_traits>

#include "pa_decode_common.h"

// Cache policy of this kernel's K/V loads. Four loads of a lane cover one 64-byte piece of
// each of 16 rows, so lines are revisited by the next load: keep them cacheable.
#ifndef PA_MFMA_LOAD_POLICY
#define PA_MFMA_LOAD_POLICY 0
#endif

namespace pagedkv {
namespace mfma {

typedef __bf16 mf_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 mf_f16x8 __attribute__((ext_vector_type(8)));
typedef short mf_s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 mf_f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Mma;

template <>
struct Mma<BF16> {
    static constexpr uint32_t kOne = 0x3F80u;
    __device__ static f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(mf_bf16x8, a),
                                                      __builtin_bit_cast(mf_bf16x8, b), c, 0, 0, 0);
    }
    __device__ static f32x4 k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mf_s16x4, a),
                                                        __builtin_bit_cast(mf_s16x4, b), c, 0, 0, 0);
    }
    // Round two fp32 values to bf16 (nearest even) and pack them (x in the low half).
    __device__ static uint32_t pack_round(float x, float y) {
        const bf16x2 h = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(uint32_t, h);
    }
    __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
    __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
    // Pack two fp32 values that are exactly representable in bf16 (no rounding needed).
    __device__ static uint32_t pack_exact(float x, float y) {
        return (__float_as_uint(x) >> 16) | (__float_as_uint(y) & 0xffff0000u);
    }
};

template <>
struct Mma<F16> {
    static constexpr uint32_t kOne = 0x3C00u;
    __device__ static f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(mf_f16x8, a),
                                                     __builtin_bit_cast(mf_f16x8, b), c, 0, 0, 0);
    }
    __device__ static f32x4 k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mf_f16x4, a),
                                                    __builtin_bit_cast(mf_f16x4, b), c, 0, 0, 0);
    }
    __device__ static uint32_t pack_round(float x, float y) {
        const f16x2 h = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(uint32_t, h);
    }
    __device__ static float lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).x; }
    __device__ static float hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2, w).y; }
    __device__ static uint32_t pack_exact(float x, float y) { return pack_round(x, y); }
};

// Eight E4M3 codes (two dwords) -> the same values in T (exact), packed as an A/B operand.
__device__ __forceinline__ u32x4 widen8(F16, uint32_t w0, uint32_t w1) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.f, true))};
}
__device__ __forceinline__ u32x4 widen8(BF16, uint32_t w0, uint32_t w1) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
}

// T: type of q, out and the MFMA operands (fp16 / bf16); KV: the pool's storage (T or FP8).
// NaN sink of a multi-token workgroup: the (query, head) columns of column tile ct.
template <typename T, int D, int G>
struct MultiNanSink {
    const DecodeArgs& a;
    int q0, nq, kvh, ct;
    __device__ size_t row(int c) const {  // output row of tile column c
        const int col = 16 * ct + c;
        return (size_t)(q0 + col / G) * a.num_q_heads + kvh * G + col % G;
    }
    __device__ bool valid(int c) const { return (16 * ct + c) / G < nq; }
    __device__ void nan_outputs() const {
        for (int i = threadIdx.x; i < 16 * D; i += blockDim.x)
            if (valid(i / D)) store_elem(T{}, a.out, row(i / D) * D + i % D, __builtin_nanf(""));
    }
    __device__ void nan_records(int p) const {
        for (int i = threadIdx.x; i < 16 * (D + 2); i += blockDim.x) {
            const int c = i / (D + 2), e = i % (D + 2);
            if (!valid(c)) continue;
            const size_t rec = row(c) * a.max_partitions + p;
            if (e < D) a.ws_o[rec * D + e] = __builtin_nanf("");
            else a.ws_ml[rec * 2 + (e - D)] = (e == D) ? -INFINITY : __builtin_nanf("");
        }
    }
};

// Prologue of a beam group's partition p for kv head kvh: the nb sequences b0 .. b0 + nb - 1
// ([BlockManager essay] §4.2: sequences forked from one prompt hold references to the same
// physical blocks). Validates every beam's length (flags and NaN outputs in partition 0, as
// the decode does), stages each beam's table slice for the partition at s_bids[j * cap + i]
// (cap = partition_size / block_size entries per beam) and validates the ids (a bad id
// flags the beam and poisons its outputs or records of this partition, as the decode does).
// After it s_blen[j] is beam j's length if it takes part in this partition, else <= t0;
// ref is the beam that reads the most blocks; ncommon counts the partition's leading blocks
// on which every beam that reads the block has ref's id (one read of each serves all beams),
// the whole slice (cap) when no beam's ids differ from ref's.
// Returns false (uniformly) when no beam of the group reaches the partition.
template <typename T, int D, int G, int NT>
__device__ bool beam_prologue(const DecodeArgs& a, int p, int kvh, int b0, int nb, int* s_bids, int* s_blen,
                              int* s_bbad, Partition& part, int& ref, int& ncommon) {
    const int tid = threadIdx.x;
    const int P = a.partition_size;
    const int lbs = a.log2_block_size;
    const int cap = P >> lbs;
    const int t0 = p * P;
    const int j0 = t0 >> lbs;
    if (tid < nb) {
        const int L = a.context_lens[b0 + tid];
        int flag = 0;
        if (L <= 0) flag = PA_FLAG_EMPTY_CONTEXT;
        else if (L > a.max_context_len || ((L - 1) >> lbs) >= a.max_blocks_per_seq) flag = PA_FLAG_BAD_LENGTH;
        if (flag && p == 0 && a.err_flag) atomicOr(a.err_flag, flag);
        s_blen[tid] = flag ? -1 : L;
        s_bbad[tid] = flag && p == 0;  // partition 0 writes the NaN outputs of a bad length
    }
    __syncthreads();
    for (int i = tid; i < nb * G * D; i += NT) {
        const int j = i / (G * D);
        if (s_bbad[j]) store_elem(T{}, a.out, ((size_t)(b0 + j) * a.num_q_heads + kvh * G) * D + i % (G * D),
                                  __builtin_nanf(""));
    }
    __syncthreads();
    if (tid < nb) s_bbad[tid] = 0;
    __syncthreads();
    for (int i = tid; i < nb * cap; i += NT) {
        const int j = i / cap;
        const int k = i - j * cap;
        const int L = s_blen[j];
        if (L <= t0) continue;  // bad length, or the beam ends before this partition
        const int nids = ((min(L, t0 + P) - 1) >> lbs) - j0 + 1;
        if (k >= nids) continue;
        int id = a.block_table[(size_t)(b0 + j) * a.max_blocks_per_seq + j0 + k];
        if ((unsigned)id >= (unsigned)a.num_blocks) {
            s_bbad[j] = 1;
            id = 0;
        }
        s_bids[i] = id;
    }
    __syncthreads();
    for (int i = tid; i < nb * G * (D + 2); i += NT) {
        const int j = i / (G * (D + 2));
        if (!s_bbad[j]) continue;
        const int r = i - j * (G * (D + 2));
        const int h = r / (D + 2);
        const int e = r - h * (D + 2);
        const size_t row = (size_t)(b0 + j) * a.num_q_heads + kvh * G + h;
        if ((s_blen[j] + P - 1) / P == 1) {
            if (e < D) store_elem(T{}, a.out, row * D + e, __builtin_nanf(""));
        } else {
            const size_t rec = row * a.max_partitions + p;
            if (e < D) a.ws_o[rec * D + e] = __builtin_nanf("");
            else a.ws_ml[rec * 2 + (e - D)] = (e == D) ? -INFINITY : __builtin_nanf("");
        }
    }
    if (tid < nb && s_bbad[tid] && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_BLOCK_ID);
    __syncthreads();
    __shared__ int s_first;  // the first block (of the slice) where some beam leaves ref's ids
    if (tid < nb && s_bbad[tid]) s_blen[tid] = -1;
    if (tid == 0) s_first = cap;
    __syncthreads();
    ref = -1;
    int end = t0;
    for (int j = 0; j < nb; ++j) {
        const int t1 = min(s_blen[j], t0 + P);
        if (t1 > end) {
            end = t1;
            ref = j;
        }
    }
    if (ref < 0) return false;
    int first = cap;
    for (int i = tid; i < nb * cap; i += NT) {
        const int j = i / cap;
        const int k = i - j * cap;
        const int L = s_blen[j];
        if (L <= t0 || j == ref) continue;
        if (k < ((min(L, t0 + P) - 1) >> lbs) - j0 + 1 && s_bids[i] != s_bids[ref * cap + k]) first = min(first, k);
    }
    if (first < cap) atomicMin(&s_first, first);
    __syncthreads();
    ncommon = s_first;
    part.nparts = 0;
    part.t0 = t0;
    part.rel_lo = 0;
    part.ntok = end - t0;
    part.j0 = j0;
    part.len = 0;
    part.npos = -1;
    part.slot = -1;
    return true;
}

// kMulti = false: one query per sequence, column n of the B operand is head kvh * G + n.
// kMulti = true: several queries per sequence (query_start), columns are (query, head)
// pairs taken query-major, 16 per workgroup (column tile blockIdx.y % col_tiles); query i of
// a sequence with n new tokens sits at position L - n + i and its column sees tokens up to
// that position only (causal mask inside the valid range).
// kBeams = true: one query per sequence, columns are (beam, head) pairs taken beam-major
// over the beams of group blockIdx.y (beam_prologue); a partition whose blocks all beams
// share is streamed once for all of them, else once per beam with the other beams' columns
// masked.
// True when every block of the pool lies within 2 GiB of the pool's start, so one buffer
// resource with 32-bit offsets reaches any two blocks (8-token-block mode 2).
inline bool pool_within_2gib(const DecodeArgs& a) {
    return (uint64_t)a.num_blocks * (uint64_t)a.block_stride <= 0x7fffffffull;
}

template <typename T, typename KV, int D, int G, int NW, bool kDoubleBuffer, bool kMulti = false,
          bool kBeams = false, int kSmallBlocks = 0>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kSmallBlocks == 1 && D == 128 && (KV::kBytes == 2 || kMulti || kBeams) ? 1 : 2))) void decode_mfma_kernel(DecodeArgs a) {
    static_assert(T::kBytes == 2, "matrix-core operands are 16-bit");
    static_assert(G >= 1 && G <= 16, "at most 16 query heads per kv head");
    static_assert(!(kMulti && kBeams), "one column mapping");
    // 8-token blocks (kSmallBlocks != 0): a 16-row tile spans two blocks. Mode 1 addresses
    // each row from its lane (64-bit addresses; 16-bit rows of 128 dims then need the registers
    // of a second wave). Mode 2 (16-bit pools lying within 2 GiB) reads both blocks through one
    // buffer and keeps two waves per SIMD.
    static_assert(kSmallBlocks == 0 || D <= 128, "8-token blocks: head_dim up to 128");
    static_assert(kSmallBlocks != 2 || KV::kBytes == 2, "mode 2: 16-bit pools");
    constexpr int NCOL = (kMulti || kBeams) ? 16 : G;  // columns whose results this workgroup keeps
    constexpr bool kFp8 = std::is_same_v<KV, FP8>;
    constexpr int NC = D / 32;             // 32-dim k-blocks of the score contraction
    constexpr int NL = D * KV::kBytes / 64;  // 16-byte loads per lane per tile row (64 B of each row)
    constexpr int NS = D / 16;             // 16-dim output slices
    constexpr int kChunk = 32;             // tokens per wave iteration (two 16-token tiles)
    using M = Mma<T>;

    __shared__ int s_ids[kBeams ? kMaxBeamIds : kMaxIdsPerPartition];
    __shared__ int s_blen[kBeams ? 16 : 1];  // beam groups: lengths of the beams in this partition
    __shared__ int s_bbad[kBeams ? 16 : 1];
    __shared__ float s_m[NW][NCOL];
    __shared__ float s_l[NW][NCOL];
    __shared__ float s_acc[NW][NCOL][D];
    // 16-bit rows of 256 bytes, several queries or beams: tiles are loaded with whole rows per
    // lane group (coalesced) and turned into the operand layout through this wave-private LDS
    // region. The operand-layout loads give the L1 one access per lane; restaging measured
    // 23% faster with 4 queries per sequence (32 sequences of 2049 tokens, 64 query / 8 kv
    // heads) and 2% with beam groups (8 groups of 4 beams at 32K tokens),
    // but 3-4% slower for the one-query decode, which keeps the direct loads.
    constexpr bool kStage = D == 128 && (kMulti || kBeams) && kSmallBlocks == 0;
    // Staged 16-bit V tiles stay in LDS, and the B operand of P V comes from transpose reads
    // (ds_read_b64_tr_b16) instead of identity-MFMA transposes: 12% faster with 4 queries per
    // sequence on that 64 / 8-head batch, equal elsewhere. The one-query decode measured the
    // same with it (staged, 4 or 8 waves), so it keeps the direct loads.
    constexpr bool kTrV = kStage && KV::kBytes == 2;
    constexpr int kCpr = D * KV::kBytes / 16;  // 16-byte chunks per row (16 or 8)
    constexpr int kRpl = 64 / kCpr;            // rows per staged load instruction (4 or 8)
    __shared__ u32x4 s_stage[kStage ? NW : 1][kStage ? 2 * 16 * kCpr : 1];
    // the new token's K and V rows as read, and for an 8-bit pool each wave's record of them
    // (fused append of the decode)
    constexpr bool kAppendable = !kMulti && !kBeams;
    using R = NewRec<KV, D>;
    constexpr int kRaw = NewRec<T, D>::kBytes;
    __shared__ __align__(16) char s_new[kAppendable ? kRaw + (kFp8 ? NW * R::kBytes : 0) : 16];

    const int p = grid_partition();
    const int kvh = blockIdx.x;
    const int b = kMulti ? (int)blockIdx.y / a.col_tiles : (int)blockIdx.y;
    const int ct = kMulti ? (int)blockIdx.y - b * a.col_tiles : 0;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int g = lane >> 4;
    const int lbs = a.log2_block_size;
    const int bs = 1 << lbs;

    // This lane's column: a head of the group (decode) or a (query, head) pair.
    int q0 = 0, nq = 1;
    if constexpr (kMulti) {
        q0 = a.query_start[b];
        nq = a.query_start[b + 1] - q0;
        // query rows outside q, or more queries than the launch has column tiles for: flagged,
        // and those rows are not written
        if (q0 < 0 || nq < 0 || q0 + nq > a.num_q_tokens || nq * G > 16 * a.col_tiles) {
            if (p == 0 && kvh == 0 && ct == 0 && threadIdx.x == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_LENGTH);
            return;
        }
        if (16 * ct >= nq * G) return;  // no query of this sequence in this tile (uniform)
    }
    // beam groups: sequences b0 .. b0 + nb - 1; column n is head n % G of beam n / G
    const int b0 = kBeams ? (int)blockIdx.y * a.beam_width : b;
    const int nb = kBeams ? min(a.beam_width, a.batch - b0) : 1;
    const int col = 16 * ct + n;
    const int qi = kMulti ? col / G : 0;       // query of the column
    const int qh = kMulti ? col - qi * G : (kBeams ? n % G : n);  // head of the column inside the group
    const bool col_valid = kMulti ? qi < nq : (kBeams ? n < nb * G : n < G);

    if constexpr (!kMulti && !kBeams) {
        if (partition_is_dead(a, p, b)) return;
    }
    if constexpr (kBeams) {  // a later partition no beam of the group reaches: leave before any load
        if (PA_EARLY_DEAD_CHECK && p > 0) {
            bool live = false;
            for (int j = 0; j < nb; ++j) {
                const int L = a.context_lens[b0 + j];
                live |= L > p * a.partition_size && L <= a.max_context_len;
            }
            if (!live) return;
        }
    }
    // Q as the B operand of S^T = K Q^T (zero in invalid columns); k-block c of lane group g
    // holds the dims the K operand gives it: 32c + 8g .. +7 for 16-bit pools, 64(c/2) + 16g +
    // 8(c%2) .. +7 for 8-bit pools.
    u32x4 qb[NC];
    {
        const size_t qrow_idx = kMulti   ? (size_t)(q0 + (col_valid ? qi : 0)) * a.num_q_heads + kvh * G + qh
                                : kBeams ? (size_t)(b0 + (col_valid ? n / G : 0)) * a.num_q_heads + kvh * G + qh
                                         : (size_t)b * a.num_q_heads + kvh * G + (col_valid ? n : 0);
        const char* qrow = static_cast<const char*>(a.q) + qrow_idx * D * 2;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int d0 = kFp8 ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
            qb[c] = col_valid ? load16(qrow + 2 * d0) : u32x4{0, 0, 0, 0};
        }
    }
    Partition part;
    int bref = 0;     // beam groups: the beam whose table is streamed over the shared blocks
    int bcommon = 0;  // beam groups: leading blocks of the partition every beam shares
    if constexpr (kBeams) {
        if (!beam_prologue<T, D, G, NW * 64>(a, p, kvh, b0, nb, s_ids, s_blen, s_bbad, part, bref, bcommon)) return;
    } else if constexpr (kMulti) {
        if (!partition_prologue_sink<T, D, NW * 64>(a, p, b, max(nq, 1), MultiNanSink<T, D, G>{a, q0, nq, kvh, ct},
                                                    s_ids, part))
            return;
    } else {
        if (!partition_prologue<T, D, G, NW * 64>(a, p, kvh, b, s_ids, part, kAppendable ? s_new : nullptr))
            return;
    }
    int ntok = part.ntok;
    int lim_col = ntok;  // tokens (relative to the partition) this lane's column may see
    if constexpr (kMulti) {
        const int first_pos = part.len - nq;  // position of query 0
        const int last_q = min(16 * ct + 15, nq * G - 1) / G;
        const int tile_end = first_pos + last_q + 1 - part.t0;  // tokens the tile's last query sees
        if (tile_end <= 0) return;  // the whole partition is after this tile's queries (uniform)
        ntok = min(ntok, tile_end);
        lim_col = col_valid ? min(ntok, first_pos + qi + 1 - part.t0) : 0;
    }
    int rel_lo = part.rel_lo;
    int c0 = rel_lo / kChunk;  // first chunk holding an attended token
    // tokens every column of the wave sees: ntok for the decode; for several queries the
    // tile's first query's limit when all 16 columns are valid (else the masked path)
    int lim_wave = ntok;
    if constexpr (kMulti) {
        const int first_pos = part.len - nq;
        lim_wave = 16 * ct + 15 < nq * G ? min(ntok, first_pos + (16 * ct) / G + 1 - part.t0) : 0;
    }
    // the table slice streamed: the sequence's, or in a beam group the reference beam's
    const int* ids = s_ids;
    const int bcap = kBeams ? a.partition_size >> a.log2_block_size : 0;
    // beam groups: a beam's column sees its own tokens of the partition
    auto beam_end = [&](int j) { return min(s_blen[j], part.t0 + a.partition_size) - part.t0; };

    // Identity B operand of the 16x16x16 transpose: k-slot (g, i) is 1 in column 4g + i.
    u32x2 ident;
    ident.x = ((4 * g + 0 == n) ? M::kOne : 0u) | (((4 * g + 1 == n) ? M::kOne : 0u) << 16);
    ident.y = ((4 * g + 2 == n) ? M::kOne : 0u) | (((4 * g + 3 == n) ? M::kOne : 0u) << 16);

    const size_t head_bytes = (size_t)bs * D * KV::kBytes;
    const size_t block_bytes = (size_t)a.block_stride;
    const char* kpool = static_cast<const char*>(a.k_pool);
    const char* vpool = static_cast<const char*>(a.v_pool);
    const uint32_t slab_bytes = (uint32_t)head_bytes;
    const uint32_t seg = 16u * g;  // lane group g reads bytes 64c + 16g .. +15 of a row
    int niters = (ntok - c0 * kChunk + kChunk * NW - 1) / (kChunk * NW);

    // Loads of one chunk: tile t rows are tokens rel + 16t + n; lanes past the partition end
    // read zeros through an out-of-range offset. With 8-bit pools, ks/vs[t] are the scales
    // of tokens rel + 16t + 4g .. +3 (the rows of this lane's scores), loaded whole when the
    // tile starts inside the partition and cleared per token before use.
    auto issue = [&](int it, u32x4 (*kk)[NL], u32x4 (*vv)[NL], u32x4* ks, u32x4* vs) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int rel = (c0 + it * NW + wave) * kChunk + 16 * t;  // wave-uniform
            if constexpr (kSmallBlocks == 1) {
                // 8-token blocks, per-lane addresses: rows 0-7 and 8-15 of the tile lie in two
                // blocks, and each lane looks up the block of its own row. A row outside
                // [rel_lo, ntok) reads the partition's first attended row instead (a valid
                // row whose line the workgroup reads anyway, never a padding slot); its score
                // is masked, so its weight is 0 on finite values. The loads take no branch, so
                // the waits of the double buffer stay exact.
                const int tok = rel + n;
                const bool live = tok < ntok && tok >= rel_lo;
                const int rt = live ? tok : rel_lo;
                const size_t row = (size_t)ids[rt >> lbs] * block_bytes + (size_t)kvh * head_bytes +
                                   (size_t)((rt & (bs - 1)) * D * KV::kBytes) + seg;
#pragma unroll
                for (int c = 0; c < NL; ++c) {
                    kk[t][c] = load16(kpool + row + 64 * c);
                    vv[t][c] = load16(vpool + row + 64 * c);
                }
                if constexpr (kFp8) {
                    // scales of tokens rel + 4g .. +3 (one aligned 16-byte word of one block);
                    // a word with none of the four attended reads the word of the first
                    // attended token instead, and scales of unattended tokens are replaced by
                    // 0 before use
                    const int tok4 = rel + 4 * g;
                    const int st = tok4 < ntok && tok4 + 3 >= rel_lo ? tok4 : (rel_lo & ~3);
                    const size_t srow = (((size_t)ids[st >> lbs] * a.num_kv_heads + kvh) << lbs) + (st & (bs - 1));
                    ks[t] = load16(a.k_scale + srow);
                    vs[t] = load16(a.v_scale + srow);
                }
                continue;
            } else if constexpr (kSmallBlocks == 2) {
                // 8-token blocks, 16-bit pools, one buffer over the tile's two blocks (the host
                // picks this mode only when the whole pool lies within 2 GiB, so any two
                // blocks do): 32-bit offsets, and a row outside [rel_lo, ntok) gets an
                // out-of-range offset and reads zeros without a memory access.
                const int j0 = rel < ntok ? rel >> lbs : 0;
                const int j1 = rel + 8 < ntok ? (rel >> lbs) + 1 : j0;
                const int id0 = __builtin_amdgcn_readfirstlane(ids[j0]);
                const int id1 = __builtin_amdgcn_readfirstlane(ids[j1]);
                const bool live = rel + n < ntok && rel + n >= rel_lo;
                const int lo = min(id0, id1);
                const size_t base = (size_t)lo * block_bytes + (size_t)kvh * head_bytes;
                const uint32_t nrec = (uint32_t)((size_t)(max(id0, id1) - lo) * block_bytes) + slab_bytes;
                const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + base, nrec);
                const __amdgpu_buffer_rsrc_t rv = make_rsrc(vpool + base, nrec);
                const uint32_t off = live ? (uint32_t)((size_t)((n < 8 ? id0 : id1) - lo) * block_bytes) +
                                                (uint32_t)((n & 7) * D * KV::kBytes) + seg
                                          : kOutOfRange;
#pragma unroll
                for (int c = 0; c < NL; ++c) {
                    kk[t][c] = buffer_load16<PA_MFMA_LOAD_POLICY>(rk, off + 64 * c);
                    vv[t][c] = buffer_load16<PA_MFMA_LOAD_POLICY>(rv, off + 64 * c);
                }
                continue;
            }
            const int id = __builtin_amdgcn_readfirstlane(ids[(rel < ntok ? rel : 0) >> lbs]);  // partitions start on a block
            const size_t slab = (size_t)id * block_bytes + (size_t)kvh * head_bytes;
            const uint32_t off = (rel + n < ntok && rel + n >= rel_lo)
                                     ? (uint32_t)(((rel & (bs - 1)) + n) * D * KV::kBytes) + seg
                                     : kOutOfRange;
            const __amdgpu_buffer_rsrc_t rk = make_rsrc(kpool + slab, slab_bytes);
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(vpool + slab, slab_bytes);
#pragma unroll
            for (int c = 0; c < NL; ++c) {
                // staged: load c covers kRpl whole rows (lane: row kRpl c + lane / kCpr, chunk
                // lane % kCpr); else 64 bytes of each of the 16 rows (the operand layout)
                const int srow = kRpl * c + lane / kCpr;
                const uint32_t so = (rel + srow < ntok && rel + srow >= rel_lo)
                                        ? (uint32_t)(((rel & (bs - 1)) + srow) * D * KV::kBytes + 16 * (lane % kCpr))
                                        : kOutOfRange;
                const uint32_t o = kStage ? so : (off == kOutOfRange ? kOutOfRange : off + 64 * c);
                kk[t][c] = buffer_load16<PA_MFMA_LOAD_POLICY>(rk, o);
                vv[t][c] = buffer_load16<PA_MFMA_LOAD_POLICY>(rv, o);
            }
            if constexpr (kFp8) {
                // scales of tokens rel + 4g .. +3 (the rows of this lane's scores): one aligned
                // 16-byte word, not read when none of the four is attended
                const size_t srow = ((size_t)id * a.num_kv_heads + kvh) << lbs;  // this slab's scales
                const int tok4 = rel + 4 * g;
                const uint32_t so = tok4 < ntok && tok4 + 3 >= rel_lo ? (uint32_t)(((rel & (bs - 1)) + 4 * g) * 4)
                                                                       : kOutOfRange;
                ks[t] = buffer_load16<PA_MFMA_LOAD_POLICY>(make_rsrc(a.k_scale + srow, (uint32_t)bs * 4), so);
                vs[t] = buffer_load16<PA_MFMA_LOAD_POLICY>(make_rsrc(a.v_scale + srow, (uint32_t)bs * 4), so);
            }
        }
    };

    float m = -INFINITY;  // running base-2 max of head n (same in all four lane groups)
    float l = 0.f;        // this lane's part of head n's running sum
    f32x4 acc[NS];        // acc[s][i] = O[head 4g + i][dim of column n in slice s]
#pragma unroll
    for (int s = 0; s < NS; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int npos = part.npos;
    // this wave's record of the new rows in the pool's storage (8-bit: quantised below)
    char* s_rec = s_new + (kFp8 ? kRaw + wave * R::kBytes : 0);
    // Staged tiles to the operand layout, in place: lane (n, g) gets row n, chunk 4c + g of
    // load c. Chunk j of row r sits at j ^ (r mod kCpr) in LDS, so the writes (whole rows) and
    // the reads (one chunk of 16 rows) spread over the banks. The region is the wave's own and
    // LDS operations of a wave complete in order: no barrier.
    auto restage = [&](u32x4 (*x)[NL]) {
        if constexpr (kStage) {
            u32x4* w = s_stage[wave];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < NL; ++c) {
                    const int r = kRpl * c + lane / kCpr;
                    w[(16 * t + r) * kCpr + ((lane % kCpr) ^ (r % kCpr))] = x[t][c];
                }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < NL; ++c) x[t][c] = w[(16 * t + n) * kCpr + ((4 * c + g) ^ (n % kCpr))];
        }
    };
    // V tiles for transpose reads: whole rows written as loaded, chunk j of row r at
    // j ^ (2r mod kCpr), so that the transpose reads (four rows, two chunks per lane group)
    // and the row writes both spread over the banks.
    auto vswz = [&](int r) { return (2 * r) & (kCpr - 1); };
    auto stage_v = [&](u32x4 (*x)[NL]) {
        if constexpr (kTrV) {
            u32x4* w = s_stage[wave];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < NL; ++c) {
                    const int r = kRpl * c + lane / kCpr;
                    w[(16 * t + r) * kCpr + ((lane % kCpr) ^ vswz(r))] = x[t][c];
                }
        }
    };
    // B operand of P V for output slice s from the staged V tiles: lane (n, g) gets dim
    // 16s + n at tokens 4g .. 4g+3 of tile 0, then of tile 1 (the k-slots of P's A operand).
    // ds_read_b64_tr_b16 gives lane i of a 16-lane group, as its value k (k = 0..3), 16-bit
    // element i % 4 of the 8-byte piece that lane i / 4 + 4k of the group addresses. So lane n
    // addresses row 4g + n / 4, dims 16s + 4 (n % 4) .. +3.
    auto tr_v = [&](int s) {
        const u32x4* w = s_stage[wave];
        const int r = 4 * g + (n >> 2);
        const int j = 2 * s + ((n & 3) >> 1);  // 16-byte chunk of dims 16s + 4 (n % 4) ..
        u32x4 vb;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const char* piece = reinterpret_cast<const char*>(w + (16 * t + r) * kCpr + (j ^ vswz(r))) + 8 * (n & 1);
            const mf_s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) mf_s16x4*)(const_cast<char*>(piece)));
            const u32x2 y = __builtin_bit_cast(u32x2, x);
            vb[2 * t] = y.x;
            vb[2 * t + 1] = y.y;
        }
        return vb;
    };
    auto compute = [&](int it, u32x4 (*kk)[NL], u32x4 (*vv)[NL], u32x4* ks, u32x4* vs) {
        const int rel0 = (c0 + it * NW + wave) * kChunk;
        restage(kk);
        if constexpr (kTrV) stage_v(vv);
        else restage(vv);
        if constexpr (kAppendable) {
            if (npos >= 0) {  // fused append: the new token's rows come from s_new (wave-uniform test)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int d = npos - (rel0 + 16 * t);
                    if (d >= 0 && d < 16) {
                        if (n == d) {  // the A-operand row of the token
#pragma unroll
                            for (int c = 0; c < NL; ++c) {
                                kk[t][c] = *reinterpret_cast<const u32x4*>(s_rec + 64 * c + seg);
                                if constexpr (!kTrV)
                                    vv[t][c] = *reinterpret_cast<const u32x4*>(s_rec + R::kRowBytes + 64 * c + seg);
                            }
                        }
                        if constexpr (kTrV) {  // the staged V row of the token
                            if (lane < kCpr)
                                s_stage[wave][(16 * t + d) * kCpr + (lane ^ vswz(d))] =
                                    *reinterpret_cast<const u32x4*>(s_rec + R::kRowBytes + 16 * lane);
                        }
                        if constexpr (kFp8) {  // the lanes whose scores include the token
                            if (g == (d >> 2)) {
                                const uint32_t* sc = reinterpret_cast<const uint32_t*>(s_rec + 2 * R::kRowBytes);
                                ks[t][d & 3] = sc[0];
                                vs[t][d & 3] = sc[1];
                            }
                        }
                    }
                }
            }
        }
        float sc[8];
        float vscale[8];  // V scale of each P entry (8-bit pools)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
            if constexpr (kFp8) {
#pragma unroll
                for (int c = 0; c < NL; ++c) {
                    st = M::k32(widen8(T{}, kk[t][c][0], kk[t][c][1]), qb[2 * c], st);
                    st = M::k32(widen8(T{}, kk[t][c][2], kk[t][c][3]), qb[2 * c + 1], st);
                }
            } else {
#pragma unroll
                for (int c = 0; c < NC; ++c) st = M::k32(kk[t][c], qb[c], st);
            }
            if (rel0 >= rel_lo && rel0 + kChunk <= lim_wave) {  // the whole chunk is visible (wave-uniform)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float d = st[i];
                    if constexpr (kFp8) {
                        d *= __uint_as_float(ks[t][i]);
                        vscale[4 * t + i] = __uint_as_float(vs[t][i]);
                    }
                    sc[4 * t + i] = d * a.scale_log2;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tok = rel0 + 16 * t + 4 * g + i;
                    const bool live = tok < lim_col && tok >= rel_lo;
                    float d = st[i];
                    if constexpr (kFp8) {
                        d *= __uint_as_float(ks[t][i]);
                        vscale[4 * t + i] = live ? __uint_as_float(vs[t][i]) : 0.f;
                    }
                    sc[4 * t + i] = live ? d * a.scale_log2 : -INFINITY;
                }
            }
        }
        float cm = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) cm = fmaxf(cm, sc[j]);
        cm = fmaxf(cm, shfl_xor(cm, 16));
        cm = fmaxf(cm, shfl_xor(cm, 32));
        // The reference max m moves only when a column's chunk max exceeds it by more than 2^8
        // (weights then stay below 256, far inside fp32 and the split of P into high and low
        // parts), so most chunks skip rescaling the accumulators; m and l stay a consistent
        // pair for the normalisation and the partition records whichever reference is used.
        const bool grow = cm > m + 8.f;
        if (__any(grow)) {
            const float mn = grow ? cm : m;
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m - mn);
            m = mn;
            l *= alpha;
            // rows 4g + i of acc belong to columns 4g + i: fetch their factors from those lanes
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
        // P as the A operand (times the V scales for 8-bit pools), split into rounded high and
        // low parts
        if constexpr (kFp8) {
#pragma unroll
            for (int j = 0; j < 8; ++j) pr[j] *= vscale[j];
        }
        u32x4 phi, plo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t h = M::pack_round(pr[2 * w], pr[2 * w + 1]);
            phi[w] = h;
            plo[w] = M::pack_round(pr[2 * w] - M::lo(h), pr[2 * w + 1] - M::hi(h));
        }
        if constexpr (kTrV) {
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const u32x4 vb = tr_v(s);
                acc[s] = M::k32(phi, vb, acc[s]);
                acc[s] = M::k32(plo, vb, acc[s]);
            }
            return;
        }
        // V rows as 16-bit words: vw[t][c] holds the 8 dims of token row n that k-block c of
        // lane group g covers
        u32x4 vw[2][NC];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                if constexpr (kFp8) {
                    vw[t][c] = (c & 1) ? widen8(T{}, vv[t][c >> 1][2], vv[t][c >> 1][3])
                                       : widen8(T{}, vv[t][c >> 1][0], vv[t][c >> 1][1]);
                } else {
                    vw[t][c] = vv[t][c];
                }
            }
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int c = s >> 1;
            f32x4 vt[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x2 half = (s & 1) ? u32x2{vw[t][c][2], vw[t][c][3]} : u32x2{vw[t][c][0], vw[t][c][1]};
                vt[t] = M::k16(half, ident, f32x4{0.f, 0.f, 0.f, 0.f});
            }
            const u32x4 vb = {M::pack_exact(vt[0][0], vt[0][1]), M::pack_exact(vt[0][2], vt[0][3]),
                              M::pack_exact(vt[1][0], vt[1][1]), M::pack_exact(vt[1][2], vt[1][3])};
            acc[s] = M::k32(phi, vb, acc[s]);
            acc[s] = M::k32(plo, vb, acc[s]);
        }
    };

    u32x4 ka[2][NL], va[2][NL], ksa[2], vsa[2];
    // One pass over the partition. A beam group takes pass 0 over the leading blocks all its
    // beams share (read once, through the reference beam's ids, for every beam's columns; the
    // wave's fast path needs the shortest beam), then pass 1 + j over beam j's tokens after
    // them (its own blocks), the other beams' columns seeing nothing.
    const int npasses = kBeams ? 1 + nb : 1;
    for (int pass = 0; pass < npasses; ++pass) {
    if constexpr (kBeams) {
        const int cend = min(bcommon << lbs, part.ntok);  // tokens in the shared blocks
        if (pass == 0) {
            if (cend == 0) continue;
            ids = s_ids + bref * bcap;
            ntok = cend;
            rel_lo = 0;
            lim_col = col_valid && s_blen[n / G] > part.t0 ? min(beam_end(n / G), cend) : 0;
            lim_wave = cend;
            for (int j = 0; j < nb; ++j)
                if (s_blen[j] > part.t0) lim_wave = min(lim_wave, beam_end(j));
        } else {
            const int j = pass - 1;
            if (s_blen[j] <= part.t0 || beam_end(j) <= cend) continue;
            ids = s_ids + j * bcap;
            ntok = beam_end(j);
            rel_lo = cend;
            lim_col = col_valid && n / G == j ? ntok : 0;
            lim_wave = 0;
        }
        c0 = rel_lo / kChunk;
        niters = (ntok - c0 * kChunk + kChunk * NW - 1) / (kChunk * NW);
    }
    if constexpr (kDoubleBuffer) {
        u32x4 kb[2][NL], vb[2][NL], ksb[2], vsb[2];
        issue(0, ka, va, ksa, vsa);
        issue(1, kb, vb, ksb, vsb);
        if constexpr (kAppendable && kFp8) {
            if (npos >= 0) quantize_new_rows<T, D>(s_new, s_rec);  // while the first loads fly
        }
        int it = 0;
        for (; it + 1 < niters; it += 2) {
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
    } else {
        if constexpr (kAppendable && kFp8) {
            if (npos >= 0) quantize_new_rows<T, D>(s_new, s_rec);
        }
        for (int it = 0; it < niters; ++it) {
            issue(it, ka, va, ksa, vsa);
            compute(it, ka, va, ksa, vsa);
        }
    }
    }

    // column n's sum over the four lane groups
    l += shfl_xor(l, 16);
    l += shfl_xor(l, 32);
    if (g == 0 && n < NCOL) {
        s_m[wave][n] = m;
        s_l[wave][n] = l;
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int c = s >> 1;  // column n of slice s
        const int dim = kTrV ? 16 * s + n
                             : (kFp8 ? 64 * (c >> 1) + 16 * (n >> 2) + 8 * (c & 1) : 32 * c + 8 * (n >> 2)) +
                                   4 * (s & 1) + (n & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * g + i < NCOL) s_acc[wave][4 * g + i][dim] = acc[s][i];
    }
    __syncthreads();
    if constexpr (kMulti) {
        // merge the waves per column; one output row (single partition) or record per column
        const MultiNanSink<T, D, G> rows{a, q0, nq, kvh, ct};
        for (int i = threadIdx.x; i < 16 * D; i += NW * 64) {
            const int c = i / D;
            const int e = i % D;
            if (!rows.valid(c)) continue;
            float M = s_m[0][c];
#pragma unroll
            for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][c]);
            const float Ms = (M == -INFINITY) ? 0.f : M;
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = __builtin_amdgcn_exp2f(s_m[w][c] - Ms);
                num = fmaf(s_acc[w][c][e], f, num);
                den = fmaf(s_l[w][c], f, den);
            }
            const size_t r = rows.row(c);
            if (part.nparts == 1) {
                store_elem(T{}, a.out, r * D + e, num / den);
            } else {
                const size_t rec = r * a.max_partitions + p;
                a.ws_o[rec * D + e] = num / den;
                if (e == 0) {
                    a.ws_ml[rec * 2] = M;
                    a.ws_ml[rec * 2 + 1] = den;
                }
            }
        }
    } else if constexpr (kBeams) {
        // merge the waves per (beam, head) column: the output row (the beam's only partition)
        // or the partition record
        const int P = a.partition_size;
        for (int i = threadIdx.x; i < 16 * D; i += NW * 64) {
            const int c = i / D;
            const int e = i % D;
            if (c >= nb * G) continue;
            const int L = s_blen[c / G];
            if (L <= part.t0) continue;  // the beam does not reach this partition, or is poisoned
            float M = s_m[0][c];
#pragma unroll
            for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][c]);
            const float Ms = (M == -INFINITY) ? 0.f : M;
            float num = 0.f, den = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = __builtin_amdgcn_exp2f(s_m[w][c] - Ms);
                num = fmaf(s_acc[w][c][e], f, num);
                den = fmaf(s_l[w][c], f, den);
            }
            const size_t r = (size_t)(b0 + c / G) * a.num_q_heads + kvh * G + c % G;
            if ((L + P - 1) / P == 1) {
                store_elem(T{}, a.out, r * D + e, num / den);
            } else {
                const size_t rec = r * a.max_partitions + p;
                a.ws_o[rec * D + e] = num / den;
                if (e == 0) {
                    a.ws_ml[rec * 2] = M;
                    a.ws_ml[rec * 2 + 1] = den;
                }
            }
        }
    } else {
        partition_epilogue<T, D, G, NW>(a, p, kvh, b, part, s_m, s_l, s_acc);
        if constexpr (kAppendable) {
            // wave 0's record (every wave's is the same; the barrier above orders it)
            if (part.npos >= 0 && !a.ws_slot) store_new_rows<KV, D, NW * 64>(a, part.slot, kvh, 1, s_new + (kFp8 ? kRaw : 0));
        }
    }
}

}  // namespace mfma
}  // namespace pagedkv
