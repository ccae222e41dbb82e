// Pieces shared by the decode kernels: the per-partition prologue (length checks, block-id
// staging in LDS) and the epilogue (merge of per-wave softmax states, output or partition
// record). Every function here is called by all threads of the workgroup.
#pragma once

#include <type_traits>

#include "pa_kernels.h"

namespace pagedkv {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * 64;

// Grid of the decode kernels: x = kv head (or group of kv heads), y = sequence (times the
// column tiles of a multi-token launch), z = partition. Work-groups are dealt to the 8 XCDs
// round-robin in linear order, x fastest, so every XCD gets an equal share of every
// partition index. (With the partition fastest, a partition count that is a multiple of 4
// sends every first partition, the only live one of a short sequence, to 2 of the 8 XCDs:
// twice the time on long-tailed lengths. Taking the last partitions first, so that the
// longest sequences start early, measured slower than this order: the dead work-groups of
// the late partitions then all queue ahead of the live ones.)
__device__ __forceinline__ int grid_partition() { return (int)blockIdx.z; }

struct Partition {
    int nparts;  // partitions of this sequence
    int t0;      // first position of this partition (a block multiple)
    int rel_lo;  // first attended token, relative to t0 (< block_size; 0 unless a window starts inside)
    int ntok;    // end of the attended tokens, relative to t0
    int j0;      // logical block of t0: s_ids[i] is the id of block j0 + i
    int len;     // the sequence's context length
    int npos;    // fused append: the new token's position relative to t0 (its rows are in s_new, and
                 // the workgroup ends with store_new_rows), or -1
    int slot;    // fused append: the new token's slot (when npos >= 0)
};

// First attended position of a sequence of length L: a sliding window keeps the last
// `window` tokens ([Valid-length essay] §3.3, §5.3), otherwise everything.
__device__ __forceinline__ int window_start(const DecodeArgs& a, int L) {
    return (a.window > 0 && L > a.window) ? L - a.window : 0;
}

// Position at which partition 0 of a sequence of length L starts: the start of the block
// holding the first attended token (0 without a window). Partitions tile [base, L).
__device__ __forceinline__ int partition_base(const DecodeArgs& a, int L) {
    return (window_start(a, L) >> a.log2_block_size) << a.log2_block_size;
}

// A work-group whose partition lies past the end of its sequence (or of a sequence with an
// invalid length, which partition 0 reports) has nothing to do. Partitions after the first
// check this before issuing any other load: a wave cannot retire while its loads are in
// flight, so a dead work-group that had issued its q and table loads would hold its slot
// for a whole memory round trip, and a launch sized for a loose max_context_len has many of
// them. Live later partitions pay one short extra round trip for the length.
#ifndef PA_EARLY_DEAD_CHECK
#define PA_EARLY_DEAD_CHECK 1
#endif
__device__ __forceinline__ bool partition_is_dead(const DecodeArgs& a, int p, int b) {
    if (!PA_EARLY_DEAD_CHECK || p == 0) return false;
    const int L = a.context_lens[b];
    if (L <= 0 || L > a.max_context_len) return true;
    return partition_base(a, L) + p * a.partition_size >= L;
}

// True on every thread when pred is true on any thread of the work-group of NT threads: one
// ballot per wave, one LDS word per wave, one barrier. (The runtime's work-group OR reads the
// dispatch packet for the group size, a dependent scalar load, and synchronises more than
// once; on short work-groups that showed up as microseconds in the prologue.) Any LDS word
// written here is read only before the next barrier of the caller, and callers reach a
// barrier between two uses.
template <int NT>
__device__ __forceinline__ bool block_any(int pred) {
    constexpr int NW = NT / 64;
    __shared__ int s_any[NW];
    const unsigned long long bal = __builtin_amdgcn_ballot_w64(pred != 0);
    if ((threadIdx.x & 63) == 0) s_any[threadIdx.x >> 6] = bal != 0;
    __syncthreads();
    int any = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) any |= s_any[w];
    return any != 0;
}

template <typename T>
__device__ __forceinline__ void store_nan(void* out, size_t base, int count) {
    for (int i = threadIdx.x; i < count; i += blockDim.x) store_elem(T{}, out, base + i, __builtin_nanf(""));
}

// Fused append: the record of one kv head's new rows in LDS holds the K row then the V row
// in the pool's storage (KV), and for 8-bit pools their two float32 scales (16 bytes). The
// prologue stages the rows as read (in q's type, NewRec<T, D>); over an 8-bit pool a wave
// then quantises them into a record of its own (quantize_new_rows).
template <typename KV, int D>
struct NewRec {
    static constexpr int kRowBytes = D * KV::kBytes;
    static constexpr bool kScaled = KV::kBytes == 1;
    static constexpr int kBytes = 2 * kRowBytes + (kScaled ? 16 : 0);
};

// Fused append into an 8-bit pool: one wave (all 64 lanes) quantises the new K and V rows of
// one kv head, raw = the two rows in q's type T, into rec (E4M3 codes, then the two scales)
// exactly as the quantising append does: s = max |x| / 448 and the code nearest x / s
// clamped to +-448, IEEE float32 divisions; all codes 0 when s = 0.
template <typename T, int D>
__device__ void quantize_new_rows(const char* raw, char* rec) {
    static_assert(T::kBytes == 2 && D % 64 == 0, "16-bit source rows of 64k elements");
    constexpr int PL = D / 64;  // elements of a row per lane
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const uint16_t* src = reinterpret_cast<const uint16_t*>(raw + which * D * 2);
        float x[PL];
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < PL; ++j) {
            const uint16_t h = src[lane + 64 * j];
            if constexpr (std::is_same_v<T, BF16>) x[j] = __uint_as_float((uint32_t)h << 16);
            else x[j] = (float)__builtin_bit_cast(_Float16, h);
            amax = fmaxf(amax, fabsf(x[j]));
        }
        amax = group_max<32>(amax);
        amax = fmaxf(amax, shfl_xor(amax, 32));
        const float sc = __fdiv_rn(amax, 448.f);
#pragma unroll
        for (int j = 0; j < PL; ++j) {
            const uint32_t code = sc != 0.f ? e4m3_encode(fminf(fmaxf(__fdiv_rn(x[j], sc), -448.f), 448.f)) : 0u;
            reinterpret_cast<uint8_t*>(rec)[which * D + lane + 64 * j] = (uint8_t)code;
        }
        if (lane == 0) reinterpret_cast<float*>(rec + 2 * D)[which] = sc;
    }
}

// Fused append, step 1: the new token's K and V rows of kv heads [kv0, kv0 + nkv) in
// registers, in q's type T (vector i of [nkv][K row, V row] held by thread i % NT in slot
// i / NT), read in the prologue's first round trip where possible; the owner parks them in
// s_new before the barrier, quantised for an 8-bit pool. NKV bounds nkv.
template <typename T, int D, int NT, int NKV>
struct NewRows {
    static constexpr int kRowVecs = D * T::kBytes / 16;
    static constexpr int kPerThread = (2 * NKV * kRowVecs + NT - 1) / NT;
    u32x4 v[kPerThread];

    __device__ void load(const DecodeArgs& a, int b, int kv0, int nkv) {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int i = threadIdx.x + k * NT;
            if (i < 2 * nkv * kRowVecs) {
                const int kv = i / (2 * kRowVecs);
                const int which = (i / kRowVecs) & 1;
                const char* src = static_cast<const char*>(which ? a.new_value : a.new_key) +
                                  (((size_t)b * a.num_kv_heads + kv0 + kv) * D) * T::kBytes + 16 * (i % kRowVecs);
                v[k] = load16(src);
            }
        }
    }
    __device__ void park(int nkv, char* s_new) const {
#pragma unroll
        for (int k = 0; k < kPerThread; ++k) {
            const int i = threadIdx.x + k * NT;
            if (i < 2 * nkv * kRowVecs) store16(s_new + (size_t)i * 16, v[k]);
        }
    }
};

// Fused append, step 2 (after the barrier, block ids checked): true if slot_mapping[b] is
// the slot of position L - 1 through the table; the stream then takes the new token's rows
// from s_new, so nothing in this launch reads the slot. Otherwise PA_FLAG_BAD_SLOT is raised
// and the rows are never written.
__device__ __forceinline__ bool check_new_slot(const DecodeArgs& a, int L, int jp, int slot, const int* s_ids) {
    const int lbs = a.log2_block_size;
    const int pos = L - 1;
    if (slot == (s_ids[(pos >> lbs) - jp] << lbs) + (pos & ((1 << lbs) - 1))) return true;
    if (threadIdx.x == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_SLOT);
    return false;
}

// Fused append, step 3 (the owner's last act, after its outputs, when the launch has no
// reduce pass): the staged rows go to the slot ([BlockManager essay] §4.4; [Valid-length
// essay] §4.1). Issued at the end so that the stores do not compete with the workgroup's own
// stream; nothing waits for them.
// The slot comes from the prologue's registers: reading slot_mapping again here would add a
// memory round trip to the end of every owner workgroup.
template <typename KV, int D, int NT>
__device__ void store_new_rows(const DecodeArgs& a, int slot, int kv0, int nkv, const char* s_new) {
    using R = NewRec<KV, D>;
    constexpr int kRowVecs = R::kRowBytes / 16;
    const int lbs = a.log2_block_size;
    const int blk = slot >> lbs;
    const int off = slot & ((1 << lbs) - 1);
    for (int i = threadIdx.x; i < 2 * nkv * kRowVecs; i += NT) {
        const int kv = i / (2 * kRowVecs);
        const int which = (i / kRowVecs) & 1;
        const int v = i % kRowVecs;
        char* dst = static_cast<char*>(const_cast<void*>(which ? a.v_pool : a.k_pool)) + (size_t)blk * a.block_stride +
                    (((((size_t)kv0 + kv) << lbs) + off) * D) * KV::kBytes + 16 * v;
        store16(dst, load16(s_new + (size_t)kv * R::kBytes + which * R::kRowBytes + 16 * v));
    }
    if constexpr (R::kScaled) {
        for (int i = threadIdx.x; i < 2 * nkv; i += NT) {
            const size_t srow = (((size_t)blk * a.num_kv_heads + kv0 + i / 2) << lbs) + off;
            float* scales = const_cast<float*>((i & 1) ? a.v_scale : a.k_scale);
            scales[srow] = reinterpret_cast<const float*>(s_new + (size_t)(i / 2) * R::kBytes + 2 * R::kRowBytes)[i & 1];
        }
    }
}

// Checks the sequence length, stages the partition's block ids in s_ids and validates
// them. Returns false when the workgroup has nothing more to do: the partition is past the
// end of the sequence, or the sequence is invalid (the sink sets its outputs, or this
// partition's records, to NaN, and the error bit is raised). Never reads a table entry or a
// pool byte that the checks have not cleared.
//
// Without a window the table slice of partition p starts at logical block p * P / block_size
// whatever the length is, so it is loaded in the same round trip as the length (entries past
// the valid blocks are read from inside the row but never used); one barrier then publishes
// the ids and the OR of their range checks. With a window the slice starts at the block of
// the window start, so the length is read first.
//
// A valid length is at least min_len (1 for a decode; the number of new queries otherwise).
// Sink provides nan_outputs() and nan_records(p) for the outputs this workgroup owns.
//
// Fused append (a.slot_mapping set; the workgroup covers kv heads [kv0, kv0 + nkv) and
// gives s_new): the workgroup whose partition holds the last position L - 1 stages the new
// token's rows in s_new, checks the slot once its ids are checked, and reports the token's
// position in part.npos: the stream takes its rows from s_new and the workgroup writes them
// to the slot when it is done (store_new_rows). NKV bounds nkv.
template <typename T, int D, int NT, typename Sink, int NKV = 1>
__device__ bool partition_prologue_sink(const DecodeArgs& a, int p, int b, int min_len, const Sink& sink,
                                        int* s_ids, Partition& part, int kv0 = 0, int nkv = 0,
                                        char* s_new = nullptr) {
    constexpr int kPerThread = (kMaxIdsPerPartition + NT - 1) / NT;
    const int tid = threadIdx.x;
    const int lbs = a.log2_block_size;
    const int P = a.partition_size;
    int L = 0, base = 0;
    if (a.window > 0) {
        L = a.context_lens[b];
        if (L <= a.max_context_len) base = partition_base(a, L);
    }
    const int jp = (base + p * P) >> lbs;  // first block of the partition
    const int32_t* trow = a.block_table + (size_t)b * a.max_blocks_per_seq;
    const int lim = min(P >> lbs, a.max_blocks_per_seq - jp);
    int idv[kPerThread];
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int i = tid + k * NT;
        idv[k] = (i < lim) ? trow[jp + i] : 0;
    }
    if (a.window <= 0) L = a.context_lens[b];
    const bool appending = a.slot_mapping != nullptr && nkv > 0 && s_new != nullptr;
    const int slot = appending ? a.slot_mapping[b] : -1;
    // the workgroup of the first kv heads that holds the last position (or partition 0, when
    // the length is bad) records the slot for a reduce pass that writes the rows
    const bool record = appending && a.ws_slot != nullptr && kv0 == 0 && tid == 0;
    // speculative only in partition 0 (the owner for every one-partition sequence): workgroups
    // of later partitions are mostly past the end of short sequences, and a wave cannot retire
    // before its loads return
    NewRows<T, D, NT, NKV> rows;
    if (appending && p == 0) rows.load(a, b, kv0, nkv);
    int flag = 0;
    if (L <= 0) flag = PA_FLAG_EMPTY_CONTEXT;
    else if (L > a.max_context_len || ((L - 1) >> lbs) >= a.max_blocks_per_seq || L < min_len)
        flag = PA_FLAG_BAD_LENGTH;
    if (flag) {
        if (p == 0) {
            if (tid == 0 && a.err_flag) atomicOr(a.err_flag, flag);
            if (record) a.ws_slot[b] = -1;
            sink.nan_outputs();
        }
        return false;
    }
    part.nparts = (L - base + P - 1) / P;
    part.len = L;
    if (p >= part.nparts) return false;
    part.t0 = base + p * P;
    part.rel_lo = max(window_start(a, L) - part.t0, 0);
    const int t1 = min(L, part.t0 + P);
    part.ntok = t1 - part.t0;
    part.j0 = jp;
    part.npos = -1;
    part.slot = slot;
    const bool last = t1 == L;
    const bool owner = slot >= 0 && last;  // holds the new token
    if (owner) {
        if (p != 0) rows.load(a, b, kv0, nkv);
        rows.park(nkv, s_new);
    }
    // only the blocks overlapping [t0, t1) are staged and checked: blocks before a window
    // may already be released (-1)
    const int nids = ((t1 - 1) >> lbs) - jp + 1;
    int bad = 0;
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
        const int i = tid + k * NT;
        if (i < nids) {
            int id = idv[k];
            if ((unsigned)id >= (unsigned)a.num_blocks) {
                bad = 1;
                id = 0;
            }
            s_ids[i] = id;
        }
    }
    if (block_any<NT>(bad)) {
        if (tid == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_BLOCK_ID);
        if (last && record) a.ws_slot[b] = -1;
        if (part.nparts == 1) sink.nan_outputs();
        else sink.nan_records(p);
        return false;
    }
    if (owner && check_new_slot(a, L, jp, slot, s_ids)) part.npos = L - 1 - part.t0;
    if (last && record) a.ws_slot[b] = part.npos >= 0 ? slot : -1;
    return true;
}

// NaN sink of a decode workgroup: query heads [h0, h0 + nq) of sequence b.
template <typename T, int D>
struct DecodeNanSink {
    const DecodeArgs& a;
    int b, h0, nq;
    __device__ void nan_outputs() const { store_nan<T>(a.out, ((size_t)b * a.num_q_heads + h0) * D, nq * D); }
    __device__ void nan_records(int p) const {
        for (int i = threadIdx.x; i < nq * (D + 2); i += blockDim.x) {
            const int g = i / (D + 2), e = i % (D + 2);
            const size_t rec = ((size_t)b * a.num_q_heads + h0 + g) * a.max_partitions + p;
            if (e < D) a.ws_o[rec * D + e] = __builtin_nanf("");
            else a.ws_ml[rec * 2 + (e - D)] = (e == D) ? -INFINITY : __builtin_nanf("");
        }
    }
};

template <typename T, int D, int NT, int NKV>
__device__ __forceinline__ bool partition_prologue_heads(const DecodeArgs& a, int p, int h0, int nq, int b,
                                                         int* s_ids, Partition& part, char* s_new = nullptr) {
    const int group = a.num_q_heads / a.num_kv_heads;
    return partition_prologue_sink<T, D, NT, DecodeNanSink<T, D>, NKV>(a, p, b, 1, DecodeNanSink<T, D>{a, b, h0, nq}, s_ids, part, h0 / group,
                                             nq / group, s_new);
}

template <typename T, int D, int G, int NT>
__device__ __forceinline__ bool partition_prologue(const DecodeArgs& a, int p, int kvh, int b, int* s_ids,
                                                   Partition& part, char* s_new = nullptr) {
    return partition_prologue_heads<T, D, NT, 1>(a, p, kvh * G, G, b, s_ids, part, s_new);
}

// Log-sum-exp combine of the `nparts` partition records of one output row, for element e:
//   sum_p w_p o_p / sum_p w_p,  w_p = l_p * 2^(m_p - max_p m_p),
// where o_p is the partition's normalised output and (m_p, l_p) its base-2 running max and
// sum (ml holds (m_p, l_p) pairs, o the o_p rows with stride D). Records are read in chunks
// of 8 whose loads are all issued before any is used, so a chunk costs one memory round
// trip; the running max and sums are rescaled between chunks. A NaN sum (bad block in that
// partition) makes the result NaN.
template <int D>
__device__ __forceinline__ float lse_combine(const float* ml, const float* o, int nparts, int e) {
    constexpr int kChunk = 8;
    float M = -INFINITY, num = 0.f, den = 0.f;
    for (int p0 = 0; p0 < nparts; p0 += kChunk) {
        float mv[kChunk], lv[kChunk], ov[kChunk];
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            const bool ok = p0 + i < nparts;
            mv[i] = ok ? ml[2 * (p0 + i)] : -INFINITY;
            lv[i] = ok ? ml[2 * (p0 + i) + 1] : 0.f;
            ov[i] = ok ? o[(size_t)(p0 + i) * D + e] : 0.f;
        }
        float Mn = M;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) Mn = fmaxf(Mn, mv[i]);
        const float Ms = (Mn == -INFINITY) ? 0.f : Mn;
        const float r = fast_exp2(M - Ms);
        num *= r;
        den *= r;
#pragma unroll
        for (int i = 0; i < kChunk; ++i) {
            if (p0 + i < nparts) {
                const float w = lv[i] * fast_exp2(mv[i] - Ms);
                den += w;
                num = fmaf(w, ov[i], num);
            }
        }
        M = Mn;
    }
    return num / den;
}

// Merges the per-wave states (s_m, s_l: base-2 running max and sum; s_acc: unnormalised
// weighted sums) of G heads and writes either the final output (single partition) or the
// partition's record (normalised output, max, sum) for the log-sum-exp reduce.
template <typename T, int D, int G, int NW = kDecodeWaves>
__device__ void partition_epilogue(const DecodeArgs& a, int p, int kvh, int b, const Partition& part,
                                   const float (*s_m)[G], const float (*s_l)[G], const float (*s_acc)[G][D]) {
    const int h0 = kvh * G;
    for (int i = threadIdx.x; i < G * D; i += NW * 64) {
        const int g = i / D;
        const int e = i % D;
        float M = s_m[0][g];
#pragma unroll
        for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
        const float Ms = (M == -INFINITY) ? 0.f : M;
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(s_m[w][g] - Ms);
            num = fmaf(s_acc[w][g][e], f, num);
            den = fmaf(s_l[w][g], f, den);
        }
        const float o = num / den;
        const size_t hrow = (size_t)b * a.num_q_heads + h0 + g;
        if (part.nparts == 1) {
            store_elem(T{}, a.out, hrow * D + e, o);
        } else {
            const size_t rec = hrow * a.max_partitions + p;
            a.ws_o[rec * D + e] = o;
            if (e == 0) {
                a.ws_ml[rec * 2] = M;
                a.ws_ml[rec * 2 + 1] = den;
            }
        }
    }
}

}  // namespace pagedkv
