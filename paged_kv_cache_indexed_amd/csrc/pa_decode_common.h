// Pieces shared by the decode kernels: the per-partition prologue (length checks, block-id
// staging in LDS) and the epilogue (merge of per-wave softmax states, output or partition
// record). Every function here is called by all threads of the workgroup.
#pragma once

#include "pa_kernels.h"

namespace pagedkv {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * 64;

struct Partition {
    int nparts;  // partitions of this sequence
    int t0;      // first position of this partition (a block multiple)
    int rel_lo;  // first attended token, relative to t0 (< block_size; 0 unless a window starts inside)
    int ntok;    // end of the attended tokens, relative to t0
    int j0;      // logical block of t0: s_ids[i] is the id of block j0 + i
    int len;     // the sequence's context length
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

template <typename T>
__device__ __forceinline__ void store_nan(void* out, size_t base, int count) {
    for (int i = threadIdx.x; i < count; i += blockDim.x) store_elem(T{}, out, base + i, __builtin_nanf(""));
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
template <typename T, int D, int NT, typename Sink>
__device__ bool partition_prologue_sink(const DecodeArgs& a, int p, int b, int min_len, const Sink& sink,
                                        int* s_ids, Partition& part) {
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
    int flag = 0;
    if (L <= 0) flag = PA_FLAG_EMPTY_CONTEXT;
    else if (L > a.max_context_len || ((L - 1) >> lbs) >= a.max_blocks_per_seq || L < min_len)
        flag = PA_FLAG_BAD_LENGTH;
    if (flag) {
        if (p == 0) {
            if (tid == 0 && a.err_flag) atomicOr(a.err_flag, flag);
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
    if (__syncthreads_or(bad)) {
        if (tid == 0 && a.err_flag) atomicOr(a.err_flag, PA_FLAG_BAD_BLOCK_ID);
        if (part.nparts == 1) sink.nan_outputs();
        else sink.nan_records(p);
        return false;
    }
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

template <typename T, int D, int NT>
__device__ __forceinline__ bool partition_prologue_heads(const DecodeArgs& a, int p, int h0, int nq, int b,
                                                         int* s_ids, Partition& part) {
    return partition_prologue_sink<T, D, NT>(a, p, b, 1, DecodeNanSink<T, D>{a, b, h0, nq}, s_ids, part);
}

template <typename T, int D, int G, int NT>
__device__ __forceinline__ bool partition_prologue(const DecodeArgs& a, int p, int kvh, int b, int* s_ids,
                                                   Partition& part) {
    return partition_prologue_heads<T, D, NT>(a, p, kvh * G, G, b, s_ids, part);
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
