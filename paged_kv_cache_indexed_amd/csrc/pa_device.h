// Device helpers for the gfx950 (CDNA4) paged-KV kernels: storage types, 16-byte vector
// access, conversions and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pagedkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Note: every reinterpretation below bit-casts the whole 16-byte vector and then takes
// constant swizzles. Bit-casting single elements of a u32x4 (bit_cast<f16x2>(v[i]))
// miscompiles with this toolchain: every i reads element 0.

// Storage tags. Every element type is moved as raw 16-byte vectors; the tag says how the
// lanes of a vector unpack to fp32 and how fp32 results round back.
struct F32 {
    static constexpr int kBytes = 4;
};
struct F16 {
    static constexpr int kBytes = 2;
};
struct BF16 {
    static constexpr int kBytes = 2;
};

// 8-bit floats in the OCP E4M3 format (bias 7, largest finite 448, S.1111.111 = NaN), one
// float32 scale per (token, kv head) row kept beside the block: a row is worth code * scale.
struct FP8 {
    static constexpr int kBytes = 1;
};

template <typename T>
struct VecInfo {
    static constexpr int kElems = 16 / T::kBytes;  // elements per 16-byte vector
};

// Buffer resource over `bytes` bytes at `base` (raw addressing, stride 0). An offset at or
// past `bytes` reads zeros without touching memory, which is how masked lanes skip padding.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferWord3);
}
// Cache policy of the K/V stream loads: 2 = non-temporal (each byte is read once).
#ifndef PA_KV_LOAD_POLICY
#define PA_KV_LOAD_POLICY 2
#endif
template <int kPolicy = PA_KV_LOAD_POLICY>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)offset, 0, kPolicy));
}

template <int kPolicy = PA_KV_LOAD_POLICY>
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t offset) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)offset, 0, kPolicy));
}

__device__ __forceinline__ u32x4 load16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

// ---- unpack 16 bytes to fp32 -------------------------------------------------------------
__device__ __forceinline__ void unpack(F32, u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ void unpack(F16, u32x4 v, float* f) {
    const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)h[i];
}
__device__ __forceinline__ void unpack(BF16, u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}

// 16 E4M3 codes -> fp32, exact. gfx950's scaled conversions read the OCP formats; with a
// scale of 1 they only widen.
__device__ __forceinline__ void unpack(FP8, u32x4 v, float* f) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[w], 1.f, false);
        const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(v[w], 1.f, true);
        f[4 * w] = lo.x;
        f[4 * w + 1] = lo.y;
        f[4 * w + 2] = hi.x;
        f[4 * w + 3] = hi.y;
    }
}

// ---- partial dot product of one 16-byte vector of K with the matching slice of q ---------
// q is kept in its storage form; products are exact in fp32 and accumulate in fp32.
__device__ __forceinline__ float dot16(F32, u32x4 q, u32x4 k) {
    float s = __uint_as_float(q[0]) * __uint_as_float(k[0]);
    s = fmaf(__uint_as_float(q[1]), __uint_as_float(k[1]), s);
    s = fmaf(__uint_as_float(q[2]), __uint_as_float(k[2]), s);
    s = fmaf(__uint_as_float(q[3]), __uint_as_float(k[3]), s);
    return s;
}
__device__ __forceinline__ float dot16(F16, u32x4 q, u32x4 k) {
    const f16x8 a = __builtin_bit_cast(f16x8, q);
    const f16x8 b = __builtin_bit_cast(f16x8, k);
    float s = __builtin_amdgcn_fdot2(a.s01, b.s01, 0.f, false);
    s = __builtin_amdgcn_fdot2(a.s23, b.s23, s, false);
    s = __builtin_amdgcn_fdot2(a.s45, b.s45, s, false);
    return __builtin_amdgcn_fdot2(a.s67, b.s67, s, false);
}
__device__ __forceinline__ float dot16(BF16, u32x4 q, u32x4 k) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, q);
    const bf16x8 b = __builtin_bit_cast(bf16x8, k);
    float s = __builtin_amdgcn_fdot2_f32_bf16(a.s01, b.s01, 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(a.s23, b.s23, s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(a.s45, b.s45, s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(a.s67, b.s67, s, false);
}

// 16 E4M3 codes of K against the matching 16 elements of q (two 16-byte vectors of fp16 or
// bf16). The codes widen exactly to q's type, products are exact in fp32 and accumulate in
// fp32.
__device__ __forceinline__ float dot16_fp8(F16, const u32x4* q, u32x4 k) {
    const f16x8 a = __builtin_bit_cast(f16x8, q[0]);
    const f16x8 b = __builtin_bit_cast(f16x8, q[1]);
    float s = __builtin_amdgcn_fdot2(a.s01, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[0], 1.f, false), 0.f, false);
    s = __builtin_amdgcn_fdot2(a.s23, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[0], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2(a.s45, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[1], 1.f, false), s, false);
    s = __builtin_amdgcn_fdot2(a.s67, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[1], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2(b.s01, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[2], 1.f, false), s, false);
    s = __builtin_amdgcn_fdot2(b.s23, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[2], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2(b.s45, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[3], 1.f, false), s, false);
    return __builtin_amdgcn_fdot2(b.s67, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(k[3], 1.f, true), s, false);
}
__device__ __forceinline__ float dot16_fp8(BF16, const u32x4* q, u32x4 k) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, q[0]);
    const bf16x8 b = __builtin_bit_cast(bf16x8, q[1]);
    float s = __builtin_amdgcn_fdot2_f32_bf16(a.s01, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[0], 1.f, false), 0.f,
                                              false);
    s = __builtin_amdgcn_fdot2_f32_bf16(a.s23, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[0], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(a.s45, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[1], 1.f, false), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(a.s67, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[1], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(b.s01, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[2], 1.f, false), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(b.s23, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[2], 1.f, true), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(b.s45, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[3], 1.f, false), s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(b.s67, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(k[3], 1.f, true), s,
                                           false);
}

// Nearest E4M3 code of x, ties to the even mantissa; |x| <= 448 and finite. Built from the
// format's definition: below 2^-6 the code counts multiples of 2^-9; above, the value is
// scaled by a power of two into [8, 16), rounded to an integer, and a carry to 16 moves to
// the next exponent. Every scaling is exact, so the only rounding is the one rint makes.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    const float a = fabsf(x);
    if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.f);
    int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;
    int m = (int)__builtin_rintf(__builtin_ldexpf(a, 3 - e)) - 8;
    if (m == 8) {
        m = 0;
        ++e;
    }
    return sign | (uint32_t)(((e + 7) << 3) | m);
}

// ---- fp32 -> storage (round to nearest even) ---------------------------------------------
__device__ __forceinline__ void store_elem(F32, void* base, size_t i, float x) {
    reinterpret_cast<float*>(base)[i] = x;
}
__device__ __forceinline__ void store_elem(F16, void* base, size_t i, float x) {
    reinterpret_cast<_Float16*>(base)[i] = (_Float16)x;
}
__device__ __forceinline__ void store_elem(BF16, void* base, size_t i, float x) {
    reinterpret_cast<__bf16*>(base)[i] = (__bf16)x;
}

// ---- wave64 cross-lane helpers -------------------------------------------------------------
// DPP control words (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm:[1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm:[2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
    const int lane = __lane_id();
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// Sum over aligned groups of N lanes; every lane of a group receives the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "group");
    if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
    if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
    if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
    if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
    if constexpr (N >= 32) x += shfl_xor(x, 16);
    if constexpr (N >= 64) x += shfl_xor(x, 32);
    return x;
}

// Maximum over aligned groups of N lanes (N <= 16); every lane of a group receives it.
template <int N>
__device__ __forceinline__ float group_max(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group");
    if constexpr (N >= 2) x = fmaxf(x, dpp<kDppQuadXor1>(x));
    if constexpr (N >= 4) x = fmaxf(x, dpp<kDppQuadXor2>(x));
    if constexpr (N >= 8) x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
    if constexpr (N >= 16) x = fmaxf(x, dpp<kDppRowMirror>(x));
    if constexpr (N >= 32) x = fmaxf(x, shfl_xor(x, 16));
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pagedkv
