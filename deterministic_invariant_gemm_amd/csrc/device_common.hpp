// Device-side helpers shared by the scalar and MFMA tiers (gfx950 only).
//
// Storage formats: f32, bf16 (upper half of an f32), f16 (IEEE binary16) and
// OCP fp8 e4m3fn.  Decoding widens exactly to f32; encoding rounds an f32 to
// nearest-even once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// DT_E4M3 operands are widened exactly to bf16 and multiplied by the bf16
// matrix instruction (f32 accumulation of every product); DT_E4M3_FAST marks
// e4m3 operands multiplied by the fp8 matrix instruction, which aligns the
// products of each group of 8 to the group's largest before adding them
// (opt-in, wider tolerance).
enum Dt : int { DT_F32 = 0, DT_BF16 = 1, DT_F16 = 2, DT_E4M3 = 3, DT_E5M2 = 4, DT_E4M3_FAST = 5 };

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---- decode (exact widening) ------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// OCP e4m3fn: bias 7, subnormal quantum 2^-9, S.1111.111 is NaN, no inf.
__device__ __forceinline__ float e4m3_bits_to_f32(uint32_t c) {
    const uint32_t s = (c & 0x80u) << 24;
    const uint32_t e = (c >> 3) & 0xfu;
    const uint32_t f = c & 0x7u;
    if (e == 0xfu && f == 0x7u) return __uint_as_float(s | 0x7fc00000u);
    if (e == 0) {
        const float v = (float)f * 0x1p-9f;  // exact
        return s ? -v : v;
    }
    return __uint_as_float(s | ((e + 120u) << 23) | (f << 20));
}

template <int DT>
__device__ __forceinline__ float load_elem(const void *base, int64_t i) {
    if constexpr (DT == DT_F32) {
        return static_cast<const float *>(base)[i];
    } else if constexpr (DT == DT_BF16) {
        return bf16_bits_to_f32(static_cast<const uint16_t *>(base)[i]);
    } else if constexpr (DT == DT_F16) {
        return f16_bits_to_f32(static_cast<const uint16_t *>(base)[i]);
    } else {
        return e4m3_bits_to_f32(static_cast<const uint8_t *>(base)[i]);
    }
}

// ---- encode (one round-to-nearest-even) -------------------------------------

// f32 -> bf16 bits, RNE; NaN stays a quiet NaN; overflow gives +-inf.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// f32 -> f16 bits via v_cvt_f16_f32 (round-to-nearest-even in the default
// mode, IEEE subnormals and overflow to inf).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two f32 -> two bf16 / f16 values, each rounded once to nearest-even (IEEE
// overflow to inf and subnormals), packed with `a` in the low half:
// v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32 in the default rounding mode.
template <int DT>
__device__ __forceinline__ uint32_t pack2_rne(float a, float b) {
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit output types");
    if constexpr (DT == DT_BF16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Eight OCP e4m3fn codes (w[0] holds codes 0..3 from its low byte up, w[1]
// codes 4..7) -> the same eight values as bf16, packed two per dword in the
// same order.  Exact: every e4m3fn value, subnormals included, is a bf16
// value.  v_cvt_scalef32_pk_bf16_fp8 (scale 1.0) converts the two codes of one
// half of a dword; each packed result is taken whole by a bit cast.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
}
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w) {
    return u32x4{e4m3x2_to_bf16x2<false>(w[0]), e4m3x2_to_bf16x2<true>(w[0]),
                 e4m3x2_to_bf16x2<false>(w[1]), e4m3x2_to_bf16x2<true>(w[1])};
}

template <int DT>
__device__ __forceinline__ void store_elem(void *base, int64_t i, float v) {
    if constexpr (DT == DT_F32) {
        static_cast<float *>(base)[i] = v;
    } else if constexpr (DT == DT_BF16) {
        static_cast<uint16_t *>(base)[i] = (uint16_t)f32_to_bf16_bits(v);
    } else {
        static_cast<uint16_t *>(base)[i] = (uint16_t)f32_to_f16_bits(v);
    }
}

// Map a linear workgroup id so that the workgroups the dispatcher places on one
// XCD (ids congruent mod 8) receive one contiguous range of logical tiles.
// The mapping is a permutation of [0, nb); it never changes which tile a
// workgroup computes arithmetically, only where it runs.
__host__ __device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nb) {
    const int64_t full = nb - nb % 8;
    if (bid >= full) return bid;
    return (bid % 8) * (full / 8) + bid / 8;
}

}  // namespace bi
