// Device-side types and helpers private to liblinbwd (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lb {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 bit pattern -> float: the pattern is the upper half of a binary32.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __builtin_bit_cast(float, h << 16);
}

// IEEE binary16 bit pattern -> float (exact).
__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// float -> bf16 bit pattern, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// two floats -> packed bf16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 (converted one at a time, the halves took four instructions)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_v __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){a, b}, bf16x2_v));
}

__device__ __forceinline__ bool aligned16(const void *p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

} // namespace lb
