// fa_device.h -- device-side building blocks shared by the MFMA kernels
// (forward prefill and backward): vector types, the 32x32x16 MFMA wrapper,
// compile-time integers for stage tags, and the lane-half exchanges.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define FA_LDS __attribute__((address_space(3)))

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// D (32x32, float32) += A (32x16) B (16x32) for 16-bit inputs; 8 elements of
// A and of B per lane (see fa_layout.h for the lane layout).
template <typename T>
struct Mfma;

template <>
struct Mfma<__bf16> {
    typedef bf16x8 x8;
    typedef bf16x4 x4;
    static __device__ __forceinline__ f32x16 run(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // D (16x16, float32) += A (16x32) B (32x16)
    static __device__ __forceinline__ f32x4 run16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static constexpr uint16_t kOne = 0x3F80;  // 1.0
};

template <>
struct Mfma<_Float16> {
    typedef f16x8 x8;
    typedef f16x4 x4;
    static __device__ __forceinline__ f32x16 run(x8 a, x8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    // D (16x16, float32) += A (16x32) B (32x16)
    static __device__ __forceinline__ f32x4 run16(x8 a, x8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static constexpr uint16_t kOne = 0x3C00;  // 1.0
};

template <int N>
struct Int {
    static constexpr int value = N;
};

// word 3 of a raw buffer descriptor on gfx9-family parts
constexpr int kBufferDword3 = 0x00020000;

// max / sum of x over lanes l and l ^ 32 (the two halves of a wave)
__device__ __forceinline__ float xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace fa
