// dtype.hpp -- storage types of the pooled tensors and their conversions
// to and from binary32 on the device.
//
// float32 is stored as float; float16 and bfloat16 as their raw 16-bit
// patterns.  Widening to binary32 is exact for all three.  Narrowing rounds
// to nearest, ties to even (IEEE 754 default), keeps subnormals, overflows
// to infinity, and turns NaN into a quiet NaN that keeps its sign and top
// fraction bits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mp3d {

struct F32 {
    using raw = float;
    static constexpr int code = 0;
    __device__ static inline float widen(float r) { return r; }
    __device__ static inline float narrow(float f) { return f; }
};

struct F16 {
    using raw = uint16_t;
    static constexpr int code = 1;
    __device__ static inline float widen(uint16_t r) {
        return (float)__builtin_bit_cast(_Float16, r);   // v_cvt_f32_f16, exact
    }
    __device__ static inline uint16_t narrow(float f) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (f != f)
            return (uint16_t)(((u >> 16) & 0x8000u) | 0x7e00u | ((u & 0x7fffffu) >> 13));
        return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, RNE
    }
};

struct BF16 {
    using raw = uint16_t;
    static constexpr int code = 2;
    __device__ static inline float widen(uint16_t r) {
        return __builtin_bit_cast(float, (uint32_t)r << 16);
    }
    __device__ static inline uint16_t narrow(float f) {
        uint32_t u = __builtin_bit_cast(uint32_t, f);
        if (f != f)
            return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u | ((u & 0x7fffffu) >> 16));
        // add half an ulp of the result, minus one unless the kept lsb is 1
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};

}  // namespace mp3d
