// dtype.hpp -- storage types of the pooled tensors and their conversions
// to and from the type the kernels compare and accumulate in (`acc`).
//
// float32 is stored as float; float16 and bfloat16 as their raw 16-bit
// patterns; all three compare and accumulate in binary32, to which widening
// is exact.  Narrowing uses gfx950's conversion instructions: round to
// nearest, ties to even (IEEE 754 default), subnormals kept, overflow to
// infinity; NaN stays a NaN.  float64 compares and accumulates in binary64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mp3d {

// A 16-byte vector as a native LLVM vector (keeps loaded data in registers;
// the HIP uint4 struct is copied through memory when assigned under a branch)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef long long i64x2 __attribute__((ext_vector_type(2)));

// Streaming (non-temporal) stores: data written once is not kept in the
// caches.  Output streams measured markedly faster this way.
template <typename V>
__device__ __forceinline__ void st_stream(V *p, V v) { __builtin_nontemporal_store(v, p); }

struct F32 {
    using raw = float;
    using acc = float;
    static constexpr int code = 0;
    // narrowing a widened value gives back its exact bits, NaN included
    static constexpr bool exact_nan = true;
    __device__ static inline float widen(float r) { return r; }
    __device__ static inline float narrow(float f) { return f; }
    __device__ static inline float back(float f) { return f; }
    // the four elements of a 16-byte vector
    // (elements are copied out before the bit cast: this clang reads lane 0
    // for __builtin_bit_cast applied directly to an ext_vector element)
    __device__ static inline void unpack(u32x4 q, float *v) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __builtin_bit_cast(float, w[i]);
    }
};

struct F16 {
    using raw = uint16_t;
    using acc = float;
    static constexpr int code = 1;
    __device__ static inline float widen(uint16_t r) {
        return (float)__builtin_bit_cast(_Float16, r);   // v_cvt_f32_f16, exact
    }
    __device__ static inline uint16_t narrow(float f) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);  // v_cvt_f16_f32, RNE
    }
    // exact for every widened value except NaN, whose payload may change
    static constexpr bool exact_nan = false;
    __device__ static inline uint16_t back(float f) {
        return __builtin_bit_cast(uint16_t, (_Float16)f);
    }
    __device__ static inline void unpack(u32x4 q, float *v) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = widen((uint16_t)(w[i] & 0xffffu));
            v[2 * i + 1] = widen((uint16_t)(w[i] >> 16));
        }
    }
};

struct BF16 {
    using raw = uint16_t;
    using acc = float;
    static constexpr int code = 2;
    __device__ static inline float widen(uint16_t r) {
        return __builtin_bit_cast(float, (uint32_t)r << 16);
    }
    __device__ static inline uint16_t narrow(float f) {
        return __builtin_bit_cast(uint16_t, (__bf16)f);    // v_cvt_pk_bf16_f32, RNE
    }
    // widening is a shift, so the top half is the original pattern
    static constexpr bool exact_nan = true;
    __device__ static inline uint16_t back(float f) {
        return (uint16_t)(__builtin_bit_cast(uint32_t, f) >> 16);
    }
    __device__ static inline void unpack(u32x4 q, float *v) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
            v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
        }
    }
};

// float64: compared and accumulated in binary64 (a binary32 accumulator
// would round every double gradient).  Only the general kernels take it.
struct F64 {
    using raw = double;
    using acc = double;
    static constexpr int code = 3;
    static constexpr bool exact_nan = true;
    __device__ static inline double widen(double r) { return r; }
    __device__ static inline double narrow(double f) { return f; }
    __device__ static inline double back(double f) { return f; }
    // the two elements of a 16-byte vector
    __device__ static inline void unpack(u32x4 q, double *v) {
        v[0] = __builtin_bit_cast(double, (uint64_t)q.x | ((uint64_t)q.y << 32));
        v[1] = __builtin_bit_cast(double, (uint64_t)q.z | ((uint64_t)q.w << 32));
    }
};

}  // namespace mp3d
