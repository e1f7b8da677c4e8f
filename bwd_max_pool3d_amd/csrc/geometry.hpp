// geometry.hpp -- window bounds on one axis, their inverse, and the
// per-call tiling plan shared by the host dispatcher and the kernels.
//
// Fixed windows follow "Struct Maxpool3dForward" (teenygrad API docs,
// description): no padding, O = (X - K)/S + 1, window o = [o*S, o*S + K).
// Adaptive windows: the PR #308 page (Add adaptive_max_pool3d_backward ...,
// Summary) requires a disjoint tiling when the axis divides evenly and an
// overlap otherwise; window o = [floor(o*X/O), ceil((o+1)*X/O)) has both
// properties.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mp3d {

// One spatial axis: extent X split into O windows; k > 0 selects fixed
// windows of width k and stride s, k == 0 adaptive windows.
struct Axis {
    int32_t X, O, k, s;

    __host__ __device__ inline int32_t start(int32_t o) const {
        return k ? o * s : (int32_t)(((int64_t)o * X) / O);
    }
    __host__ __device__ inline int32_t end(int32_t o) const {
        return k ? o * s + k : (int32_t)((((int64_t)o + 1) * X + O - 1) / O);
    }
    // First window whose end lies beyond position p (windows before it
    // cannot contain p or anything after it).
    __host__ __device__ inline int32_t first_reaching(int32_t p) const {
        if (k) return p < k ? 0 : (p - k) / s + 1;
        return (int32_t)(((int64_t)p * O) / X);
    }
    // Last window that starts at or before position p, clamped to O-1.
    __host__ __device__ inline int32_t last_starting(int32_t p) const {
        int64_t o = k ? (int64_t)(p / s)
                      : ((((int64_t)p + 1) * O) - 1) / X;
        return o < O - 1 ? (int32_t)o : O - 1;
    }
};

// Unsigned division by a runtime constant through a multiply-high
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994): for n < 2^31 and 1 <= d < 2^31,
// n / d == (umulhi(n, m) + n) >> l with l = ceil(log2 d) and
// m = floor(2^32 * (2^l - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, l;

    FastDiv() = default;
    __host__ explicit FastDiv(uint32_t div) : d(div) {
        l = 0;
        while ((1ull << l) < div) ++l;
        m = (uint32_t)((((1ull << l) - div) << 32) / div + 1);
    }
    __host__ __device__ inline uint32_t div(uint32_t n) const {
#ifdef __HIP_DEVICE_COMPILE__
        uint32_t t = __umulhi(n, m);
#else
        uint32_t t = (uint32_t)(((uint64_t)n * m) >> 32);
#endif
        return (t + n) >> l;
    }
};

// What one launch needs to know about the tensor and its windows.
struct Geom {
    int64_t planes;          // N*C
    Axis ax[3];              // d, h, w
    int32_t in_plane;        // D*H*W (fits int32 by validation)
    int32_t out_plane;       // OD*OH*OW
};

}  // namespace mp3d
