// geometry.hpp -- window bounds on one axis, their inverse, and the
// per-call tiling plan shared by the host dispatcher and the kernels.
//
// Fixed windows follow "Struct Maxpool3dForward" (teenygrad API docs,
// description): no padding, O = (X - K)/S + 1, window o = [o*S, o*S + K).
// Adaptive windows: the PR #308 page (Add adaptive_max_pool3d_backward ...,
// Summary) requires a disjoint tiling when the axis divides evenly and an
// overlap otherwise; window o = [floor(o*X/O), ceil((o+1)*X/O)) has both
// properties.
// Padding and dilation of fixed windows: the pages give no pooling rule
// beyond "no padding".  Reading taken: window o takes the k taps
// o*S - pad + j*dil, a tap outside the axis is padding that never wins, and
// the taps span (k-1)*dil + 1 positions (the effective kernel of the
// FlagGems conv_transpose2d PR page, Implementation, scatter condition).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mp3d {

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

// One spatial axis: extent X split into O windows; k > 0 selects fixed
// windows, k == 0 adaptive windows.  A fixed window o has k taps at
// o*s - pad + j*dil (j < k), spanning ext = (k-1)*dil + 1 positions; taps
// outside [0, X) are padding and never taken.  `plain`: no padding,
// dilation 1 and no window past the axis end (window o is [o*s, o*s + k)).
// When every numerator below fits 31 bits (`fast`), the divisions by O, X
// and s use precomputed multiply-high constants instead of 64-bit division.
struct Axis {
    int32_t X, O, k, s;
    int32_t pad, dil, ext;
    FastDiv dO, dX, dS;
    int32_t fast;

    __host__ static Axis make(int32_t X, int32_t O, int32_t k, int32_t s, int32_t pad = 0,
                              int32_t dil = 1) {
        Axis a;
        a.X = X; a.O = O; a.k = k; a.s = s;
        a.pad = k ? pad : 0;
        a.dil = k ? dil : 1;
        a.ext = k ? (k - 1) * dil + 1 : 0;
        a.dO = FastDiv((uint32_t)O);
        a.dX = FastDiv((uint32_t)X);
        a.dS = FastDiv((uint32_t)(s > 0 ? s : 1));
        const int64_t lim = (int64_t)1 << 31;
        a.fast = ((int64_t)O + 1) * X + O < lim && ((int64_t)X + 1) * O + X < lim;
        return a;
    }

    __host__ __device__ inline bool plain() const {
        return k == 0 || (pad == 0 && dil == 1 && (int64_t)(O - 1) * s + k <= X);
    }
    // taps are every position of the span: dilation 1
    __host__ __device__ inline bool contiguous() const { return dil == 1; }

    // Span [start, end) of window o, clipped to the axis.  With dilation 1
    // these are exactly the window's taps inside the input, so a kernel
    // that scans [start, end) serves padded and ceil-mode windows as they
    // are; with dilation > 1 the span also holds positions between taps.
    __host__ __device__ inline int32_t start(int32_t o) const {
        if (k) { const int32_t b = o * s - pad; return b > 0 ? b : 0; }
        if (fast) return (int32_t)dO.div((uint32_t)(o * X));
        return (int32_t)(((int64_t)o * X) / O);
    }
    __host__ __device__ inline int32_t end(int32_t o) const {
        if (k) { const int32_t e = o * s - pad + ext; return e < X ? e : X; }
        if (fast) return (int32_t)dO.div((uint32_t)((o + 1) * X + O - 1));
        return (int32_t)((((int64_t)o + 1) * X + O - 1) / O);
    }
    // First window whose span ends beyond position p (windows before it
    // cannot contain p or anything after it).
    __host__ __device__ inline int32_t first_reaching(int32_t p) const {
        if (k) return p + pad < ext ? 0 : (int32_t)dS.div((uint32_t)(p + pad - ext)) + 1;
        if (fast) return (int32_t)dX.div((uint32_t)(p * O));
        return (int32_t)(((int64_t)p * O) / X);
    }
    // Last window whose span starts at or before position p, clamped to O-1.
    __host__ __device__ inline int32_t last_starting(int32_t p) const {
        int32_t o;
        if (k) o = (int32_t)dS.div((uint32_t)(p + pad));
        else if (fast) o = (int32_t)dX.div((uint32_t)((p + 1) * O - 1));
        else o = (int32_t)(((((int64_t)p + 1) * O) - 1) / X);
        return o < O - 1 ? o : O - 1;
    }
};

// Taps of window o on one axis: tap j (0 <= j < n) sits at b + j*t; the
// taps inside [0, X) are j0..j1 (j0 > j1: none).
struct Taps {
    int32_t b, t, n, j0, j1;
};

__host__ __device__ inline Taps window_taps(const Axis &a, int32_t o)
{
    Taps r;
    if (a.k) {
        r.b = o * a.s - a.pad;
        r.t = a.dil;
        r.n = a.k;
    } else {
        r.b = a.start(o);
        r.t = 1;
        r.n = a.end(o) - r.b;
    }
    r.j0 = r.b >= 0 ? 0 : (r.t == 1 ? -r.b : (-r.b + r.t - 1) / r.t);
    const int32_t room = a.X - 1 - r.b;                // last position minus the first tap's
    const int32_t last = r.t == 1 ? room : room / r.t;
    r.j1 = room < 0 ? -1 : (last < r.n - 1 ? last : r.n - 1);
    return r;
}

// Splits a linear tile number into (plane, i0, i1, i2) for tiles counted
// plane-major with n0 x n1 x n2 tiles per plane (i2 fastest).
struct TileSplit {
    FastDiv d2, d1, d0;
    int32_t n0, n1, n2;
    int32_t fast;              // tile numbers fit 31 bits

    __host__ static TileSplit make(int64_t planes, int32_t n0, int32_t n1, int32_t n2) {
        TileSplit t;
        t.n0 = n0; t.n1 = n1; t.n2 = n2;
        t.d0 = FastDiv((uint32_t)n0);
        t.d1 = FastDiv((uint32_t)n1);
        t.d2 = FastDiv((uint32_t)n2);
        t.fast = planes * n0 * n1 * n2 < ((int64_t)1 << 31);
        return t;
    }
    __host__ __device__ inline void split(int64_t t, int64_t *plane, int32_t *i0, int32_t *i1,
                                          int32_t *i2) const {
        if (fast) {
            uint32_t q = (uint32_t)t;
            uint32_t r = d2.div(q); *i2 = (int32_t)(q - r * (uint32_t)n2); q = r;
            r = d1.div(q); *i1 = (int32_t)(q - r * (uint32_t)n1); q = r;
            r = d0.div(q); *i0 = (int32_t)(q - r * (uint32_t)n0);
            *plane = r;
        } else {
            int64_t q = t;
            *i2 = (int32_t)(q % n2); q /= n2;
            *i1 = (int32_t)(q % n1); q /= n1;
            *i0 = (int32_t)(q % n0);
            *plane = q / n0;
        }
    }
};

// What one launch needs to know about the tensor and its windows.
struct Geom {
    int64_t planes;          // N*C
    Axis ax[3];              // d, h, w
    int32_t in_plane;        // D*H*W (fits int32 by validation)
    int32_t out_plane;       // OD*OH*OW

    __host__ __device__ inline bool plain() const {
        return ax[0].plain() && ax[1].plain() && ax[2].plain();
    }
    __host__ __device__ inline bool contiguous() const {
        return ax[0].contiguous() && ax[1].contiguous() && ax[2].contiguous();
    }
};

}  // namespace mp3d
