// idxsrc.hpp -- where the backward kernels take each window's argmax from.
//
// The backward (PR #308 page, Summary) sends gy[o] to the argmax of window
// o.  The argmax either comes from the index array the forward wrote, or is
// recomputed from the forward's input and output, which lets a caller run
// the values-only forward and keep no index at all (the teenygrad kernel ABI
// passes no index buffer, "Struct Maxpool3dForward", Kernel trait; its
// backward receives the forward's inputs and output, RuntimeOp).
#pragma once

#include <algorithm>

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

// From an index array, int32 or int64.
template <typename IT>
struct IdxArray {
    static constexpr int kSlots = kBwdRound; // windows per thread per slab round
    const IT *p;
    __device__ __forceinline__ int32_t operator()(int64_t o) const { return ld_idx(p, o); }
};

// Recomputed from x and y: the first tap of window o, in d, h, w scan
// order, whose element equals y[o] (the first NaN when y[o] is NaN); -1 if
// none does.  When y is what the forward wrote this is the forward's own
// argmax, since the forward keeps the first element equal to the window's
// maximum (the first NaN if the window holds one); -0 and +0 compare equal
// on both sides.
template <typename T>
struct IdxRecompute {
    static constexpr int kSlots = 2;       // windows per thread per slab round
    const typename T::raw *x;
    const typename T::raw *y;
    Geom g;
    int32_t fast32;            // every output number fits 31 bits: plane_div applies
    int32_t km3;               // every window has at most 3 taps per axis
    int32_t w8;                // every window has at most 8 taps along w
    FastDiv plane_div;         // by out_plane
    FastDiv ow_div, oh_div;    // by OW, then by OH

    using A = typename T::acc;
    __device__ __forceinline__ static bool hit(A v, A want, bool nan) {
        return nan ? v != v : v == want;
    }

    // Loads are issued in groups that do not wait on one another: the whole
    // 3x3x3 block when windows are that small, else one row of up to 8 taps
    // at a time.  Tap numbers are clamped to the in-range taps, so a
    // repeated tap copies the first in-range row, slice or element just
    // before it (the same first match, at the same position) or the last
    // one after it (never first).
    __device__ __forceinline__ int32_t operator()(int64_t o) const {
        using R = typename T::raw;
        int64_t plane;
        if (fast32) plane = plane_div.div((uint32_t)o);
        else plane = o / g.out_plane;
        const uint32_t r0 = (uint32_t)(o - plane * g.out_plane);
        const uint32_t r = ow_div.div(r0);
        const int32_t ow = (int32_t)(r0 - r * (uint32_t)g.ax[2].O);
        const uint32_t od = oh_div.div(r);
        const int32_t oh = (int32_t)(r - od * (uint32_t)g.ax[1].O);
        const Taps td = window_taps(g.ax[0], (int32_t)od);
        const Taps th = window_taps(g.ax[1], oh);
        const Taps tw = window_taps(g.ax[2], ow);
        if (td.j0 > td.j1 || th.j0 > th.j1 || tw.j0 > tw.j1) return -1;
        const int32_t H = g.ax[1].X, W = g.ax[2].X;
        const R *xp = x + plane * (int64_t)g.in_plane;
        const A want = T::widen(y[o]);
        const bool nan = want != want;
        if (km3) {
            int32_t pos[27];
            R v[27];
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int32_t d = td.b + min(max(a, td.j0), td.j1) * td.t;
                    const int32_t h = th.b + min(max(b, th.j0), th.j1) * th.t;
#pragma unroll
                    for (int c = 0; c < 3; ++c) {
                        const int32_t q = (d * H + h) * W + tw.b + min(max(c, tw.j0), tw.j1) * tw.t;
                        pos[(a * 3 + b) * 3 + c] = q;
                        v[(a * 3 + b) * 3 + c] = xp[q];
                    }
                }
            int32_t found = -1;
#pragma unroll
            for (int q = 26; q >= 0; --q)
                if (hit(T::widen(v[q]), want, nan)) found = pos[q];
            return found;
        }
        for (int32_t a = td.j0; a <= td.j1; ++a) {
            const int32_t d = td.b + a * td.t;
            for (int32_t b = th.j0; b <= th.j1; ++b) {
                const int32_t row = (d * H + th.b + b * th.t) * W + tw.b;
                if (w8) {
                    R v[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) v[c] = xp[row + min(max(c, tw.j0), tw.j1) * tw.t];
                    int32_t found = -1;
#pragma unroll
                    for (int c = 7; c >= 0; --c)
                        if (hit(T::widen(v[c]), want, nan)) found = row + min(max(c, tw.j0), tw.j1) * tw.t;
                    if (found >= 0) return found;
                } else {
                    for (int32_t c = tw.j0; c <= tw.j1; ++c) {
                        const int32_t q = row + c * tw.t;
                        if (hit(T::widen(xp[q]), want, nan)) return q;
                    }
                }
            }
        }
        return -1;
    }
};

}  // namespace mp3d
