// idxsrc.hpp -- where the backward kernels take each window's argmax from.
//
// The backward (PR #308 page, Summary) sends gy[o] to the argmax of window
// o.  The argmax either comes from the index array the forward wrote, or is
// recomputed from the forward's input and output, which lets a caller run
// the values-only forward and keep no index at all (the teenygrad kernel ABI
// passes no index buffer, "Struct Maxpool3dForward", Kernel trait; its
// backward receives the forward's inputs and output, RuntimeOp).
#pragma once

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

// From an index array, int32 or int64.
template <typename IT>
struct IdxArray {
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
    const typename T::raw *x;
    const typename T::raw *y;
    Geom g;
    int32_t fast32;            // every output number fits 31 bits: plane_div applies
    FastDiv plane_div;         // by out_plane
    FastDiv ow_div, oh_div;    // by OW, then by OH

    __device__ int32_t operator()(int64_t o) const {
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
        const int32_t H = g.ax[1].X, W = g.ax[2].X;
        const typename T::raw *xp = x + plane * (int64_t)g.in_plane;
        const float want = T::widen(y[o]);
        const bool nan = want != want;
        for (int32_t a = td.j0; a <= td.j1; ++a) {
            const int32_t d = td.b + a * td.t;
            for (int32_t b = th.j0; b <= th.j1; ++b) {
                const int32_t row = (d * H + th.b + b * th.t) * W;
                for (int32_t c = tw.j0; c <= tw.j1; ++c) {
                    const int32_t q = row + tw.b + c * tw.t;
                    const float v = T::widen(xp[q]);
                    if (nan ? v != v : v == want) return q;
                }
            }
        }
        return -1;
    }
};

}  // namespace mp3d
