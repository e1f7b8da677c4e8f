// idxsrc.hpp -- where the backward kernels take each window's argmax from.
//
// The backward (PR #308 page, Summary) sends gy[o] to the argmax of window
// o.  The argmax either comes from the index array the forward wrote, or is
// recomputed from the forward's input and output, which lets a caller run
// the values-only forward and keep no index at all (the teenygrad kernel ABI
// passes no index buffer, "Struct Maxpool3dForward", Kernel trait; its
// backward receives the forward's inputs and output, RuntimeOp), or is
// taken from a forward run into a caller's workspace and checked against y.
#pragma once

#include <algorithm>
#include <type_traits>

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

// From an index array, int32 or int64.
template <typename IT>
struct IdxArray {
    static constexpr int kSlots = kBwdRound; // windows per thread per slab round
    const IT *p;
    __device__ __forceinline__ int32_t operator()(int64_t o) const { return ld_idx(p, o); }
    // four consecutive indices from o (a multiple of 4), as vector loads
    // (the array must start on 16 bytes: aligned4)
    __device__ __forceinline__ void load4(int64_t o, int32_t (&ix)[4]) const {
        if constexpr (sizeof(IT) == 4) {
            const i32x4 v = *reinterpret_cast<const i32x4 *>(p + o);
            ix[0] = v.x; ix[1] = v.y; ix[2] = v.z; ix[3] = v.w;
        } else {
            const i64x2 a = *reinterpret_cast<const i64x2 *>(p + o);
            const i64x2 b = *reinterpret_cast<const i64x2 *>(p + o + 2);
            const int64_t v[4] = {a.x, a.y, b.x, b.y};
#pragma unroll
            for (int k = 0; k < 4; ++k) ix[k] = v[k] == (int64_t)(int32_t)v[k] ? (int32_t)v[k] : -1;
        }
    }
    __host__ bool aligned4() const { return (uintptr_t)p % 16 == 0; }
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

// The first tap of window (od, oh, ow) of one plane (xp) equal to want, in
// d, h, w scan order (the first NaN when want is NaN); -1 if none is.  A
// plain loop over the window's in-range taps, one load at a time: it serves
// the windows whose y is not their maximum, which are rare, and keeps the
// callers' common path small.
template <typename T>
__device__ __forceinline__ int32_t scan_first_equal(const typename T::raw *xp, const Geom &g,
                                                    int32_t od, int32_t oh, int32_t ow,
                                                    typename T::acc want)
{
    const Taps td = window_taps(g.ax[0], od), th = window_taps(g.ax[1], oh);
    const Taps tw = window_taps(g.ax[2], ow);
    const int32_t H = g.ax[1].X, W = g.ax[2].X;
    const bool nan = want != want;
    for (int32_t a = td.j0; a <= td.j1; ++a)
        for (int32_t b = th.j0; b <= th.j1; ++b) {
            const int32_t row = ((td.b + a * td.t) * H + th.b + b * th.t) * W + tw.b;
            for (int32_t c = tw.j0; c <= tw.j1; ++c) {
                const typename T::acc v = T::widen(xp[row + c * tw.t]);
                if (nan ? v != v : v == want) return row + c * tw.t;
            }
        }
    return -1;
}

// Recomputed from x and y by way of the forward's own argmax and maximum
// (idxf, yf: the forward run on x into a caller's workspace).  Where y[o]
// equals yf[o] (both NaN, or equal as numbers) every tap equal to y[o] is a
// maximum of the window, so the first of them is the forward's argmax (the
// first maximum; the first NaN when the window holds one); elsewhere the
// window is scanned in x.  The same result as IdxRecompute, for three
// streamed loads per window in the common case.
template <typename T>
struct IdxChecked {
    static constexpr int kSlots = kBwdRound;   // windows per thread per slab round
    const int32_t *idxf;
    const typename T::raw *yf;
    const typename T::raw *x;
    const typename T::raw *y;
    Geom g;
    FastDiv ow_div, oh_div;    // by OW, then by OH

    // Two phases, so that a caller with several windows in hand issues
    // every window's loads before the first compare: load (no branch), then
    // settled (the common case: the forward's argmax stands) or rescan
    // (the window scanned in x; it loads y[o] again, so that nothing of a
    // window is held across the scans of the others).
    // 16-bit storage is held widened to 32 bits as loaded (a whole register)
    using Word = std::conditional_t<(sizeof(typename T::raw) < 4), uint32_t, typename T::raw>;
    struct Pending {
        Word y, yf;
        int32_t idx;
    };
    __device__ __forceinline__ Pending load(int64_t o) const {
        return {(Word)y[o], (Word)yf[o], idxf[o]};
    }
    // Pins a pending window's values at this point of the program: a
    // caller that passed a barrier since load calls it first, so that the
    // compares that follow stay below the barrier (hoisted above it, they
    // make the wave wait for its loads before the barrier instead of
    // behind it).
    __device__ __forceinline__ static void pin(Pending &q) {
        asm volatile("" : "+v"(q.y), "+v"(q.yf), "+v"(q.idx));
    }
    __device__ __forceinline__ static bool settled(const Pending &q) {
        using A = typename T::acc;
        using R = typename T::raw;
        const A want = T::widen((R)q.y), got = T::widen((R)q.yf);
        return want != want ? got != got : got == want;
    }
    __device__ __forceinline__ int32_t rescan(int64_t o) const {
        const typename T::acc want = T::widen(y[o]);
        const int64_t plane = o / g.out_plane;
        const uint32_t r0 = (uint32_t)(o - plane * g.out_plane);
        const uint32_t r = ow_div.div(r0);
        const uint32_t od = oh_div.div(r);
        return scan_first_equal<T>(x + plane * (int64_t)g.in_plane, g, (int32_t)od,
                                   (int32_t)(r - od * (uint32_t)g.ax[1].O),
                                   (int32_t)(r0 - r * (uint32_t)g.ax[2].O), want);
    }
    __device__ __forceinline__ int32_t operator()(int64_t o) const {
        const Pending q = load(o);
        return settled(q) ? q.idx : rescan(o);
    }
};

// Index sources that split a query into load and resolve, and what a
// caller holds between the two (unused for the others).
template <typename S> struct two_phase_src : std::false_type {};
template <typename T> struct two_phase_src<IdxChecked<T>> : std::true_type {};
template <typename S, typename = void> struct pending_of { using type = int32_t; };
template <typename S> struct pending_of<S, std::void_t<typename S::Pending>> {
    using type = typename S::Pending;
};

}  // namespace mp3d
