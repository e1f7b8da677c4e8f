// forward_ex.hip -- the forward for every geometry the fast kernels do not
// take: fixed windows with padding or dilation (and ceil-mode output
// extents, which only change O), and int64 indices.  One thread per output.
//
// Definition as in the other forward kernels ("Struct Maxpool3dForward",
// teenygrad, description; PR #308 page, Summary): y is the first maximum of
// the window in d, h, w scan order, NaN ranking above every number, and idx
// its flat plane position (d*H + h)*W + w.  Padding: a tap outside the axis
// is never taken; a window with no tap inside the input (possible only
// when dilation steps over the whole axis) gives y = -inf and idx = -1.
#include <math.h>

#include <algorithm>

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

template <typename A>
__device__ __forceinline__ bool better(A v, A best)
{
    return v > best || (v != v && best == best);     // strictly greater, or the first NaN
}

// KM = 3: every window has at most three taps per axis.  The thread loads
// a 3x3x3 block of taps with each tap number clamped to the window's
// in-range taps [j0, j1]: a clamped tap repeats the first in-range row or
// slice just before it, or the last one after it, so the first maximum in
// scan order -- and its position -- is the same as over the window's own
// taps.  All 27 loads are issued before the scan.
// KM = 0: loops over the in-range taps.
template <typename T, typename IT, int KM>
__global__ void __launch_bounds__(kBlock)
fwd_ex_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
              IT *__restrict__ idx, ExPlan p)
{
    using R = typename T::raw;
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X, OH = B.O, OW = Cw.O;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < p.total;
         e += (int64_t)gridDim.x * kBlock) {
        int64_t plane;
        uint32_t o;
        if (p.fast32) {
            plane = p.plane_div.div((uint32_t)e);
            o = (uint32_t)e - (uint32_t)plane * (uint32_t)p.g.out_plane;
        } else {
            plane = e / p.g.out_plane;
            o = (uint32_t)(e - plane * p.g.out_plane);
        }
        const uint32_t r = p.ow_div.div(o);
        const int32_t ow = (int32_t)(o - r * (uint32_t)OW);
        const uint32_t od = p.oh_div.div(r);
        const int32_t oh = (int32_t)(r - od * (uint32_t)OH);
        const Taps td = window_taps(A, (int32_t)od), th = window_taps(B, oh), tw = window_taps(Cw, ow);
        const R *xp = x + plane * (int64_t)p.g.in_plane;
        const bool empty = td.j0 > td.j1 || th.j0 > th.j1 || tw.j0 > tw.j1;
        int32_t pbest = -1;
        R rbest = T::narrow(-INFINITY);
        if constexpr (KM == 3) {
            int32_t cd[3], ch[3], cw[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                // empty windows load position 0 (in bounds) and are overridden
                cd[j] = empty ? 0 : td.b + min(max(j, td.j0), td.j1) * td.t;
                ch[j] = empty ? 0 : th.b + min(max(j, th.j0), th.j1) * th.t;
                cw[j] = empty ? 0 : tw.b + min(max(j, tw.j0), tw.j1) * tw.t;
            }
            R v[27];
            int32_t pos[27];
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int b = 0; b < 3; ++b) {
                    const int32_t row = (cd[a] * H + ch[b]) * W;
#pragma unroll
                    for (int c = 0; c < 3; ++c) {
                        pos[(a * 3 + b) * 3 + c] = row + cw[c];
                        v[(a * 3 + b) * 3 + c] = xp[row + cw[c]];
                    }
                }
            typename T::acc best = T::widen(v[0]);
            pbest = pos[0];
            rbest = v[0];
#pragma unroll
            for (int q = 1; q < 27; ++q) {
                const typename T::acc f = T::widen(v[q]);
                if (better(f, best)) {
                    best = f;
                    pbest = pos[q];
                    rbest = v[q];
                }
            }
            if (empty) {
                pbest = -1;
                rbest = T::narrow(-INFINITY);
            }
        } else {
            if (!empty) {
                typename T::acc best = 0;
                for (int32_t a = td.j0; a <= td.j1; ++a) {
                    const int32_t d = td.b + a * td.t;
                    for (int32_t b = th.j0; b <= th.j1; ++b) {
                        const int32_t row = (d * H + th.b + b * th.t) * W;
                        for (int32_t c = tw.j0; c <= tw.j1; ++c) {
                            const int32_t q = row + tw.b + c * tw.t;
                            const R v = xp[q];
                            const typename T::acc f = T::widen(v);
                            if (pbest < 0 || better(f, best)) {
                                best = f;
                                pbest = q;
                                rbest = v;
                            }
                        }
                    }
                }
            }
        }
        y[e] = rbest;
        if (idx) idx[e] = (IT)pbest;
    }
}

}  // namespace

template <typename T, typename IT>
hipError_t launch_forward_ex(const void *x, void *y, IT *idx, const ExPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t grid = std::min<int64_t>((p.total + kBlock - 1) / kBlock, (int64_t)1 << 20);
    if (p.km == 3)
        launch_kernel((fwd_ex_kernel<T, IT, 3>), dim3((uint32_t)grid), dim3(kBlock), 0, s,
                           (const R *)x, (R *)y, idx, p);
    else
        launch_kernel((fwd_ex_kernel<T, IT, 0>), dim3((uint32_t)grid), dim3(kBlock), 0, s,
                           (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

template hipError_t launch_forward_ex<F32, int32_t>(const void *, void *, int32_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<F16, int32_t>(const void *, void *, int32_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<BF16, int32_t>(const void *, void *, int32_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<F32, int64_t>(const void *, void *, int64_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<F16, int64_t>(const void *, void *, int64_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<BF16, int64_t>(const void *, void *, int64_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<F64, int32_t>(const void *, void *, int32_t *, const ExPlan &, hipStream_t);
template hipError_t launch_forward_ex<F64, int64_t>(const void *, void *, int64_t *, const ExPlan &, hipStream_t);

}  // namespace mp3d
