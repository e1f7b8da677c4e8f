// small.hip -- forward and backward for small tensors with small windows,
// where the cost is latency, not bandwidth: one thread per output (forward)
// or per input element (backward), every load it needs issued at once.
// Also the ordered gather for any geometry, the general fallback of the
// ordered (bit-reproducible) backward.
//
// Definitions as in the other kernels: the forward takes the first maximum
// of each window in d, h, w scan order, NaN ranking above every number
// ("Struct Maxpool3dForward", teenygrad, description; PR #308 page,
// Summary); the backward sets gx[p] to the sum of gy[o] over the outputs o
// whose idx[o] is p (PR #308 page, Summary).
#include <algorithm>

#include "dtype.hpp"
#include "idxsrc.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

__device__ __forceinline__ bool better(float v, float best)
{
    return v > best || (v != v && best == best);     // strictly greater, or the first NaN
}

// One thread per output.  Windows are at most kSmallK wide on every axis;
// the thread loads a kSmallK^3 block whose slots past the window's end
// repeat its last element, so that a repeat comes after the element it
// copies in scan order and never wins.
template <typename T, typename IT>
__global__ void __launch_bounds__(kBlock)
fwd_small_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                 IT *__restrict__ idx, SmallPlan p)
{
    using R = typename T::raw;
    constexpr int K = kSmallK;
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X;
    const uint32_t e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= p.total) return;
    const uint32_t plane = p.plane_div.div(e);
    const int32_t o = (int32_t)(e - plane * (uint32_t)p.g.out_plane);
    const uint32_t r = p.a2_div.div((uint32_t)o);
    const int32_t ow = o - (int32_t)r * Cw.O;
    const uint32_t od = p.a1_div.div(r);
    const int32_t oh = (int32_t)(r - od * (uint32_t)B.O);
    const int32_t d0 = A.start((int32_t)od), nd = A.end((int32_t)od) - d0;
    const int32_t h0 = B.start(oh), nh = B.end(oh) - h0;
    const int32_t w0 = Cw.start(ow), nw = Cw.end(ow) - w0;
    const R *xp = x + (int64_t)plane * p.g.in_plane;

    R v[K][K][K];
    int32_t at[K][K][K];
#pragma unroll
    for (int dd = 0; dd < K; ++dd)
#pragma unroll
        for (int hh = 0; hh < K; ++hh)
#pragma unroll
            for (int ww = 0; ww < K; ++ww) {
                at[dd][hh][ww] = ((d0 + min(dd, nd - 1)) * H + h0 + min(hh, nh - 1)) * W + w0 +
                                 min(ww, nw - 1);
                v[dd][hh][ww] = xp[at[dd][hh][ww]];
            }
    R rbest = v[0][0][0];
    int32_t pbest = at[0][0][0];
    float best = T::widen(rbest);
#pragma unroll
    for (int dd = 0; dd < K; ++dd)
#pragma unroll
        for (int hh = 0; hh < K; ++hh)
#pragma unroll
            for (int ww = 0; ww < K; ++ww) {
                const float c = T::widen(v[dd][hh][ww]);
                const bool take = better(c, best);
                best = take ? c : best;
                rbest = take ? v[dd][hh][ww] : rbest;
                pbest = take ? at[dd][hh][ww] : pbest;
            }
    y[e] = rbest;
    if (idx) idx[e] = pbest;
}

// One thread per input element, reached by at most two windows per axis.
// The (at most 8) windows are visited in ascending output order, so the
// binary32 sum from +0 is the same fold the ordered definition gives, bit
// for bit, and it is rounded once.
template <typename T, typename Src>
__global__ void __launch_bounds__(kBlock)
bwd_small_kernel(const typename T::raw *__restrict__ gy, const Src src,
                 typename T::raw *__restrict__ gx, SmallPlan p)
{
    using R = typename T::raw;
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t OH = B.O, OW = Cw.O;
    const uint32_t e = blockIdx.x * kBlock + threadIdx.x;
    if (e >= p.total) return;
    const uint32_t plane = p.plane_div.div(e);
    const int32_t i = (int32_t)(e - plane * (uint32_t)p.g.in_plane);
    const uint32_t r = p.a2_div.div((uint32_t)i);
    const int32_t w = i - (int32_t)r * Cw.X;
    const uint32_t d = p.a1_div.div(r);
    const int32_t h = (int32_t)(r - d * (uint32_t)B.X);
    int32_t lo[3], hi[3];
    lo[0] = A.first_reaching((int32_t)d);
    hi[0] = A.last_starting((int32_t)d);
    lo[1] = B.first_reaching(h);
    hi[1] = B.last_starting(h);
    lo[2] = Cw.first_reaching(w);
    hi[2] = Cw.last_starting(w);
    const int32_t O[3] = {A.O, OH, OW};
    const int64_t obase = (int64_t)plane * p.g.out_plane;

    int32_t ri[8];
    R rg[8];
    bool on[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        int32_t c[3];
        bool valid = true;
#pragma unroll
        for (int a = 0; a < 3; ++a) {
            const int32_t q = lo[a] + ((k >> (2 - a)) & 1);
            valid = valid && q <= hi[a];
            c[a] = min(max(q, 0), O[a] - 1);          // in range even when unused
        }
        const int64_t o = obase + ((int64_t)c[0] * OH + c[1]) * OW + c[2];
        ri[k] = src(o);
        rg[k] = gy[o];
        on[k] = valid;
    }
    typename T::acc acc = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (on[k] && ri[k] == i) acc = acc + T::widen(rg[k]);
    gx[e] = T::narrow(acc);
}

// Any geometry: one thread per input element (grid-stride) visits every
// window containing it, in ascending output order, and keeps the elements
// whose argmax it is: the ordered binary32 sum from +0, rounded once.  The
// general fallback of the ordered backward; loads follow one another.
template <typename T, typename Src>
__global__ void __launch_bounds__(kBlock)
bwd_ordered_kernel(const typename T::raw *__restrict__ gy, const Src src,
                   typename T::raw *__restrict__ gx, OrdPlan p)
{
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t OH = B.O, OW = Cw.O;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < p.total;
         e += (int64_t)gridDim.x * kBlock) {
        const int64_t plane = e / p.g.in_plane;
        const int32_t i = (int32_t)(e - plane * p.g.in_plane);
        const uint32_t r = p.a2_div.div((uint32_t)i);
        const int32_t w = i - (int32_t)r * Cw.X;
        const uint32_t d = p.a1_div.div(r);
        const int32_t h = (int32_t)(r - d * (uint32_t)B.X);
        const int32_t d0 = A.first_reaching((int32_t)d), d1 = A.last_starting((int32_t)d);
        const int32_t h0 = B.first_reaching(h), h1 = B.last_starting(h);
        const int32_t w0 = Cw.first_reaching(w), w1 = Cw.last_starting(w);
        const int64_t obase = plane * p.g.out_plane;
        typename T::acc acc = 0;
        for (int32_t od = d0; od <= d1; ++od)
            for (int32_t oh = h0; oh <= h1; ++oh)
                for (int32_t ow = w0; ow <= w1; ++ow) {
                    const int64_t o = obase + ((int64_t)od * OH + oh) * OW + ow;
                    const int32_t v = src(o);
                    const typename T::acc g = T::widen(gy[o]);
                    if (v == i) acc = acc + g;
                }
        gx[e] = T::narrow(acc);
    }
}

}  // namespace

template <typename T, typename Src>
hipError_t launch_backward_ordered(const void *gy, const Src &src, void *gx, const OrdPlan &p,
                                   hipStream_t s)
{
    using R = typename T::raw;
    const int64_t grid = std::min<int64_t>((p.total + kBlock - 1) / kBlock, (int64_t)1 << 20);
    launch_kernel((bwd_ordered_kernel<T, Src>), dim3((uint32_t)grid), dim3(kBlock), 0, s,
                       (const R *)gy, src, (R *)gx, p);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_forward_small(const void *x, void *y, IT *idx, const SmallPlan &p,
                                hipStream_t s)
{
    using R = typename T::raw;
    launch_kernel((fwd_small_kernel<T, IT>), dim3((p.total + kBlock - 1) / kBlock), dim3(kBlock), 0,
                       s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

template <typename T, typename Src>
hipError_t launch_backward_small(const void *gy, const Src &src, void *gx, const SmallPlan &p,
                                 hipStream_t s)
{
    using R = typename T::raw;
    launch_kernel((bwd_small_kernel<T, Src>), dim3((p.total + kBlock - 1) / kBlock), dim3(kBlock), 0,
                       s, (const R *)gy, src, (R *)gx, p);
    return hipGetLastError();
}



template hipError_t launch_backward_ordered<F32, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F32, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F32, IdxRecompute<F32>>(const void *, const IdxRecompute<F32> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F32, IdxChecked<F32>>(const void *, const IdxChecked<F32> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_small<F32, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_small<F32, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F16, IdxRecompute<F16>>(const void *, const IdxRecompute<F16> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F16, IdxChecked<F16>>(const void *, const IdxChecked<F16> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_small<F16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_small<F16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_ordered<BF16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<BF16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<BF16, IdxRecompute<BF16>>(const void *, const IdxRecompute<BF16> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<BF16, IdxChecked<BF16>>(const void *, const IdxChecked<BF16> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_small<BF16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_small<BF16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const SmallPlan &, hipStream_t);

template hipError_t launch_backward_ordered<F64, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F64, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F64, IdxRecompute<F64>>(const void *, const IdxRecompute<F64> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_ordered<F64, IdxChecked<F64>>(const void *, const IdxChecked<F64> &, void *, const OrdPlan &, hipStream_t);
template hipError_t launch_backward_small<F64, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const SmallPlan &, hipStream_t);
template hipError_t launch_backward_small<F64, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const SmallPlan &, hipStream_t);

template hipError_t launch_forward_small<F32, int32_t>(const void *, void *, int32_t *, const SmallPlan &, hipStream_t);
template hipError_t launch_forward_small<F16, int32_t>(const void *, void *, int32_t *, const SmallPlan &, hipStream_t);
template hipError_t launch_forward_small<BF16, int32_t>(const void *, void *, int32_t *, const SmallPlan &, hipStream_t);
template hipError_t launch_forward_small<F32, int64_t>(const void *, void *, int64_t *, const SmallPlan &, hipStream_t);
template hipError_t launch_forward_small<F16, int64_t>(const void *, void *, int64_t *, const SmallPlan &, hipStream_t);
template hipError_t launch_forward_small<BF16, int64_t>(const void *, void *, int64_t *, const SmallPlan &, hipStream_t);

}  // namespace mp3d
