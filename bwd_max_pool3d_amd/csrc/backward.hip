// backward.hip -- route each output gradient to its window's argmax.
//
// Definition (PR #308 page, "Add adaptive_max_pool3d_backward Moore
// Threads specialized operator", Summary): gx[p] is the sum of gy[o] over
// the outputs o whose argmax idx[o] is p, and 0 where none is.
//
// The page splits the work two ways, and so does this file:
//  * bwd_gather: when the windows tile every axis each input is reached by
//    at most one window, so every gx element is computed in one pass from
//    the single window containing it -- no zero pass, no atomics, one
//    coalesced store per element.
//  * bwd_tile: when windows overlap several outputs may land on one input.
//    Each workgroup owns a box of one plane's gx, zero-fills a binary32
//    accumulator for it in LDS, adds every gy whose idx falls in the box
//    with LDS float atomics, then rounds and stores the box once.  The
//    zero fill, the atomic scatter and the cast of the page's scheme all
//    happen on-chip, so HBM sees gy and idx read and gx written once.
// Accumulation is binary32 from +0 (so -0 contributions give +0) and the
// sum is rounded once to the storage type.
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

template <typename T>
__global__ void __launch_bounds__(kBlock)
bwd_tile_kernel(const typename T::raw *__restrict__ gy, const int32_t *__restrict__ idx,
                typename T::raw *__restrict__ gx, BwdPlan p)
{
    extern __shared__ __align__(16) float acc[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t D = A.X, H = B.X, W = Cw.X;
    for (int64_t t = blockIdx.x; t < p.ntiles; t += gridDim.x) {
        int64_t q = t;
        const int32_t tw = (int32_t)(q % p.ntw); q /= p.ntw;
        const int32_t th = (int32_t)(q % p.nth); q /= p.nth;
        const int32_t td = (int32_t)(q % p.ntd);
        const int64_t plane = q / p.ntd;
        const int32_t d0 = td * p.td, d1 = min(d0 + p.td, D);
        const int32_t h0 = th * p.th, h1 = min(h0 + p.th, H);
        const int32_t w0 = tw * p.tw, w1 = min(w0 + p.tw, W);
        const int32_t ld = d1 - d0, lh = h1 - h0, lw = w1 - w0;
        const int32_t n = ld * lh * lw;
        const bool full = (lh == H && lw == W);

        for (int32_t e = threadIdx.x; e < n; e += kBlock) acc[e] = 0.0f;
        __syncthreads();

        // windows that can reach the box along each axis
        const int32_t od0 = A.first_reaching(d0), od1 = A.last_starting(d1 - 1) + 1;
        const int32_t oh0 = B.first_reaching(h0), oh1 = B.last_starting(h1 - 1) + 1;
        const int32_t ow0 = Cw.first_reaching(w0), ow1 = Cw.last_starting(w1 - 1) + 1;
        if (od0 < od1 && oh0 < oh1 && ow0 < ow1) {
            const int32_t cd = od1 - od0, ch = oh1 - oh0, cw = ow1 - ow0;
            const int32_t nw = cd * ch * cw;
            const int64_t obase = plane * (int64_t)p.g.out_plane;
            const int32_t ibase = d0 * H * W;
            for (int32_t e = threadIdx.x; e < nw; e += kBlock) {
                const int32_t owl = e % cw, r = e / cw, ohl = r % ch, odl = r / ch;
                const int64_t o = obase + ((od0 + odl) * B.O + oh0 + ohl) * Cw.O + ow0 + owl;
                const int32_t i = idx[o];
                int32_t loc = -1;
                if (full) {
                    const int32_t l = i - ibase;
                    if ((uint32_t)l < (uint32_t)n) loc = l;
                } else if ((uint32_t)i < (uint32_t)p.g.in_plane) {
                    const int32_t d = i / (H * W), rem = i - d * H * W;
                    const int32_t h = rem / W, w = rem - h * W;
                    if (d >= d0 && d < d1 && h >= h0 && h < h1 && w >= w0 && w < w1)
                        loc = ((d - d0) * lh + (h - h0)) * lw + (w - w0);
                }
                if (loc >= 0) atomicAdd(&acc[loc], T::widen(gy[o]));
            }
        }
        __syncthreads();

        typename T::raw *gp = gx + plane * (int64_t)p.g.in_plane;
        if (full) {
            typename T::raw *dst = gp + d0 * H * W;
            for (int32_t e = threadIdx.x; e < n; e += kBlock) dst[e] = T::narrow(acc[e]);
        } else {
            for (int32_t e = threadIdx.x; e < n; e += kBlock) {
                const int32_t w = e % lw, r = e / lw, h = r % lh, d = r / lh;
                gp[((d0 + d) * H + h0 + h) * W + w0 + w] = T::narrow(acc[e]);
            }
        }
        __syncthreads();   // LDS is reused by the next tile
    }
}

template <typename T>
__global__ void __launch_bounds__(kBlock)
bwd_gather_kernel(const typename T::raw *__restrict__ gy, const int32_t *__restrict__ idx,
                  typename T::raw *__restrict__ gx, GatherPlan p)
{
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
    const int32_t OH = p.g.ax[1].O, OW = p.g.ax[2].O;
    const int64_t total = p.g.planes * (int64_t)p.g.in_plane;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kBlock) {
        const int64_t plane = e / p.g.in_plane;
        const int32_t i = (int32_t)(e - plane * p.g.in_plane);
        const int32_t w = i % W, r = i / W, h = r % H, d = r / H;
        const int64_t o = plane * (int64_t)p.g.out_plane +
                          ((d / p.qd) * OH + h / p.qh) * OW + w / p.qw;
        typename T::raw out = T::narrow(0.0f);
        if (idx[o] == i) out = T::narrow(0.0f + T::widen(gy[o]));
        gx[e] = out;
    }
}

}  // namespace

template <typename T>
hipError_t launch_backward_tile(const void *gy, const int32_t *idx, void *gx,
                                const BwdPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t grid = p.ntiles < (1 << 24) ? p.ntiles : (1 << 24);
    hipLaunchKernelGGL(bwd_tile_kernel<T>, dim3((uint32_t)grid), dim3(kBlock),
                       p.lds_bytes, s, (const R *)gy, idx, (R *)gx, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_backward_gather(const void *gy, const int32_t *idx, void *gx,
                                  const GatherPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t total = p.g.planes * (int64_t)p.g.in_plane;
    int64_t grid = (total + kBlock - 1) / kBlock;
    if (grid > (1 << 20)) grid = 1 << 20;
    hipLaunchKernelGGL(bwd_gather_kernel<T>, dim3((uint32_t)grid), dim3(kBlock), 0, s,
                       (const R *)gy, idx, (R *)gx, p);
    return hipGetLastError();
}

template hipError_t launch_backward_tile<F32>(const void *, const int32_t *, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F16>(const void *, const int32_t *, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<BF16>(const void *, const int32_t *, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_gather<F32>(const void *, const int32_t *, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F16>(const void *, const int32_t *, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<BF16>(const void *, const int32_t *, void *, const GatherPlan &, hipStream_t);

}  // namespace mp3d
