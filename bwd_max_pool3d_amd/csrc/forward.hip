// forward.hip -- forward window maximum with int32 per-plane argmax.
//
// Definition ("Struct Maxpool3dForward", teenygrad API docs, description;
// PR #308 page, Summary, for adaptive windows): y[o] is the largest
// element of window o and idx[o] its flat plane position (d*H + h)*W + w.
// The window is scanned d, h, w ascending and the running best is replaced
// only by a strictly larger element, or by a NaN when the best is not NaN,
// so ties go to the earliest element and the first NaN wins.
//
// fwd_tile: each workgroup takes a tile of outputs of one plane, copies the
// input box under it from HBM into LDS with 16-byte coalesced loads (the
// box is one contiguous span when it covers whole H*W slices), and every
// thread then reduces windows out of LDS.  Elements shared by neighbouring
// windows (overlap along d, h or w) are fetched from HBM once per tile.
//
// fwd_direct: one thread per output reading its window straight from
// global memory; used only when no single window's box fits in LDS.
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

__device__ inline bool better(float v, float best) {
    return v > best || (v != v && best == best);
}

// Copy `count` elements from global `src` to LDS `dst`, where dst and src
// agree modulo 16 bytes: the unaligned head and tail go element by
// element, the body in 16-byte vectors with four loads in flight per
// thread before their LDS stores.
template <typename R>
__device__ inline void copy_span(R *dst, const R *__restrict__ src, int32_t count) {
    const int tid = threadIdx.x;
    const uintptr_t a = (uintptr_t)src;
    int32_t head = (int32_t)(((16u - (a & 15u)) & 15u) / sizeof(R));
    if (head > count) head = count;
    const int32_t nvec = (int32_t)(((int64_t)(count - head) * (int32_t)sizeof(R)) / 16);
    const int32_t tail0 = head + nvec * (int32_t)(16 / sizeof(R));
    if (tid < head) dst[tid] = src[tid];
    const uint4 *vs = reinterpret_cast<const uint4 *>(src + head);
    uint4 *vd = reinterpret_cast<uint4 *>(dst + head);
    int32_t i = tid;
    for (; i + 3 * kBlock < nvec; i += 4 * kBlock) {
        uint4 a0 = vs[i];
        uint4 a1 = vs[i + kBlock];
        uint4 a2 = vs[i + 2 * kBlock];
        uint4 a3 = vs[i + 3 * kBlock];
        vd[i] = a0;
        vd[i + kBlock] = a1;
        vd[i + 2 * kBlock] = a2;
        vd[i + 3 * kBlock] = a3;
    }
    for (; i < nvec; i += kBlock) vd[i] = vs[i];
    if (tid < count - tail0) dst[tail0 + tid] = src[tail0 + tid];
}

template <typename T>
__global__ void __launch_bounds__(kBlock)
fwd_tile_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                int32_t *__restrict__ idx, FwdPlan p)
{
    using R = typename T::raw;
    extern __shared__ __align__(16) unsigned char smem[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X;
    const int32_t ntab = p.tod + p.toh + p.tow;
    int2 *tab = reinterpret_cast<int2 *>(smem);
    unsigned char *boxbase = smem + ((ntab * (int)sizeof(int2) + 15) & ~15);

    for (int64_t t = blockIdx.x; t < p.ntiles; t += gridDim.x) {
        int64_t q = t;
        const int32_t tw = (int32_t)(q % p.ntw); q /= p.ntw;
        const int32_t th = (int32_t)(q % p.nth); q /= p.nth;
        const int32_t td = (int32_t)(q % p.ntd);
        const int64_t plane = q / p.ntd;
        const int32_t od0 = td * p.tod, od1 = min(od0 + p.tod, A.O);
        const int32_t oh0 = th * p.toh, oh1 = min(oh0 + p.toh, B.O);
        const int32_t ow0 = tw * p.tow, ow1 = min(ow0 + p.tow, Cw.O);
        const int32_t bd0 = A.start(od0), bd1 = A.end(od1 - 1);
        const int32_t bh0 = p.full_h ? 0 : B.start(oh0);
        const int32_t bh1 = p.full_h ? H : B.end(oh1 - 1);
        const int32_t bw0 = p.full_w ? 0 : Cw.start(ow0);
        const int32_t bw1 = p.full_w ? W : Cw.end(ow1 - 1);
        const int32_t ld = bd1 - bd0, lh = bh1 - bh0, lw = bw1 - bw0;
        const R *xp = x + plane * (int64_t)p.g.in_plane;

        R *box;
        if (p.full_h && p.full_w) {
            const R *src = xp + bd0 * H * W;
            box = reinterpret_cast<R *>(boxbase + ((uintptr_t)src & 15u));
            copy_span(box, src, ld * H * W);
        } else {
            box = reinterpret_cast<R *>(boxbase);
            const int32_t n = ld * lh * lw;
            for (int32_t e = threadIdx.x; e < n; e += kBlock) {
                const int32_t w = e % lw, r = e / lw, h = r % lh, d = r / lh;
                box[e] = xp[((bd0 + d) * H + bh0 + h) * W + bw0 + w];
            }
        }
        for (int32_t j = threadIdx.x; j < ntab; j += kBlock) {
            int2 v = make_int2(0, 0);
            if (j < p.tod) {
                const int32_t o = od0 + j;
                if (o < od1) v = make_int2(A.start(o), A.end(o));
            } else if (j < p.tod + p.toh) {
                const int32_t o = oh0 + j - p.tod;
                if (o < oh1) v = make_int2(B.start(o), B.end(o));
            } else {
                const int32_t o = ow0 + j - p.tod - p.toh;
                if (o < ow1) v = make_int2(Cw.start(o), Cw.end(o));
            }
            tab[j] = v;
        }
        __syncthreads();

        const int32_t cd = od1 - od0, ch = oh1 - oh0, cw = ow1 - ow0;
        const int32_t nout = cd * ch * cw;
        const int64_t obase = plane * (int64_t)p.g.out_plane;
        for (int32_t e = threadIdx.x; e < nout; e += kBlock) {
            const int32_t owl = e % cw, r = e / cw, ohl = r % ch, odl = r / ch;
            const int2 wd = tab[odl], wh = tab[p.tod + ohl], ww = tab[p.tod + p.toh + owl];
            int32_t rb = ((wd.x - bd0) * lh + (wh.x - bh0)) * lw - bw0;
            R rbest = box[rb + ww.x];
            float best = T::widen(rbest);
            int32_t pbest = (wd.x * H + wh.x) * W + ww.x;
            for (int32_t d = wd.x; d < wd.y; ++d) {
                for (int32_t h = wh.x; h < wh.y; ++h) {
                    const int32_t rowl = ((d - bd0) * lh + (h - bh0)) * lw - bw0;
                    const int32_t rowp = (d * H + h) * W;
                    for (int32_t w = ww.x; w < ww.y; ++w) {
                        const R rv = box[rowl + w];
                        const float v = T::widen(rv);
                        if (better(v, best)) {
                            best = v;
                            rbest = rv;
                            pbest = rowp + w;
                        }
                    }
                }
            }
            const int64_t o = obase + ((od0 + odl) * B.O + oh0 + ohl) * Cw.O + ow0 + owl;
            y[o] = rbest;
            idx[o] = pbest;
        }
        __syncthreads();   // LDS is reused by the next tile
    }
}

template <typename T>
__global__ void __launch_bounds__(kBlock)
fwd_direct_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                  int32_t *__restrict__ idx, Geom g)
{
    using R = typename T::raw;
    const Axis A = g.ax[0], B = g.ax[1], Cw = g.ax[2];
    const int32_t H = B.X, W = Cw.X;
    const int64_t total = g.planes * (int64_t)g.out_plane;
    for (int64_t e = (int64_t)blockIdx.x * kBlock + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kBlock) {
        const int64_t plane = e / g.out_plane;
        const int32_t o = (int32_t)(e - plane * g.out_plane);
        const int32_t ow = o % Cw.O, r = o / Cw.O, oh = r % B.O, od = r / B.O;
        const int32_t d0 = A.start(od), d1 = A.end(od);
        const int32_t h0 = B.start(oh), h1 = B.end(oh);
        const int32_t w0 = Cw.start(ow), w1 = Cw.end(ow);
        const R *xp = x + plane * (int64_t)g.in_plane;
        int32_t pbest = (d0 * H + h0) * W + w0;
        R rbest = xp[pbest];
        float best = T::widen(rbest);
        for (int32_t d = d0; d < d1; ++d)
            for (int32_t h = h0; h < h1; ++h) {
                const int32_t rowp = (d * H + h) * W;
                for (int32_t w = w0; w < w1; ++w) {
                    const R rv = xp[rowp + w];
                    const float v = T::widen(rv);
                    if (better(v, best)) {
                        best = v;
                        rbest = rv;
                        pbest = rowp + w;
                    }
                }
            }
        y[e] = rbest;
        idx[e] = pbest;
    }
}

}  // namespace

template <typename T>
hipError_t launch_forward_tile(const void *x, void *y, int32_t *idx,
                               const FwdPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t grid = p.ntiles < (1 << 24) ? p.ntiles : (1 << 24);
    hipLaunchKernelGGL(fwd_tile_kernel<T>, dim3((uint32_t)grid), dim3(kBlock),
                       p.lds_bytes, s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_forward_direct(const void *x, void *y, int32_t *idx,
                                 const Geom &g, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t total = g.planes * (int64_t)g.out_plane;
    int64_t grid = (total + kBlock - 1) / kBlock;
    if (grid > (1 << 20)) grid = 1 << 20;
    hipLaunchKernelGGL(fwd_direct_kernel<T>, dim3((uint32_t)grid), dim3(kBlock), 0, s,
                       (const R *)x, (R *)y, idx, g);
    return hipGetLastError();
}

template hipError_t launch_forward_tile<F32>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<F16>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<BF16>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_direct<F32>(const void *, void *, int32_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<F16>(const void *, void *, int32_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<BF16>(const void *, void *, int32_t *, const Geom &, hipStream_t);

}  // namespace mp3d
