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
#include <algorithm>

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

__device__ __forceinline__ bool better(float v, float best) {
    return v > best || (v != v && best == best);
}

constexpr int kPrefetch = 16;   // 16-byte vectors per thread carried between tiles

// A tile: a block of outputs of one plane and the input box under it.
struct Tile {
    int64_t plane;
    int32_t od0, od1, oh0, oh1, ow0, ow1;   // outputs [od0, od1) x ...
    int32_t bd0, bd1, bh0, bh1, bw0, bw1;   // input box [bd0, bd1) x ...
};

__device__ __forceinline__ Tile tile_at(const FwdPlan &p, int64_t t)
{
    const Axis &A = p.g.ax[0], &B = p.g.ax[1], &Cw = p.g.ax[2];
    Tile r;
    int32_t td, th, tw;
    p.split.split(t, &r.plane, &td, &th, &tw);
    r.od0 = td * p.tod; r.od1 = min(r.od0 + p.tod, A.O);
    r.oh0 = th * p.toh; r.oh1 = min(r.oh0 + p.toh, B.O);
    r.ow0 = tw * p.tow; r.ow1 = min(r.ow0 + p.tow, Cw.O);
    r.bd0 = A.start(r.od0); r.bd1 = A.end(r.od1 - 1);
    r.bh0 = p.full_h ? 0 : B.start(r.oh0); r.bh1 = p.full_h ? B.X : B.end(r.oh1 - 1);
    r.bw0 = p.full_w ? 0 : Cw.start(r.ow0); r.bw1 = p.full_w ? Cw.X : Cw.end(r.ow1 - 1);
    return r;
}

// A contiguous span of x split into an unaligned head, whole 16-byte
// vectors, and a tail.  The LDS copy starts at the same address modulo 16,
// so the vectors land aligned.
struct SpanShape {
    int32_t head, nvec, tail0, count;
};

template <typename R>
__device__ __forceinline__ SpanShape span_shape(const R *src, int32_t count)
{
    SpanShape s;
    const uintptr_t a = (uintptr_t)src;
    s.head = min((int32_t)(((16u - (a & 15u)) & 15u) / sizeof(R)), count);
    s.nvec = (int32_t)(((int64_t)(count - s.head) * (int32_t)sizeof(R)) / 16);
    s.tail0 = s.head + s.nvec * (int32_t)(16 / sizeof(R));
    s.count = count;
    return s;
}

// Registers holding one tile's span between its load and its LDS store.
template <typename R>
struct SpanRegs {
    u32x4 v[kPrefetch];
    R head, tail;
};

template <typename R>
__device__ __forceinline__ void span_fetch(SpanRegs<R> &r, const R *__restrict__ src, const SpanShape &s)
{
    const int tid = threadIdx.x;
    const u32x4 *vs = reinterpret_cast<const u32x4 *>(src + s.head);
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const int32_t i = k * kBlock + tid;
        if (i < s.nvec) r.v[k] = vs[i];
    }
    if (tid < s.head) r.head = src[tid];
    if (tid < s.count - s.tail0) r.tail = src[s.tail0 + tid];
}

template <typename R>
__device__ __forceinline__ void span_put(const SpanRegs<R> &r, R *dst, const SpanShape &s)
{
    const int tid = threadIdx.x;
    u32x4 *vd = reinterpret_cast<u32x4 *>(dst + s.head);
#pragma unroll
    for (int k = 0; k < kPrefetch; ++k) {
        const int32_t i = k * kBlock + tid;
        if (i < s.nvec) vd[i] = r.v[k];
    }
    if (tid < s.head) dst[tid] = r.head;
    if (tid < s.count - s.tail0) dst[s.tail0 + tid] = r.tail;
}

// Window bounds of the tile's outputs, per axis, into the LDS table.
__device__ __forceinline__ void write_table(int2 *tab, const FwdPlan &p, const Tile &tl)
{
    const Axis &A = p.g.ax[0], &B = p.g.ax[1], &Cw = p.g.ax[2];
    const int32_t ntab = p.tod + p.toh + p.tow;
    for (int32_t j = threadIdx.x; j < ntab; j += kBlock) {
        int2 v = make_int2(0, 0);
        if (j < p.tod) {
            const int32_t o = tl.od0 + j;
            if (o < tl.od1) v = make_int2(A.start(o), A.end(o));
        } else if (j < p.tod + p.toh) {
            const int32_t o = tl.oh0 + j - p.tod;
            if (o < tl.oh1) v = make_int2(B.start(o), B.end(o));
        } else {
            const int32_t o = tl.ow0 + j - p.tod - p.toh;
            if (o < tl.ow1) v = make_int2(Cw.start(o), Cw.end(o));
        }
        tab[j] = v;
    }
}

// Reduce every window of the tile out of its LDS box.
//  stage B: for every box row and output column, the first maximum of the
//           row over that column's window (value, column) -> LDS;
//  stage C: every output combines the row partials of its window's (d, h)
//           rows in ascending order, then stores y (the element's own
//           bits, read back from the box) and idx.
template <typename T, typename IT>
__device__ __forceinline__ void reduce_tile(const FwdPlan &p, const Tile &tl, const int2 *tab,
                                   const typename T::raw *box, float *pv, int32_t *pw,
                                   typename T::raw *__restrict__ y, IT *__restrict__ idx)
{
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X, OH = p.g.ax[1].O, OW = p.g.ax[2].O;
    const int32_t tid = threadIdx.x;
    const int32_t lh = tl.bh1 - tl.bh0, lw = tl.bw1 - tl.bw0;
    const int32_t cd = tl.od1 - tl.od0, ch = tl.oh1 - tl.oh0, cw = tl.ow1 - tl.ow0;
    const int32_t nrow = (tl.bd1 - tl.bd0) * lh;

    for (int32_t ob = 0; ob < cw; ob += kBlock) {
        const int32_t cwb = min(cw - ob, kBlock);
        const int32_t owl = ob + tid % cwb, rstep = kBlock / cwb;
        if (tid < rstep * cwb) {
            const int2 ww = tab[p.tod + p.toh + owl];
            for (int32_t r = tid / cwb; r < nrow; r += rstep) {
                const int32_t rb = r * lw - tl.bw0;
                float best = T::widen(box[rb + ww.x]);
                int32_t bw = ww.x;
#pragma unroll 4
                for (int32_t w = ww.x + 1; w < ww.y; ++w) {
                    const float v = T::widen(box[rb + w]);
                    if (better(v, best)) {
                        best = v;
                        bw = w;
                    }
                }
                pv[r * cw + owl] = best;
                pw[r * cw + owl] = bw;
            }
        }
    }
    __syncthreads();

    const int64_t obase = tl.plane * (int64_t)p.g.out_plane;
    for (int32_t ob = 0; ob < cw; ob += kBlock) {
        const int32_t cwb = min(cw - ob, kBlock);
        const int32_t owl = ob + tid % cwb, qstep = kBlock / cwb;
        if (tid < qstep * cwb) {
            for (int32_t qq = tid / cwb; qq < cd * ch; qq += qstep) {
                const int32_t odl = qq / ch, ohl = qq - odl * ch;
                const int2 wd = tab[odl], wh = tab[p.tod + ohl];
                float best = pv[((wd.x - tl.bd0) * lh + (wh.x - tl.bh0)) * cw + owl];
                int32_t bd = wd.x, bh = wh.x;
                for (int32_t d = wd.x; d < wd.y; ++d) {
                    const int32_t r0 = (d - tl.bd0) * lh - tl.bh0;
#pragma unroll 4
                    for (int32_t h = wh.x; h < wh.y; ++h) {
                        const float v = pv[(r0 + h) * cw + owl];
                        if (better(v, best)) {
                            best = v;
                            bd = d;
                            bh = h;
                        }
                    }
                }
                const int32_t rr = (bd - tl.bd0) * lh + (bh - tl.bh0);
                const int32_t bw = pw[rr * cw + owl];
                const int64_t o = obase + ((tl.od0 + odl) * OH + tl.oh0 + ohl) * OW + tl.ow0 + owl;
                y[o] = box[rr * lw + bw - tl.bw0];
                if (idx) idx[o] = (bd * H + bh) * W + bw;
            }
        }
    }
}

template <typename T, typename IT>
__global__ void __launch_bounds__(kBlock)
fwd_tile_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                IT *__restrict__ idx, FwdPlan p)
{
    using R = typename T::raw;
    extern __shared__ __align__(16) unsigned char smem[];
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
    // LDS: window table | row partials (value, column) | input box
    int2 *tab = reinterpret_cast<int2 *>(smem);
    float *pv = reinterpret_cast<float *>(smem + p.tab_bytes);
    int32_t *pw = reinterpret_cast<int32_t *>(smem + p.tab_bytes + p.part_bytes);
    unsigned char *boxbase = smem + p.tab_bytes + 2 * p.part_bytes;
    const int64_t first = xcd_local_block(blockIdx.x, gridDim.x);

    if (p.full_h && p.full_w) {
        // Boxes are whole slices, one contiguous span of the plane.  The
        // workgroup is persistent and pipelined: the next tile's span is
        // in flight in registers while the current tile is reduced.
        SpanRegs<R> regs;
        if (first < p.ntiles) {
            const Tile tl = tile_at(p, first);
            const R *src = x + tl.plane * (int64_t)p.g.in_plane + tl.bd0 * H * W;
            span_fetch(regs, src, span_shape(src, (tl.bd1 - tl.bd0) * H * W));
        }
        for (int64_t t = first; t < p.ntiles; t += gridDim.x) {
            const Tile tl = tile_at(p, t);
            const R *src = x + tl.plane * (int64_t)p.g.in_plane + tl.bd0 * H * W;
            R *box = reinterpret_cast<R *>(boxbase + ((uintptr_t)src & 15u));
            span_put(regs, box, span_shape(src, (tl.bd1 - tl.bd0) * H * W));
            write_table(tab, p, tl);
            __syncthreads();
            if (t + gridDim.x < p.ntiles) {
                const Tile nx = tile_at(p, t + gridDim.x);
                const R *ns = x + nx.plane * (int64_t)p.g.in_plane + nx.bd0 * H * W;
                span_fetch(regs, ns, span_shape(ns, (nx.bd1 - nx.bd0) * H * W));
            }
            reduce_tile<T, IT>(p, tl, tab, box, pv, pw, y, idx);
            __syncthreads();   // LDS is reused by the next tile
        }
    } else {
        for (int64_t t = first; t < p.ntiles; t += gridDim.x) {
            const Tile tl = tile_at(p, t);
            const R *xp = x + tl.plane * (int64_t)p.g.in_plane;
            R *box = reinterpret_cast<R *>(boxbase);
            const int32_t lh = tl.bh1 - tl.bh0, lw = tl.bw1 - tl.bw0;
            const int32_t n = (tl.bd1 - tl.bd0) * lh * lw;
            for (int32_t e = threadIdx.x; e < n; e += kBlock) {
                const int32_t w = e % lw, r = e / lw, h = r % lh, d = r / lh;
                box[e] = xp[((tl.bd0 + d) * H + tl.bh0 + h) * W + tl.bw0 + w];
            }
            write_table(tab, p, tl);
            __syncthreads();
            reduce_tile<T, IT>(p, tl, tab, box, pv, pw, y, idx);
            __syncthreads();
        }
    }
}

template <typename T, typename IT>
__global__ void __launch_bounds__(kBlock)
fwd_direct_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                  IT *__restrict__ idx, Geom g)
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
        if (idx) idx[e] = pbest;
    }
}

}  // namespace

template <typename T, typename IT>
hipError_t launch_forward_tile(const void *x, void *y, IT *idx, const FwdPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    // persistent: as many workgroups as can be resident at once
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fwd_tile_kernel<T, IT>, kBlock,
                                                     p.lds_bytes) != hipSuccess || per_cu < 1)
        per_cu = 1;
    int64_t grid = std::min<int64_t>(p.ntiles, (int64_t)per_cu * device_cus());
    if (grid >= 64) grid &= ~(int64_t)7;    // a multiple of 8 lets blocks map per XCD
    launch_kernel((fwd_tile_kernel<T, IT>), dim3((uint32_t)grid), dim3(kBlock),
                       p.lds_bytes, s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

template <typename T, typename IT>
hipError_t launch_forward_direct(const void *x, void *y, IT *idx, const Geom &g, hipStream_t s)
{
    using R = typename T::raw;
    const int64_t total = g.planes * (int64_t)g.out_plane;
    int64_t grid = (total + kBlock - 1) / kBlock;
    if (grid > (1 << 20)) grid = 1 << 20;
    launch_kernel((fwd_direct_kernel<T, IT>), dim3((uint32_t)grid), dim3(kBlock), 0, s,
                       (const R *)x, (R *)y, idx, g);
    return hipGetLastError();
}

template hipError_t launch_forward_tile<F32, int32_t>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<F16, int32_t>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<BF16, int32_t>(const void *, void *, int32_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<F32, int64_t>(const void *, void *, int64_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<F16, int64_t>(const void *, void *, int64_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_tile<BF16, int64_t>(const void *, void *, int64_t *, const FwdPlan &, hipStream_t);
template hipError_t launch_forward_direct<F32, int32_t>(const void *, void *, int32_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<F16, int32_t>(const void *, void *, int32_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<BF16, int32_t>(const void *, void *, int32_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<F32, int64_t>(const void *, void *, int64_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<F16, int64_t>(const void *, void *, int64_t *, const Geom &, hipStream_t);
template hipError_t launch_forward_direct<BF16, int64_t>(const void *, void *, int64_t *, const Geom &, hipStream_t);

}  // namespace mp3d
