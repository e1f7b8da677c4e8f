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
#include <algorithm>
#include <climits>

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// Blocks are dealt to the 8 XCDs round-robin by block id; renumber them so
// that each XCD walks one contiguous run of tiles (tiles of one plane re-read
// the windows on their borders through that XCD's L2).
__device__ __forceinline__ uint32_t xcd_local_block(uint32_t b, uint32_t nblocks)
{
    if (nblocks % 8u) return b;
    return (b % 8u) * (nblocks / 8u) + b / 8u;
}

// Pack VE rounded accumulator values into one 16-byte store.
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float *a)
{
    if constexpr (sizeof(typename T::raw) == 4) {
        return *reinterpret_cast<const u32x4 *>(a);
    } else {
        const float4 u = *reinterpret_cast<const float4 *>(a);
        const float4 v = *reinterpret_cast<const float4 *>(a + 4);
        auto two = [](float lo, float hi) {
            return (uint32_t)T::narrow(lo) | ((uint32_t)T::narrow(hi) << 16);
        };
        return u32x4{two(u.x, u.y), two(u.z, u.w), two(v.x, v.y), two(v.z, v.w)};
    }
}

constexpr int kRound = 8;   // windows per thread fetched per round

// An input box of one plane and the windows that can reach it.
struct BTile {
    int64_t plane;
    int32_t d0, d1, h0, h1, w0, w1;        // input box
    int32_t od0, oh0, ow0, cd, ch, cw;      // reaching windows: [od0, od0+cd) x ...
    int32_t n, nw;                          // box elements, reaching windows
    bool full;                              // whole rows and slices: one span
};

__device__ __forceinline__ BTile btile_at(const BwdPlan &p, int64_t t)
{
    const Axis &A = p.g.ax[0], &B = p.g.ax[1], &Cw = p.g.ax[2];
    BTile b;
    int32_t td, th, tw;
    p.split.split(t, &b.plane, &td, &th, &tw);
    b.d0 = td * p.td; b.d1 = min(b.d0 + p.td, A.X);
    b.h0 = th * p.th; b.h1 = min(b.h0 + p.th, B.X);
    b.w0 = tw * p.tw; b.w1 = min(b.w0 + p.tw, Cw.X);
    b.n = (b.d1 - b.d0) * (b.h1 - b.h0) * (b.w1 - b.w0);
    b.full = (b.h1 - b.h0 == B.X) && (b.w1 - b.w0 == Cw.X);
    b.od0 = A.first_reaching(b.d0);
    b.oh0 = B.first_reaching(b.h0);
    b.ow0 = Cw.first_reaching(b.w0);
    b.cd = max(A.last_starting(b.d1 - 1) + 1 - b.od0, 0);
    b.ch = max(B.last_starting(b.h1 - 1) + 1 - b.oh0, 0);
    b.cw = max(Cw.last_starting(b.w1 - 1) + 1 - b.ow0, 0);
    b.nw = b.cd * b.ch * b.cw;
    return b;
}

// Issue the loads of one round of (idx, gy) pairs of tile b; i = INT_MIN
// marks an empty slot.  Decoding waits until the values are needed.
template <typename T>
__device__ __forceinline__ void fetch_round(const BwdPlan &p, const BTile &b, int32_t round,
                                            const typename T::raw *__restrict__ gy,
                                            const int32_t *__restrict__ idx,
                                            int32_t (&ri)[kRound], typename T::raw (&rg)[kRound])
{
    const int64_t obase = b.plane * (int64_t)p.g.out_plane;
    const int32_t OH = p.g.ax[1].O, OW = p.g.ax[2].O;
#pragma unroll
    for (int k = 0; k < kRound; ++k) {
        const int32_t e = (round * kRound + k) * kBlock + (int32_t)threadIdx.x;
        ri[k] = INT32_MIN;
        if (e < b.nw) {
            int32_t owl, ohl, odl;
            if (b.full) {       // cw == OW and ch == OH: divide by launch constants
                const uint32_t r = p.ow_div.div((uint32_t)e);
                owl = e - (int32_t)r * OW;
                odl = (int32_t)p.oh_div.div(r);
                ohl = (int32_t)r - odl * OH;
            } else {
                owl = e % b.cw;
                const int32_t r = e / b.cw;
                ohl = r % b.ch;
                odl = r / b.ch;
            }
            const int64_t o = obase + ((b.od0 + odl) * OH + b.oh0 + ohl) * OW + b.ow0 + owl;
            ri[k] = idx[o];
            rg[k] = gy[o];
        }
    }
}

template <typename T>
__global__ void __launch_bounds__(kBlock)
bwd_tile_kernel(const typename T::raw *__restrict__ gy, const int32_t *__restrict__ idx,
                typename T::raw *__restrict__ gx, BwdPlan p)
{
    using R = typename T::raw;
    constexpr int VE = 16 / (int)sizeof(R);   // gx elements per 16-byte store
    extern __shared__ __align__(16) float acc[];
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
    const int32_t tid = threadIdx.x;
    const int64_t first = xcd_local_block(blockIdx.x, gridDim.x);

    // The workgroup is persistent: round 0 of the next tile's (idx, gy)
    // loads is issued before this tile's store phase.
    int32_t ri[kRound];
    R rg[kRound];
    if (first < p.ntiles) fetch_round<T>(p, btile_at(p, first), 0, gy, idx, ri, rg);

    for (int64_t t = first; t < p.ntiles; t += gridDim.x) {
        const BTile b = btile_at(p, t);
        const int32_t lh = b.h1 - b.h0, lw = b.w1 - b.w0;
        R *gp = gx + b.plane * (int64_t)p.g.in_plane;
        R *dst = gp + b.d0 * H * W;                 // the box, when rows are whole

        // the accumulator is shifted so that its element e and dst[e] share
        // their alignment: whole 16-byte gx vectors map to aligned LDS reads
        const int32_t mis = (int32_t)(((uintptr_t)dst / sizeof(R)) % VE);
        const int32_t head = b.full ? min((VE - mis) % VE, b.n) : 0;
        const int32_t shift = (4 - head % 4) % 4;
        float *a = acc + shift;
        const int32_t ibase = b.d0 * H * W;

        // zero fill, 16 bytes at a time
        for (int32_t e = tid; e < (b.n + shift + 3) / 4; e += kBlock)
            reinterpret_cast<u32x4 *>(acc)[e] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        for (int32_t round = 0;; ++round) {
#pragma unroll
            for (int k = 0; k < kRound; ++k) {
                const int32_t i = ri[k];
                int32_t loc = -1;
                if (b.full) {
                    const uint32_t l = (uint32_t)i - (uint32_t)ibase;
                    if (i != INT32_MIN && l < (uint32_t)b.n) loc = (int32_t)l;
                } else if ((uint32_t)i < (uint32_t)p.g.in_plane) {
                    const int32_t d = i / (H * W), rem = i - d * H * W;
                    const int32_t h = rem / W, w = rem - h * W;
                    if (d >= b.d0 && d < b.d1 && h >= b.h0 && h < b.h1 && w >= b.w0 && w < b.w1)
                        loc = ((d - b.d0) * lh + (h - b.h0)) * lw + (w - b.w0);
                }
                if (loc >= 0) atomicAdd(&a[loc], T::widen(rg[k]));   // ds_add_f32 scatter
            }
            if ((round + 1) * kRound * kBlock >= b.nw) break;
            fetch_round<T>(p, b, round + 1, gy, idx, ri, rg);
        }
        __syncthreads();
        if (t + gridDim.x < p.ntiles) fetch_round<T>(p, btile_at(p, t + gridDim.x), 0, gy, idx, ri, rg);

        // one rounding store per gx element
        if (b.full) {
            const int32_t nvec = (b.n - head) / VE;
            const int32_t tail0 = head + nvec * VE;
            if (tid < head) dst[tid] = T::narrow(a[tid]);
            u32x4 *vd = reinterpret_cast<u32x4 *>(dst + head);
            int32_t i = tid;
            for (; i + 3 * kBlock < nvec; i += 4 * kBlock) {     // four LDS reads in flight
                const u32x4 v0 = pack16<T>(a + head + i * VE);
                const u32x4 v1 = pack16<T>(a + head + (i + kBlock) * VE);
                const u32x4 v2 = pack16<T>(a + head + (i + 2 * kBlock) * VE);
                const u32x4 v3 = pack16<T>(a + head + (i + 3 * kBlock) * VE);
                st_stream(vd + i, v0);
                st_stream(vd + i + kBlock, v1);
                st_stream(vd + i + 2 * kBlock, v2);
                st_stream(vd + i + 3 * kBlock, v3);
            }
            for (; i < nvec; i += kBlock) st_stream(vd + i, pack16<T>(a + head + i * VE));
            if (tid < b.n - tail0) dst[tail0 + tid] = T::narrow(a[tail0 + tid]);
        } else {
            for (int32_t e = tid; e < b.n; e += kBlock) {
                const int32_t w = e % lw, r = e / lw, h = r % lh, d = r / lh;
                gp[((b.d0 + d) * H + b.h0 + h) * W + b.w0 + w] = T::narrow(a[e]);
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
    // one workgroup per tile (measured faster than a persistent grid here:
    // the store phases of many resident workgroups overlap)
    int64_t grid = std::min<int64_t>(p.ntiles, (int64_t)1 << 24);
    if (grid >= 64) grid &= ~(int64_t)7;    // a multiple of 8 lets blocks map per XCD
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
