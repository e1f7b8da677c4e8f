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
//  * bwd_slab / bwd_box: when windows overlap several outputs may land on
//    one input.  Each workgroup owns a box of one plane's gx (whole slices
//    when they fit), zero-fills an accumulator for it in LDS (binary32;
//    binary64 for the float64 dtype), adds
//    every gy whose idx falls in the box with an LDS compare-and-swap loop,
//    then rounds and stores the box once.  The zero fill, the atomic
//    scatter and the cast of the page's scheme all happen on-chip, so HBM
//    sees gy and idx read and gx written once.
// (Small tensors take the ordered gather of small.hip instead.)
// Accumulation is binary32 from +0 (so -0 contributions give +0) and the
// sum is rounded once to the storage type.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "colstage.hpp"
#include "dtype.hpp"
#include "idxsrc.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// Pack VE rounded accumulator values into one 16-byte store (binary32 and
// binary64 cells are stored as they are).
template <typename T>
__device__ __forceinline__ u32x4 pack16(const typename T::acc *a)
{
    if constexpr (sizeof(typename T::raw) == sizeof(typename T::acc)) {
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

// a[0] += v in LDS as a compare-and-swap loop.  On gfx950 the LDS float
// atomic add (ds_add_f32) measured about 193 cycles per wave instruction
// per CU against about 14 for a read plus ds_cmpst_rtn_b32; without a
// collision the loop body runs once.  Each successful swap applies exactly
// one addition, so the element ends as a binary32 fold of its
// contributions in the order the swaps landed.
__device__ __forceinline__ void lds_add(float *a, float v)
{
    uint32_t *u = reinterpret_cast<uint32_t *>(a);
    uint32_t old = *u;
    for (;;) {
        const uint32_t want = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, old) + v);
        const uint32_t seen = atomicCAS(u, old, want);
        if (seen == old) break;
        old = seen;
    }
}

// The same in binary64 (the float64 dtype), with a 64-bit compare-and-swap.
__device__ __forceinline__ void lds_add(double *a, double v)
{
    unsigned long long *u = reinterpret_cast<unsigned long long *>(a);
    unsigned long long old = *u;
    for (;;) {
        const unsigned long long want =
            __builtin_bit_cast(unsigned long long, __builtin_bit_cast(double, old) + v);
        const unsigned long long seen = atomicCAS(u, old, want);
        if (seen == old) break;
        old = seen;
    }
}

constexpr int kSlabBlock = kSlabThreads;  // threads per slab workgroup

// Round the accumulator a[0, n) into dst[0, n): 16-byte streaming stores for
// the aligned body (four LDS reads in flight per thread), element stores
// for the unaligned head and tail.  a[e] and dst[e] share their alignment
// modulo one 16-byte vector.
template <typename T, int NT>
__device__ __forceinline__ void store_span(typename T::raw *dst, const typename T::acc *a, int32_t n,
                                           int32_t head)
{
    constexpr int VE = 16 / (int)sizeof(typename T::raw);
    const int32_t tid = threadIdx.x;
    const int32_t nvec = (n - head) / VE;
    const int32_t tail0 = head + nvec * VE;
    if (tid < head) dst[tid] = T::narrow(a[tid]);
    u32x4 *vd = reinterpret_cast<u32x4 *>(dst + head);
    int32_t i = tid;
    for (; i + 3 * NT < nvec; i += 4 * NT) {
        const u32x4 v0 = pack16<T>(a + head + i * VE);
        const u32x4 v1 = pack16<T>(a + head + (i + NT) * VE);
        const u32x4 v2 = pack16<T>(a + head + (i + 2 * NT) * VE);
        const u32x4 v3 = pack16<T>(a + head + (i + 3 * NT) * VE);
        st_stream(vd + i, v0);
        st_stream(vd + i + NT, v1);
        st_stream(vd + i + 2 * NT, v2);
        st_stream(vd + i + 3 * NT, v3);
    }
    for (; i < nvec; i += NT) st_stream(vd + i, pack16<T>(a + head + i * VE));
    if (tid < n - tail0) dst[tail0 + tid] = T::narrow(a[tail0 + tid]);
}

// Slabs of whole H*W slices [d0, d1) of one plane.  Every window of the
// output slices [od0, od1) that can reach the slab is one contiguous run of
// gy and idx, and the slab is one contiguous run of gx.
//
// ORD false: the scatter adds with lds_add (compare-and-swap), in the order
// the swaps land.  ORD true: one round holds every window (the plan sees to
// it); each window's class is its rank among the windows containing its
// argmax, (rank_d * mh + rank_h) * mw + rank_w, and the classes are added
// in ascending order, one phase each.  For one input the ranks order its
// windows as their flat output numbers do, so each element's fold is the
// ascending-order sum, and within a phase every input has at most one
// window, so plain LDS read-modify-writes suffice.
template <typename T, typename Src, int NT, bool ORD, int kRound>
__global__ void __launch_bounds__(NT)
bwd_slab_kernel(const typename T::raw *__restrict__ gy, const Src src,
                typename T::raw *__restrict__ gx, BwdPlan p, int64_t tile0)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(R);
    constexpr int AE = 16 / (int)sizeof(Acc);   // accumulator cells per 16 bytes
    extern __shared__ __align__(16) unsigned char smem[];
    Acc *acc = reinterpret_cast<Acc *>(smem);
    const Axis A = p.g.ax[0];
    const int32_t HW = p.g.ax[1].X * p.g.ax[2].X;
    const int32_t OHW = p.g.ax[1].O * p.g.ax[2].O;
    const int32_t tid = threadIdx.x;

    const int64_t t = tile0 + xcd_local_block(blockIdx.x, gridDim.x);
    if (t >= p.ntiles) return;                   // whole workgroup: no barrier skipped
    int64_t plane;
    int32_t td, th, tw;
    p.split.split(t, &plane, &td, &th, &tw);
    const int32_t d0 = td * p.td, d1 = min(d0 + p.td, A.X);
    const int32_t n = (d1 - d0) * HW;
    const int32_t od0 = A.first_reaching(d0);
    const int32_t nw = max(A.last_starting(d1 - 1) + 1 - od0, 0) * OHW;
    const int64_t wbase = plane * (int64_t)p.g.out_plane + (int64_t)od0 * OHW;
    const int32_t ibase = d0 * HW;
    R *dst = gx + plane * (int64_t)p.g.in_plane + ibase;

    // the accumulator is shifted so that a[e] and dst[e] share alignment
    const int32_t mis = (int32_t)(((uintptr_t)dst / sizeof(R)) % VE);
    const int32_t head = min((VE - mis) % VE, n);
    const int32_t shift = (AE - head % AE) % AE;
    Acc *a = acc + shift;

    int32_t ri[kRound];
    R rg[kRound];
    // the first round's windows: their loads are in flight during the zero
    // fill.  A two-phase source's loads are resolved only after it
    // (settle): a branch between the loads of two windows would make each
    // wait for the one before.
    typename pending_of<Src>::type q[kRound];
    auto fetch = [&](int32_t round) {
#pragma unroll
        for (int k = 0; k < kRound; ++k) {
            const int32_t e = (round * kRound + k) * NT + tid;
            if constexpr (two_phase_src<Src>::value) {
                if (e < nw) {
                    q[k] = src.load(wbase + e);
                    rg[k] = gy[wbase + e];
                }
            } else {
                ri[k] = -1;
                if (e < nw) {
                    ri[k] = src(wbase + e);
                    rg[k] = gy[wbase + e];
                }
            }
        }
    };
    auto settle = [&](int32_t round) {
        if constexpr (two_phase_src<Src>::value) {
#pragma unroll
            for (int k = 0; k < kRound; ++k) Src::pin(q[k]);
            uint32_t miss = 0;
#pragma unroll
            for (int k = 0; k < kRound; ++k) {
                const int32_t e = (round * kRound + k) * NT + tid;
                ri[k] = -1;
                if (e < nw) {
                    ri[k] = q[k].idx;
                    if (!Src::settled(q[k])) miss |= 1u << k;
                }
            }
            if (miss) {
#pragma unroll
                for (int k = 0; k < kRound; ++k)
                    if (miss >> k & 1u) ri[k] = src.rescan(wbase + (round * kRound + k) * NT + tid);
            }
        }
    };
    fetch(0);
    for (int32_t e = tid; e < (n + shift + AE - 1) / AE; e += NT)
        reinterpret_cast<u32x4 *>(acc)[e] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    settle(0);
    if constexpr (ORD && !two_phase_src<Src>::value) {
        // keeps the class computation below the barrier: hoisted above it,
        // it makes the wave wait for its loads before the barrier instead of
        // behind it
#pragma unroll
        for (int k = 0; k < kRound; ++k) asm volatile("" : "+v"(ri[k]));
    }
    if constexpr (ORD) {
        const Axis B = p.g.ax[1], Cw = p.g.ax[2];
        const uint32_t W = (uint32_t)Cw.X, OW = (uint32_t)Cw.O;
        // first window reaching x, in 32 bits (the plan admits only axes
        // where that form is exact)
        auto reach = [](const Axis &ax, uint32_t x) -> uint32_t {
            if (ax.k) return (uint32_t)ax.first_reaching((int32_t)x);
            return ax.dX.div(x * (uint32_t)ax.O);
        };
        const int32_t nslot = (nw + NT - 1) / NT;     // slots that hold a window somewhere
        int32_t cls[kRound];
#pragma unroll
        for (int k = 0; k < kRound; ++k) {
            cls[k] = -1;
            if (k >= nslot) continue;
            const uint32_t e = (uint32_t)(k * NT + tid);
            const uint32_t l = (uint32_t)ri[k] - (uint32_t)ibase;
            if (ri[k] >= 0 && l < (uint32_t)n) {
                const uint32_t pos = (uint32_t)ri[k];
                const uint32_t pd = p.hw_div.div(pos), prow = pos - pd * (uint32_t)HW;
                const uint32_t ph = p.w_div.div(prow), pw = prow - ph * W;
                const uint32_t q = p.ohw_div.div(e), orow = e - q * (uint32_t)OHW;
                const uint32_t oh = p.ow_div.div(orow), ow = orow - oh * OW;
                const uint32_t rd = (uint32_t)od0 + q - reach(A, pd);
                const uint32_t rh = oh - reach(B, ph);
                const uint32_t rw = ow - reach(Cw, pw);
                // an idx outside its window gives a rank out of range: dropped
                if (rd < (uint32_t)p.md && rh < (uint32_t)p.mh && rw < (uint32_t)p.mw)
                    cls[k] = (int32_t)((rd * p.mh + rh) * p.mw + rw);
            }
        }
        for (int32_t j = 0; j < p.nphase; ++j) {
#pragma unroll
            for (int k = 0; k < kRound; ++k)
                if (k < nslot && cls[k] == j) a[ri[k] - ibase] += T::widen(rg[k]);
            __syncthreads();
        }
    } else {
        for (int32_t round = 0;; ++round) {
#pragma unroll
            for (int k = 0; k < kRound; ++k) {
                const uint32_t l = (uint32_t)ri[k] - (uint32_t)ibase;
                if (ri[k] >= 0 && l < (uint32_t)n) lds_add(&a[l], T::widen(rg[k]));
            }
            if ((round + 1) * kRound * NT >= nw) break;
            if constexpr (two_phase_src<Src>::value) {
                // later rounds (slabs reached by more windows than one
                // round holds) ask each window in one call
#pragma unroll
                for (int k = 0; k < kRound; ++k) {
                    const int32_t e = ((round + 1) * kRound + k) * NT + tid;
                    ri[k] = -1;
                    if (e < nw) {
                        ri[k] = src(wbase + e);
                        rg[k] = gy[wbase + e];
                    }
                }
            } else {
                fetch(round + 1);
            }
        }
        __syncthreads();
    }
    store_span<T, NT>(dst, a, n, head);
}

// Index-free backward by column stages: a slab [d0, d1) of whole slices of
// one plane.  The argmax of window o is the first tap equal to y[o] (the
// first NaN when y[o] is NaN).  The column forward's two stages give every
// window reaching the slab its first maximum (the first NaN when it holds
// one); where that element equals y[o], every tap equal to y[o] is a
// maximum, so the first of them is that element.  Elsewhere -- y not the
// window's maximum -- the window is scanned in memory.  The LDS
// that held the D-partials then becomes the slab's accumulator, as in the
// slab kernel.
//
// The fallback scan (scan_first_equal, a plain loop) runs only where y is
// not the window's maximum, and adds few registers to those of the common
// path.
template <typename T, int MAXKD, int NT, int KS, int KHW>
__global__ void __launch_bounds__(NT)
bwd_rc_kernel(const typename T::raw *__restrict__ x, const typename T::raw *__restrict__ y,
              const typename T::raw *__restrict__ gy, typename T::raw *__restrict__ gx, RcPlan p,
              uint32_t tile0)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(R);
    constexpr int AE = 16 / (int)sizeof(Acc);
    extern __shared__ __align__(16) unsigned char smem[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t W = Cw.X, HW = B.X * W, OHW = B.O * Cw.O;
    const int32_t tid = threadIdx.x;
    int2 *tab = reinterpret_cast<int2 *>(smem);          // window spans: oh, then ow
    unsigned char *region = smem + p.tab_bytes;          // D-partials, then the accumulator

    const uint32_t t = tile0 + xcd_local_block(blockIdx.x, gridDim.x);
    if (t >= p.ntiles) return;                           // whole workgroup: no barrier skipped
    const uint32_t plane = p.ntd_div.div(t);
    const int32_t sd = (int32_t)(t - plane * (uint32_t)p.ntd);
    const int32_t d0 = sd * p.td, d1 = min(d0 + p.td, A.X);
    const int32_t n = (d1 - d0) * HW;
    const int32_t od0 = A.first_reaching(d0);
    const int32_t cd = max(A.last_starting(d1 - 1) + 1 - od0, 0);
    const int32_t nwin = cd * OHW;                       // <= KS * NT (the plan)
    const int64_t obase = (int64_t)plane * p.g.out_plane + (int64_t)od0 * OHW;
    const R *xp = x + (int64_t)plane * p.g.in_plane;

    // y and gy of the windows, in flight during stage D
    R ry[KS], rg[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int32_t e = k * NT + tid;
        ry[k] = R{};
        rg[k] = R{};
        if (e < nwin) {
            ry[k] = y[obase + e];
            rg[k] = gy[obase + e];
        }
    }
    for (int32_t j = tid; j < B.O + Cw.O; j += NT)
        tab[j] = j < B.O ? make_int2(B.start(j), B.end(j))
                         : make_int2(Cw.start(j - B.O), Cw.end(j - B.O));
    // the partials: packed words for 16-bit storage types, else split
    // arrays of values and d offsets
    constexpr bool PK = sizeof(R) == 2;
    using Part = std::conditional_t<PK, PartPacked<T>, PartSplit<T>>;
    Part part;
    if constexpr (PK) {
        part = Part{reinterpret_cast<uint32_t *>(region)};
    } else {
        part = Part{reinterpret_cast<Acc *>(region),
                    region + (((int64_t)cd * HW * (int64_t)sizeof(Acc) + 15) & ~(int64_t)15)};
    }
    if (cd > 0) col_stage_d<T, MAXKD, NT>(xp, A, HW, od0, cd, part);   // uniform
    __syncthreads();

    int32_t ri[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const int32_t e = k * NT + tid;
        ri[k] = -1;
        if (e < nwin) {
            const uint32_t q = p.ow_div.div((uint32_t)e);
            const int32_t ow = e - (int32_t)q * Cw.O;
            const uint32_t odl = p.oh_div.div(q);
            const int32_t oh = (int32_t)(q - odl * (uint32_t)B.O);
            Acc m;
            uint32_t bk;
            const Part sp = part.at((int32_t)odl * HW);
            if constexpr (KHW > 0)
                bk = col_scan_k<KHW>(sp, W, tab[oh], tab[B.O + ow], m);
            else
                bk = col_scan(sp, W, tab[oh], tab[B.O + ow], m);
            const int32_t bi = (int32_t)(bk & 0xffffffu);
            const Acc best = sp.value(bi);               // NaN exactly when bk names a NaN
            const Acc want = T::widen(ry[k]);
            const bool same = want != want ? best != best : best == want;
            ri[k] = same ? (A.start(od0 + (int32_t)odl) + (int32_t)(bk >> 24)) * HW + bi
                         : scan_first_equal<T>(xp, p.g, od0 + (int32_t)odl, oh, ow, want);
        }
    }
    __syncthreads();                                     // the D-partials are consumed

    R *dst = gx + (int64_t)plane * p.g.in_plane + (int64_t)d0 * HW;
    // the accumulator is shifted so that a[e] and dst[e] share alignment
    const int32_t mis = (int32_t)(((uintptr_t)dst / sizeof(R)) % VE);
    const int32_t head = min((VE - mis) % VE, n);
    const int32_t shift = (AE - head % AE) % AE;
    Acc *a = reinterpret_cast<Acc *>(region) + shift;
    for (int32_t e = tid; e < (n + shift + AE - 1) / AE; e += NT)
        reinterpret_cast<u32x4 *>(region)[e] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    const uint32_t ibase = (uint32_t)d0 * (uint32_t)HW;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const uint32_t l = (uint32_t)ri[k] - ibase;
        if (ri[k] >= 0 && l < (uint32_t)n) lds_add(&a[l], T::widen(rg[k]));
    }
    __syncthreads();
    store_span<T, NT>(dst, a, n, head);
}

// General boxes [d0,d1) x [h0,h1) x [w0,w1) (a slice does not fit in LDS).
template <typename T, typename Src>
__global__ void __launch_bounds__(kBlock)
bwd_box_kernel(const typename T::raw *__restrict__ gy, const Src src,
               typename T::raw *__restrict__ gx, BwdPlan p)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    extern __shared__ __align__(16) unsigned char smem[];
    Acc *acc = reinterpret_cast<Acc *>(smem);
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X;
    const int32_t tid = threadIdx.x;
    for (int64_t t = blockIdx.x; t < p.ntiles; t += gridDim.x) {
        int64_t plane;
        int32_t td, th, tw;
        p.split.split(t, &plane, &td, &th, &tw);
        const int32_t d0 = td * p.td, d1 = min(d0 + p.td, A.X);
        const int32_t h0 = th * p.th, h1 = min(h0 + p.th, H);
        const int32_t w0 = tw * p.tw, w1 = min(w0 + p.tw, W);
        const int32_t lh = h1 - h0, lw = w1 - w0, n = (d1 - d0) * lh * lw;
        const int32_t od0 = A.first_reaching(d0), oh0 = B.first_reaching(h0);
        const int32_t ow0 = Cw.first_reaching(w0);
        const int32_t cd = max(A.last_starting(d1 - 1) + 1 - od0, 0);
        const int32_t ch = max(B.last_starting(h1 - 1) + 1 - oh0, 0);
        const int32_t cw = max(Cw.last_starting(w1 - 1) + 1 - ow0, 0);
        const int64_t obase = plane * (int64_t)p.g.out_plane;

        for (int32_t e = tid; e < n; e += kBlock) acc[e] = Acc(0);
        __syncthreads();
        for (int32_t e = tid; e < cd * ch * cw; e += kBlock) {
            const int32_t owl = e % cw, r = e / cw, ohl = r % ch, odl = r / ch;
            const int64_t o = obase + ((od0 + odl) * B.O + oh0 + ohl) * Cw.O + ow0 + owl;
            const int32_t i = src(o);
            if ((uint32_t)i < (uint32_t)p.g.in_plane) {
                const int32_t d = i / (H * W), rem = i - d * H * W;
                const int32_t h = rem / W, w = rem - h * W;
                if (d >= d0 && d < d1 && h >= h0 && h < h1 && w >= w0 && w < w1)
                    lds_add(&acc[((d - d0) * lh + (h - h0)) * lw + (w - w0)], T::widen(gy[o]));
            }
        }
        __syncthreads();
        R *gp = gx + plane * (int64_t)p.g.in_plane;
        for (int32_t e = tid; e < n; e += kBlock) {
            const int32_t w = e % lw, r = e / lw, h = r % lh, d = r / lh;
            gp[((d0 + d) * H + h0 + h) * W + w0 + w] = T::narrow(acc[e]);
        }
        __syncthreads();   // LDS is reused by the next tile
    }
}

// Windows tile every axis (q = X / O per axis): input (d, h, w) lies in the
// one window (d / qd, h / qh, w / qw), and window o covers the qd x qh x qw
// box at (od*qd, oh*qh, ow*qw).  A thread takes kGatherV consecutive windows
// of one output row: it loads their idx and gy (16-byte and 8-byte vectors
// where aligned), then writes each of the qd*qh input rows under them -- the
// qw*kGatherV elements of a row are contiguous, gy where idx names the
// element and +0 elsewhere -- with 16-byte streaming stores where the row
// segment is aligned, else element stores.
constexpr int kGatherV = 4;

// QW: qw as a compile-time constant (1 or 2), 0 for any qw.
template <typename T, typename Src, int QW>
__global__ void __launch_bounds__(kBlock)
bwd_gather_kernel(const typename T::raw *__restrict__ gy, const Src src,
                  typename T::raw *__restrict__ gx, GatherPlan p)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int V = kGatherV;
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
    const int32_t OD = p.g.ax[0].O, OH = p.g.ax[1].O, OW = p.g.ax[2].O;
    const int32_t G = (OW + V - 1) / V;                 // window groups per output row
    const int64_t total = p.g.planes * (int64_t)OD * OH * G;
    for (int64_t t = (int64_t)blockIdx.x * kBlock + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * kBlock) {
        int64_t row;                                   // output row: plane * OD * OH + od * OH + oh
        int32_t grp;
        if (p.fast) {
            const uint32_t q = p.grp_div.div((uint32_t)t);
            row = q;
            grp = (int32_t)((uint32_t)t - q * (uint32_t)G);
        } else {
            row = t / G;
            grp = (int32_t)(t - row * G);
        }
        int64_t plane;
        int32_t od, oh;
        if (p.fast) {
            const uint32_t q = p.oh_div.div((uint32_t)row);
            oh = (int32_t)((uint32_t)row - q * (uint32_t)OH);
            const uint32_t q2 = p.od_div.div(q);
            od = (int32_t)(q - q2 * (uint32_t)OD);
            plane = q2;
        } else {
            const int64_t q = row / OH;
            oh = (int32_t)(row - q * OH);
            plane = q / OD;
            od = (int32_t)(q - plane * OD);
        }
        const int32_t ow0 = grp * V, nwin = min(V, OW - ow0);
        const int64_t o0 = plane * (int64_t)p.g.out_plane + ((int64_t)od * OH + oh) * OW + ow0;
        int32_t ix[V];
        Acc gv[V];
        if (nwin == V && p.vec_in && (o0 & (V - 1)) == 0) {
            src.load4(o0, ix);
            if constexpr (sizeof(R) == 2) {
                const u32x2 g2 = *reinterpret_cast<const u32x2 *>(gy + o0);
                const uint32_t gw[2] = {g2.x, g2.y};
#pragma unroll
                for (int k = 0; k < V; ++k) gv[k] = T::widen((R)(gw[k / 2] >> (16 * (k % 2))));
            } else {
#pragma unroll
                for (int k = 0; k < V; ++k) gv[k] = T::widen(gy[o0 + k]);
            }
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                ix[k] = -1;
                gv[k] = Acc(0);
                if (k < nwin) {
                    ix[k] = src(o0 + k);
                    gv[k] = T::widen(gy[o0 + k]);
                }
            }
        }
        // 0 + gy: a -0 gradient gives +0, as the accumulate path does
        R val[V];
#pragma unroll
        for (int k = 0; k < V; ++k) val[k] = T::narrow(Acc(0) + gv[k]);
        const R zero = T::narrow(Acc(0));
        const int32_t qw = QW ? QW : p.qw;
        const int32_t w0 = ow0 * qw;                    // the row segment under the windows
        R *gp = gx + plane * (int64_t)p.g.in_plane;
        for (int32_t dd = 0; dd < p.qd; ++dd) {
            for (int32_t hh = 0; hh < p.qh; ++hh) {
                const int32_t pos0 = ((od * p.qd + dd) * H + oh * p.qh + hh) * W + w0;
                R *seg = gp + pos0;
                if constexpr (QW > 0 && (QW * V * sizeof(R)) % 16 == 0) {
                    if (nwin == V && ((uintptr_t)seg & 15) == 0) {
                        // QW * V elements, whole 16-byte vectors; element q
                        // lies in window q / QW
                        constexpr int NE = QW * V, VE = 16 / (int)sizeof(R);
                        R e[NE];
#pragma unroll
                        for (int q = 0; q < NE; ++q) e[q] = ix[q / QW] == pos0 + q ? val[q / QW] : zero;
#pragma unroll
                        for (int c = 0; c < NE; c += VE) {
                            uint32_t w4[4];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                if constexpr (sizeof(R) == 2)
                                    w4[j] = (uint32_t)e[c + 2 * j] | ((uint32_t)e[c + 2 * j + 1] << 16);
                                else if constexpr (sizeof(R) == 4)
                                    w4[j] = __builtin_bit_cast(uint32_t, e[c + j]);
                                else
                                    w4[j] = (uint32_t)(__builtin_bit_cast(uint64_t, e[c + j / 2]) >> (32 * (j % 2)));
                            }
                            st_stream(reinterpret_cast<u32x4 *>(seg + c), u32x4{w4[0], w4[1], w4[2], w4[3]});
                        }
                        continue;
                    }
                }
                // element stores: any qw, any alignment, a short last group
                for (int32_t k = 0; k < nwin; ++k) {
                    int32_t ik = ix[0];
                    R vk = val[0];
#pragma unroll
                    for (int kk = 1; kk < V; ++kk) {
                        ik = kk == k ? ix[kk] : ik;
                        vk = kk == k ? val[kk] : vk;
                    }
                    for (int32_t ww = 0; ww < qw; ++ww) {
                        const int32_t q = k * qw + ww;
                        seg[q] = ik == pos0 + q ? vk : zero;
                    }
                }
            }
        }
    }
}

// The gather again, by 16-byte chunk columns: when rows are whole chunks
// (W * element size a multiple of 16, gx on 16 bytes) and a chunk holds
// whole windows along w (QW divides the chunk's VE elements), thread u is
// chunk c of a slice (elements [c*VE, c*VE + VE) of the H*W slice, c < nc =
// H*W / VE) under output slice od of one plane.  It reads the idx and gy of
// the NW = VE / QW windows above that chunk once and stores the chunk in
// each of the qd input slices od*qd .. od*qd + qd - 1.  The lanes of a wave
// store consecutive chunks of one slice, so every store instruction covers
// whole cache lines of gx (the window-group kernel above writes rows qd*qh
// apart per instruction, and its streaming stores then leave partial
// lines); a window's idx and gy are read by the qh rows of chunks under
// it, which sit in the same or the next wave.
template <typename T, typename Src, int QW>
__global__ void __launch_bounds__(kBlock)
bwd_gather_chunk_kernel(const typename T::raw *__restrict__ gy, const Src src,
                        typename T::raw *__restrict__ gx, GatherPlan p)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(R);
    constexpr int NW = VE / QW;
    static_assert(NW * QW == VE, "whole windows per chunk");
    const int32_t W = p.g.ax[2].X, HW = p.g.ax[1].X * W;
    const int32_t OD = p.g.ax[0].O, OH = p.g.ax[1].O, OW = p.g.ax[2].O;
    const int32_t nc = p.nc;
    const int64_t total = p.g.planes * (int64_t)OD * nc;
    const R zero = T::narrow(Acc(0));
    for (int64_t u = (int64_t)blockIdx.x * kBlock + threadIdx.x; u < total;
         u += (int64_t)gridDim.x * kBlock) {
        int64_t op, plane;                                 // op = plane * OD + od
        if (p.fast_col) {
            op = p.nc_div.div((uint32_t)u);
            plane = p.od_div.div((uint32_t)op);
        } else {
            op = u / nc;
            plane = op / OD;
        }
        const int32_t c = (int32_t)(u - op * nc);
        const int32_t od = (int32_t)(op - plane * OD);
        const int32_t e = c * VE;                          // element in the slice
        const int32_t h = (int32_t)p.w_div.div((uint32_t)e);
        const int32_t w0 = e - h * W;
        const int32_t oh = (int32_t)p.qh_div.div((uint32_t)h);
        const int64_t o0 = plane * (int64_t)p.g.out_plane + ((int64_t)od * OH + oh) * OW + w0 / QW;
        int32_t ix[NW];
        R gr[NW];
        if constexpr (NW == 4) {
            if (p.vec_in && (o0 & 3) == 0) {
                // four windows: idx as one 16-byte vector (two for int64),
                // gy as one 8- or 16-byte vector
                src.load4(o0, ix);
                if constexpr (sizeof(R) == 2) {
                    const u32x2 g2 = *reinterpret_cast<const u32x2 *>(gy + o0);
                    gr[0] = (R)g2.x; gr[1] = (R)(g2.x >> 16); gr[2] = (R)g2.y; gr[3] = (R)(g2.y >> 16);
                } else {
#pragma unroll
                    for (int k = 0; k < NW; ++k) gr[k] = gy[o0 + k];
                }
            } else {
#pragma unroll
                for (int k = 0; k < NW; ++k) {
                    ix[k] = src(o0 + k);
                    gr[k] = gy[o0 + k];
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < NW; ++k) {
                ix[k] = src(o0 + k);
                gr[k] = gy[o0 + k];
            }
        }
        // 0 + gy: a -0 gradient gives +0, as the accumulate path does
        R g0[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) g0[k] = T::narrow(Acc(0) + T::widen(gr[k]));
        const int32_t d0 = od * p.qd;
        R *col = gx + plane * (int64_t)p.g.in_plane + (int64_t)d0 * HW + e;
        for (int32_t dd = 0; dd < p.qd; ++dd) {
            const int32_t pos0 = (d0 + dd) * HW + e;       // plane position of the chunk
            uint32_t w4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(R) == 2) {
                    const int q = 2 * j;
                    const R lo = ix[q / QW] == pos0 + q ? g0[q / QW] : zero;
                    const R hi = ix[(q + 1) / QW] == pos0 + q + 1 ? g0[(q + 1) / QW] : zero;
                    w4[j] = (uint32_t)lo | ((uint32_t)hi << 16);
                } else if constexpr (sizeof(R) == 4) {
                    w4[j] = __builtin_bit_cast(uint32_t, ix[j / QW] == pos0 + j ? g0[j / QW] : zero);
                } else {
                    const int q = j / 2;
                    const R v = ix[q / QW] == pos0 + q ? g0[q / QW] : zero;
                    w4[j] = (uint32_t)(__builtin_bit_cast(uint64_t, v) >> (32 * (j % 2)));
                }
            }
            st_stream(reinterpret_cast<u32x4 *>(col + (int64_t)dd * HW),
                      u32x4{w4[0], w4[1], w4[2], w4[3]});
        }
    }
}

}  // namespace

template <typename T, typename Src>
hipError_t launch_backward_tile(const void *gy, const Src &src, void *gx, const BwdPlan &p,
                                hipStream_t s)
{
    using R = typename T::raw;
    if (!p.slab) {
        // boxes are strided over the workgroups
        const int64_t grid = std::min<int64_t>(p.ntiles, kMaxTileGrid);
        launch_kernel((bwd_box_kernel<T, Src>), dim3((uint32_t)grid), dim3(kBlock), p.lds_bytes, s,
                      (const R *)gy, src, (R *)gx, p);
        return hipGetLastError();
    }
    // one workgroup per slab, in launches of at most kMaxTileGrid workgroups
    // (so workgroups x threads stay within one dispatch); a multiple of 8
    // lets blocks map per XCD (the surplus blocks exit at once)
    for (int64_t t0 = 0; t0 < p.ntiles; t0 += kMaxTileGrid) {
        const uint32_t grid = tile_grid(p.ntiles, t0);
        if (p.nphase)
            launch_kernel((bwd_slab_kernel<T, Src, kOrdThreads, true, kOrdRound>),
                          dim3((uint32_t)grid), dim3(kOrdThreads), p.lds_bytes, s, (const R *)gy,
                          src, (R *)gx, p, t0);
        else
            launch_kernel((bwd_slab_kernel<T, Src, kSlabBlock, false, Src::kSlots>),
                          dim3((uint32_t)grid), dim3(kSlabBlock), p.lds_bytes, s, (const R *)gy,
                          src, (R *)gx, p, t0);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <typename T>
hipError_t launch_backward_rc(const void *x, const void *y, const void *gy, void *gx,
                              const RcPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    // one workgroup per slab, in launches of at most kMaxTileGrid workgroups;
    // a multiple of 8 lets blocks map per XCD (the surplus exits)
    auto go = [&](auto kern) {
        for (int64_t t0 = 0; t0 < (int64_t)p.ntiles; t0 += kMaxTileGrid) {
            const uint32_t grid = tile_grid(p.ntiles, t0);
            launch_kernel(kern, dim3((uint32_t)grid), dim3(kBlock), p.lds_bytes, s, (const R *)x,
                          (const R *)y, (const R *)gy, (R *)gx, p, (uint32_t)t0);
        }
    };
    // window slots per thread: the fewest of 1, 2, 4, 8, 16 that hold the
    // windows reaching a slab
    auto slots = [&](auto k1, auto k2, auto k4, auto k8, auto k16) {
        if (p.slots <= 1) go(k1);
        else if (p.slots <= 2) go(k2);
        else if (p.slots <= 4) go(k4);
        else if (p.slots <= 8) go(k8);
        else go(k16);
    };
    // windows of at most 3 taps per axis: exact 3-slice loads and a
    // 3 x 3 scan with every load issued at once; else loops
    if (p.small3)
        slots(bwd_rc_kernel<T, 3, kBlock, 1, 3>, bwd_rc_kernel<T, 3, kBlock, 2, 3>,
              bwd_rc_kernel<T, 3, kBlock, 4, 3>, bwd_rc_kernel<T, 3, kBlock, 8, 3>,
              bwd_rc_kernel<T, 3, kBlock, 16, 3>);
    else if (p.maxkd <= 4)
        slots(bwd_rc_kernel<T, 4, kBlock, 1, 0>, bwd_rc_kernel<T, 4, kBlock, 2, 0>,
              bwd_rc_kernel<T, 4, kBlock, 4, 0>, bwd_rc_kernel<T, 4, kBlock, 8, 0>,
              bwd_rc_kernel<T, 4, kBlock, 16, 0>);
    else
        slots(bwd_rc_kernel<T, 8, kBlock, 1, 0>, bwd_rc_kernel<T, 8, kBlock, 2, 0>,
              bwd_rc_kernel<T, 8, kBlock, 4, 0>, bwd_rc_kernel<T, 8, kBlock, 8, 0>,
              bwd_rc_kernel<T, 8, kBlock, 16, 0>);
    return hipGetLastError();
}

template <typename T, typename Src>
hipError_t launch_backward_gather(const void *gy, const Src &src, void *gx, const GatherPlan &p,
                                  hipStream_t s)
{
    using R = typename T::raw;
    constexpr int VE = 16 / (int)sizeof(R);
    // one chunk per thread where rows are whole chunks and windows fit
    // chunks (qw 1 or 2; qw 2 and 8-byte elements: a chunk is one window)
    const bool rows16 = ((int64_t)p.g.ax[2].X * (int64_t)sizeof(R)) % 16 == 0 &&
                        (uintptr_t)gx % 16 == 0;
    if (rows16 && (p.qw == 1 || (p.qw == 2 && VE % 2 == 0))) {
        // one thread per chunk column: planes * OD * (H*W / VE) threads
        GatherPlan q = p;
        q.nc = p.g.ax[1].X * p.g.ax[2].X / VE;
        q.nc_div = FastDiv((uint32_t)q.nc);
        const int64_t cols = p.g.planes * (int64_t)p.g.ax[0].O * q.nc;
        q.fast_col = cols < ((int64_t)1 << 31);
        int64_t grid = std::min<int64_t>((cols + kBlock - 1) / kBlock, kMaxTileGrid);
        if (grid >= 64) grid = (grid + 7) & ~(int64_t)7;
        q.vec_in = src.aligned4() && (uintptr_t)gy % 16 == 0;
        if (p.qw == 1)
            launch_kernel((bwd_gather_chunk_kernel<T, Src, 1>), dim3((uint32_t)grid), dim3(kBlock),
                          0, s, (const R *)gy, src, (R *)gx, q);
        else
            launch_kernel((bwd_gather_chunk_kernel<T, Src, 2>), dim3((uint32_t)grid), dim3(kBlock),
                          0, s, (const R *)gy, src, (R *)gx, q);
        return hipGetLastError();
    }
    GatherPlan q = p;
    q.vec_in = src.aligned4() && (sizeof(R) != 2 || (uintptr_t)gy % 8 == 0);
    if (q.qw == 1)
        launch_kernel((bwd_gather_kernel<T, Src, 1>), dim3(q.grid), dim3(kBlock), 0, s,
                      (const R *)gy, src, (R *)gx, q);
    else if (q.qw == 2)
        launch_kernel((bwd_gather_kernel<T, Src, 2>), dim3(q.grid), dim3(kBlock), 0, s,
                      (const R *)gy, src, (R *)gx, q);
    else
        launch_kernel((bwd_gather_kernel<T, Src, 0>), dim3(q.grid), dim3(kBlock), 0, s,
                      (const R *)gy, src, (R *)gx, q);
    return hipGetLastError();
}

template hipError_t launch_backward_tile<F32, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F32, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F32, IdxRecompute<F32>>(const void *, const IdxRecompute<F32> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F32, IdxChecked<F32>>(const void *, const IdxChecked<F32> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F16, IdxRecompute<F16>>(const void *, const IdxRecompute<F16> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F16, IdxChecked<F16>>(const void *, const IdxChecked<F16> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<BF16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<BF16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<BF16, IdxRecompute<BF16>>(const void *, const IdxRecompute<BF16> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<BF16, IdxChecked<BF16>>(const void *, const IdxChecked<BF16> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F64, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F64, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F64, IdxRecompute<F64>>(const void *, const IdxRecompute<F64> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_tile<F64, IdxChecked<F64>>(const void *, const IdxChecked<F64> &, void *, const BwdPlan &, hipStream_t);
template hipError_t launch_backward_rc<F32>(const void *, const void *, const void *, void *, const RcPlan &, hipStream_t);
template hipError_t launch_backward_rc<F16>(const void *, const void *, const void *, void *, const RcPlan &, hipStream_t);
template hipError_t launch_backward_rc<BF16>(const void *, const void *, const void *, void *, const RcPlan &, hipStream_t);
template hipError_t launch_backward_rc<F64>(const void *, const void *, const void *, void *, const RcPlan &, hipStream_t);
template hipError_t launch_backward_gather<F32, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F32, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<BF16, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<BF16, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F64, IdxArray<int32_t>>(const void *, const IdxArray<int32_t> &, void *, const GatherPlan &, hipStream_t);
template hipError_t launch_backward_gather<F64, IdxArray<int64_t>>(const void *, const IdxArray<int64_t> &, void *, const GatherPlan &, hipStream_t);

}  // namespace mp3d
