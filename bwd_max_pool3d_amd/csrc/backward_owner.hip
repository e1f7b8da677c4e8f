// backward_owner.hip -- the overlapping-window backward as an owner gather:
// each element's contributions are summed by one window, out of LDS, with
// no atomics.
//
// Definition (PR #308 page, "Add adaptive_max_pool3d_backward Moore
// Threads specialized operator", Summary): gx[p] is the sum of gy[o] over
// the outputs o whose argmax idx[o] is p, and 0 where none is.  The page's
// non-divisible scheme zero-fills gx, scatters gy with atomic adds and
// casts in a last pass.  Here a workgroup owns a slab [d0, d1) of whole
// slices of one plane's gx, staged in LDS in the storage type, and
//  1. zero-fills the staged slab and copies the (idx, gy) of every window
//     that can reach it (one contiguous run of each) into an LDS table;
//  2. gives every window a thread: among the windows containing its argmax
//     p, enumerated in ascending output order, the first whose idx is p --
//     the owner of p -- adds the gy of every window whose idx is p, from +0
//     in the accumulation type, and writes the sum, rounded once, to the
//     staged element.  Every element has at most one writer, and its value
//     is the ascending-order fold: the same bit for bit on every run, and
//     the ordered definition itself;
//  3. writes the staged slab out with 16-byte streaming stores.
// The staged slab takes the storage type's bytes in LDS, not a binary32
// accumulator per element (half as much for 16-bit types), so more of gx
// is in flight on each CU.  Fixed or adaptive axes, padding, dilation (a
// position in a window's span that is not one of its taps never equals a
// valid idx) and ceil-mode extents all take this path.
#include <algorithm>

#include "dtype.hpp"
#include "idxsrc.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// D2: every position lies in at most two windows per axis.
template <typename T, typename Src, int NT, bool D2>
__global__ void __launch_bounds__(NT)
bwd_owner_kernel(const typename T::raw *__restrict__ gy, const Src src,
                 typename T::raw *__restrict__ gx, OwnerPlan p, int64_t tile0)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(R);          // elements per 16-byte vector
    constexpr int S = NT == 256 ? 2 * kOwnerSlots : kOwnerSlots;   // windows per thread per round
    extern __shared__ __align__(16) unsigned char smem[];
    R *stage = reinterpret_cast<R *>(smem);
    int32_t *tix = reinterpret_cast<int32_t *>(smem + p.st_bytes);
    R *tgy = reinterpret_cast<R *>(smem + p.st_bytes + p.ti_bytes);
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t W = Cw.X, HW = B.X * W, OW = Cw.O, OHW = B.O * OW;
    const int32_t tid = threadIdx.x;

    const int64_t t = tile0 + xcd_local_block(blockIdx.x, gridDim.x);
    if (t >= p.ntiles) return;                           // whole workgroup: no barrier skipped
    int64_t plane;
    int32_t sd;
    if (p.fast) {
        const uint32_t q = p.ntd_div.div((uint32_t)t);
        plane = q;
        sd = (int32_t)((uint32_t)t - q * (uint32_t)p.ntd);
    } else {
        plane = t / p.ntd;
        sd = (int32_t)(t - plane * p.ntd);
    }
    const int32_t d0 = sd * p.td, d1 = min(d0 + p.td, A.X);
    const int32_t n = (d1 - d0) * HW;                 // elements of the slab
    const int32_t ibase = d0 * HW;                    // plane position of its first
    const int32_t od0 = A.first_reaching(d0);
    const int32_t nw = max(A.last_starting(d1 - 1) + 1 - od0, 0) * OHW;
    const int64_t wbase = plane * (int64_t)p.g.out_plane + (int64_t)od0 * OHW;
    R *dst = gx + plane * (int64_t)p.g.in_plane + ibase;
    // stage[e + mis] is dst[e]: stage and dst share their alignment
    // within a 16-byte vector
    const int32_t mis = (int32_t)(((uintptr_t)dst / sizeof(R)) % VE);
    R *st = stage + mis;

    // 1. the windows' (idx, gy): the first round in flight during the
    // zero fill.  Slots past the run load its last window again (no
    // branch between the loads) and are dropped.
    int32_t ri[S];
    R rg[S];
    auto fetch = [&](int32_t base) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int32_t e = min(base + k * NT + tid, nw - 1);
            ri[k] = src(wbase + e);
            rg[k] = gy[wbase + e];
        }
    };
    if (nw > 0) fetch(0);                             // uniform
    for (int32_t i = tid; i < (n + mis + VE - 1) / VE; i += NT)
        reinterpret_cast<u32x4 *>(stage)[i] = u32x4{0u, 0u, 0u, 0u};
    for (int32_t base = 0; base < nw;) {
#pragma unroll
        for (int k = 0; k < S; ++k) {
            const int32_t e = base + k * NT + tid;
            if (e < nw) {
                tix[e] = ri[k];
                tgy[e] = rg[k];
            }
        }
        base += S * NT;
        if (base < nw) fetch(base);
    }
    __syncthreads();

    // 2. one window per thread at a time: the owner of its argmax sums
    for (int32_t e = tid; e < nw; e += NT) {
        const int32_t pos = tix[e];
        const uint32_t l = (uint32_t)(pos - ibase);
        if (pos < 0 || l >= (uint32_t)n) continue;
        const uint32_t pd = p.hw_div.div((uint32_t)pos);
        const uint32_t rem = (uint32_t)pos - pd * (uint32_t)HW;
        const uint32_t ph = p.w_div.div(rem);
        const int32_t pw = (int32_t)(rem - ph * (uint32_t)W);
        const int32_t a0 = A.first_reaching((int32_t)pd), a1 = A.last_starting((int32_t)pd);
        const int32_t h0 = B.first_reaching((int32_t)ph), h1 = B.last_starting((int32_t)ph);
        const int32_t w0 = Cw.first_reaching(pw), w1 = Cw.last_starting(pw);
        // the windows containing pos, in ascending output order (= table order)
        Acc s = Acc(0);
        bool owner = true;
        if constexpr (D2) {
            // at most two windows per axis: all eight candidates at once,
            // their table reads issued together; an absent candidate
            // reads the window itself and is masked off
            int32_t ti[8];
            bool ok[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int32_t od = a0 + (c >> 2), oh = h0 + ((c >> 1) & 1), ow = w0 + (c & 1);
                ok[c] = od <= a1 && oh <= h1 && ow <= w1;
                ti[c] = ok[c] ? (od - od0) * OHW + oh * OW + ow : e;
            }
            int32_t cx[8];
            R cg[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                cx[c] = tix[ti[c]];
                cg[c] = tgy[ti[c]];
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const bool m = ok[c] && cx[c] == pos;
                owner = owner && !(m && ti[c] < e);
                const Acc t = s + T::widen(cg[c]);
                s = m ? t : s;
            }
        } else {
            for (int32_t od = a0; od <= a1 && owner; ++od)
                for (int32_t oh = h0; oh <= h1 && owner; ++oh) {
                    const int32_t row = (od - od0) * OHW + oh * OW;
                    for (int32_t ow = w0; ow <= w1; ++ow) {
                        const int32_t ti = row + ow;
                        if (tix[ti] == pos) {
                            if (ti < e) { owner = false; break; }
                            s += T::widen(tgy[ti]);
                        }
                    }
                }
        }
        if (owner) st[l] = T::narrow(s);
    }
    __syncthreads();

    // 3. the staged slab out: 16-byte streaming stores for the aligned
    // body, element stores for the head and tail
    const int32_t head = min((VE - mis) % VE, n);
    const int32_t nvec = (n - head) / VE, tail0 = head + nvec * VE;
    if (tid < head) dst[tid] = st[tid];
    const u32x4 *sv = reinterpret_cast<const u32x4 *>(st + head);
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    int32_t i = tid;
    for (; i + 3 * NT < nvec; i += 4 * NT) {
        const u32x4 v0 = sv[i], v1 = sv[i + NT], v2 = sv[i + 2 * NT], v3 = sv[i + 3 * NT];
        st_stream(dv + i, v0);
        st_stream(dv + i + NT, v1);
        st_stream(dv + i + 2 * NT, v2);
        st_stream(dv + i + 3 * NT, v3);
    }
    for (; i < nvec; i += NT) st_stream(dv + i, sv[i]);
    if (tid < n - tail0) dst[tail0 + tid] = st[tail0 + tid];
}

}  // namespace

template <typename T, typename Src>
hipError_t launch_backward_owner(const void *gy, const Src &src, void *gx, const OwnerPlan &p,
                                 hipStream_t s)
{
    using R = typename T::raw;
    // one workgroup per slab, in launches of at most kMaxTileGrid workgroups;
    // a multiple of 8 lets blocks map per XCD (the surplus exits)
    auto go = [&](auto kern, int nt) {
        for (int64_t t0 = 0; t0 < p.ntiles; t0 += kMaxTileGrid) {
            const uint32_t grid = tile_grid(p.ntiles, t0);
            launch_kernel(kern, dim3((uint32_t)grid), dim3(nt), p.lds_bytes, s, (const R *)gy,
                          src, (R *)gx, p, t0);
        }
    };
    if (p.depth2) {
        if (p.threads == 256) go(bwd_owner_kernel<T, Src, 256, true>, 256);
        else go(bwd_owner_kernel<T, Src, 512, true>, 512);
    } else {
        if (p.threads == 256) go(bwd_owner_kernel<T, Src, 256, false>, 256);
        else go(bwd_owner_kernel<T, Src, 512, false>, 512);
    }
    return hipGetLastError();
}

#define MP3D_OWNER(T, S)                                                                           \
    template hipError_t launch_backward_owner<T, S>(const void *, const S &, void *,              \
                                                    const OwnerPlan &, hipStream_t);
MP3D_OWNER(F32, IdxArray<int32_t>)
MP3D_OWNER(F32, IdxArray<int64_t>)
MP3D_OWNER(F16, IdxArray<int32_t>)
MP3D_OWNER(F16, IdxArray<int64_t>)
MP3D_OWNER(BF16, IdxArray<int32_t>)
MP3D_OWNER(BF16, IdxArray<int64_t>)
MP3D_OWNER(F64, IdxArray<int32_t>)
MP3D_OWNER(F64, IdxArray<int64_t>)
#undef MP3D_OWNER

}  // namespace mp3d
