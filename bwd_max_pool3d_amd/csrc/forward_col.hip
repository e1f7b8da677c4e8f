// forward_col.hip -- forward for any window rule (fixed or adaptive) when
// whole H*W slices can be read as 16-byte vectors, the windows along D are
// at most 8 wide, and a tile's D-partials fit in LDS.
//
// Same definition as the other forward kernels ("Struct Maxpool3dForward",
// teenygrad, description; PR #308 page, Summary): per window, the first
// maximum in d, h, w scan order, NaN ranking above every number.
//
// A workgroup owns one plane and a run of output slices od, and computes
// every window's first maximum with the two stages of colstage.hpp: the
// D-reduce in registers from coalesced 16-byte column loads, then one scan
// per window over the D-partials in LDS.  NT threads: 256, or 512 when the
// tile's D-partials need much LDS and few workgroups fit on a CU.
#include <algorithm>

#include "colstage.hpp"
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// KHW > 0: every window has at most KHW taps along h and along w.
template <typename T, typename IT, int MAXKD, int NT, int KHW>
__global__ void __launch_bounds__(NT)
fwd_col_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
               IT *__restrict__ idx, ColPlan p, uint32_t tile0)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    extern __shared__ __align__(16) unsigned char smem[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X, HW = H * W;
    const int32_t tid = threadIdx.x;

    // LDS: window table (oh then ow) | D-partial values | D-partial d offsets
    int2 *tab = reinterpret_cast<int2 *>(smem);
    Acc *pv = reinterpret_cast<Acc *>(smem + p.tab_bytes);
    uint8_t *pd = reinterpret_cast<uint8_t *>(smem + p.tab_bytes + p.pv_bytes);

    const uint32_t t = tile0 + xcd_local_block(blockIdx.x, gridDim.x);
    if (t >= p.ntiles) return;                 // whole workgroup: no barrier skipped
    const uint32_t plane = p.ntd_div.div(t);
    const int32_t td = (int32_t)(t - plane * (uint32_t)p.ntd);
    const int32_t od0 = td * p.tod, od1 = min(od0 + p.tod, A.O);
    const int32_t cd = od1 - od0;
    const R *xp = x + (int64_t)plane * p.g.in_plane;

    for (int32_t j = tid; j < B.O + Cw.O; j += NT)
        tab[j] = j < B.O ? make_int2(B.start(j), B.end(j))
                         : make_int2(Cw.start(j - B.O), Cw.end(j - B.O));

    col_stage_d<T, MAXKD, NT>(xp, A, HW, od0, cd, PartSplit<T>{pv, pd});
    __syncthreads();

    // stage HW
    const int32_t per_slice = B.O * Cw.O;
    const int32_t nout = cd * per_slice;
    const int64_t obase = (int64_t)plane * p.g.out_plane + (int64_t)od0 * per_slice;
    for (int32_t e = tid; e < nout; e += NT) {
        const uint32_t q = p.ow_div.div((uint32_t)e);
        const int32_t ow = e - (int32_t)q * Cw.O;
        const uint32_t odl = p.oh_div.div(q);
        const int32_t oh = (int32_t)(q - odl * (uint32_t)B.O);
        const Acc *sv = pv + odl * HW;
        Acc m;
        const PartSplit<T> sp{pv + odl * HW, pd + odl * HW};
        uint32_t bk;
        if constexpr (KHW > 0)
            bk = col_scan_max<KHW>(sp, W, tab[oh], tab[B.O + ow], m);
        else
            bk = col_scan(sp, W, tab[oh], tab[B.O + ow], m);
        const int32_t bi = (int32_t)(bk & 0xffffffu);
        const int32_t pos = (A.start(od0 + (int32_t)odl) + (int32_t)(bk >> 24)) * HW + bi;
        const Acc best = sv[bi];          // the element itself: keeps the sign of a zero
        R raw;
        if (T::exact_nan || best == best)
            raw = T::back(best);
        else
            raw = xp[pos];                // NaN: copy the element's own bits
        st_stream(y + obase + e, raw);
        if (idx) st_stream(idx + obase + e, (IT)pos);
    }
}

template <typename T, typename IT, int MAXKD>
hipError_t launch_col(const void *x, void *y, IT *idx, const ColPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    // one workgroup per tile, in launches of at most kMaxTileGrid workgroups;
    // a multiple of 8 lets blocks map per XCD (the surplus exits)
    for (int64_t t0 = 0; t0 < (int64_t)p.ntiles; t0 += kMaxTileGrid) {
        const uint32_t grid = tile_grid(p.ntiles, t0);
        auto go = [&](auto kern, int nt) {
            launch_kernel(kern, dim3(grid), dim3(nt), p.lds_bytes, s, (const R *)x, (R *)y, idx, p,
                          (uint32_t)t0);
        };
        // windows of at most 6 x 6 taps along h, w: one value read per
        // partial (col_scan_max); larger ones: col_scan
        if (p.lds_bytes > kColBigLds) {
            if (p.khw <= 6) go(fwd_col_kernel<T, IT, MAXKD, kColBigThreads, 6>, kColBigThreads);
            else go(fwd_col_kernel<T, IT, MAXKD, kColBigThreads, 0>, kColBigThreads);
        } else {
            if (p.khw <= 6) go(fwd_col_kernel<T, IT, MAXKD, kBlock, 6>, kBlock);
            else go(fwd_col_kernel<T, IT, MAXKD, kBlock, 0>, kBlock);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

template <typename T, typename IT>
hipError_t launch_forward_col(const void *x, void *y, IT *idx, const ColPlan &p, hipStream_t s)
{
    if (p.maxkd <= 4) return launch_col<T, IT, 4>(x, y, idx, p, s);
    return launch_col<T, IT, 8>(x, y, idx, p, s);
}

template hipError_t launch_forward_col<F32, int32_t>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F16, int32_t>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<BF16, int32_t>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F32, int64_t>(const void *, void *, int64_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F16, int64_t>(const void *, void *, int64_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<BF16, int64_t>(const void *, void *, int64_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F64, int32_t>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F64, int64_t>(const void *, void *, int64_t *, const ColPlan &, hipStream_t);

}  // namespace mp3d
