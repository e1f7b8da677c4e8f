// forward_col.hip -- forward for any window rule (fixed or adaptive) when
// whole H*W slices can be read as 16-byte vectors, the windows along D are
// at most MAXKD wide, and the tile's D-partials fit in LDS.
//
// Same definition as the other forward kernels ("Struct Maxpool3dForward",
// teenygrad, description; PR #308 page, Summary): per window, the first
// maximum in d, h, w scan order, NaN ranking above every number.
//
// The reduction is split by axis so that every memory access is coalesced
// and conflict-free:
//  stage D (registers): a workgroup owns one plane and a run of output
//    slices od.  Thread i owns the 16-byte column groups i, i+256, ... of
//    the H*W slice.  For each od it loads the window's slices of its column
//    straight from HBM (the next window's loads are issued before the
//    current window is reduced), and reduces them element-wise into
//    (value, first d) pairs, written to LDS in slice layout.  A slice shared
//    by two windows is re-read from L2, not HBM.
//  stage HW (LDS): each output scans its h, w window over the D-partials in
//    ascending order; among equal values the smaller d wins, so the result
//    is the first maximum in (d, h, w) order.
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// Loads of one window's slices of one column group: slot j holds slice
// ds + j while j < n.  Plain (cached) loads: a slice shared by two
// neighbouring windows is then served from L2 the second time; streaming
// loads bypass L2 and read it from HBM again.
template <int MAXKD>
struct ColWin {
    u32x4 q[MAXKD];
};

template <typename R, int MAXKD>
__device__ __forceinline__ void col_load(ColWin<MAXKD> &w, const R *__restrict__ col, int32_t hw,
                                         int32_t n)
{
#pragma unroll
    for (int j = 0; j < MAXKD; ++j)
        if (j < n) w.q[j] = *reinterpret_cast<const u32x4 *>(col + (int64_t)j * hw);
}

// Element-wise first maximum over the n loaded slices; writes the values
// and the winning slice offset (0..n-1) of the VE elements to LDS.
template <typename T, int MAXKD>
__device__ __forceinline__ void col_reduce(const ColWin<MAXKD> &w, int32_t n, float *pv,
                                           uint8_t *pd)
{
    constexpr int VE = 16 / (int)sizeof(typename T::raw);
    float best[VE];
    int32_t bd[VE];
    T::unpack(w.q[0], best);
#pragma unroll
    for (int i = 0; i < VE; ++i) bd[i] = 0;
#pragma unroll
    for (int j = 1; j < MAXKD; ++j) {
        if (j < n) {
            float v[VE];
            T::unpack(w.q[j], v);
#pragma unroll
            for (int i = 0; i < VE; ++i) {
                const bool take = (best[i] == best[i]) && !(v[i] <= best[i]);
                best[i] = take ? v[i] : best[i];
                bd[i] = take ? j : bd[i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < VE; ++i) {
        pv[i] = best[i];
        pd[i] = (uint8_t)bd[i];
    }
}

template <typename T, int MAXKD>
__global__ void __launch_bounds__(kBlock)
fwd_col_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
               int32_t *__restrict__ idx, ColPlan p)
{
    using R = typename T::raw;
    constexpr int VE = 16 / (int)sizeof(R);
    extern __shared__ __align__(16) unsigned char smem[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X, HW = H * W;
    const int32_t tid = threadIdx.x;

    // LDS: window table (oh then ow) | D-partial values | D-partial offsets
    int2 *tab = reinterpret_cast<int2 *>(smem);
    float *pv = reinterpret_cast<float *>(smem + p.tab_bytes);
    uint8_t *pd = reinterpret_cast<uint8_t *>(smem + p.tab_bytes + p.pv_bytes);

    const uint32_t t = blockIdx.x;
    const uint32_t plane = p.ntd_div.div(t);
    const int32_t td = (int32_t)(t - plane * (uint32_t)p.ntd);
    const int32_t od0 = td * p.tod, od1 = min(od0 + p.tod, A.O);
    const int32_t cd = od1 - od0;
    const R *xp = x + (int64_t)plane * p.g.in_plane;

    for (int32_t j = tid; j < B.O + Cw.O; j += kBlock)
        tab[j] = j < B.O ? make_int2(B.start(j), B.end(j))
                         : make_int2(Cw.start(j - B.O), Cw.end(j - B.O));

    // stage D
    const int32_t ngroups = HW / VE;
    for (int32_t gi = tid; gi < ngroups; gi += kBlock) {
        const R *col = xp + gi * VE;
        ColWin<MAXKD> wa, wb;
        int32_t ds = A.start(od0);
        int32_t na = A.end(od0) - ds;
        col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, na);
        for (int32_t odl = 0; odl < cd; odl += 2) {
            int32_t nb = 0, dsb = 0;
            if (odl + 1 < cd) {
                dsb = A.start(od0 + odl + 1);
                nb = A.end(od0 + odl + 1) - dsb;
                col_load<R, MAXKD>(wb, col + (int64_t)dsb * HW, HW, nb);
            }
            col_reduce<T, MAXKD>(wa, na, pv + odl * HW + gi * VE, pd + odl * HW + gi * VE);
            if (odl + 2 < cd) {
                ds = A.start(od0 + odl + 2);
                na = A.end(od0 + odl + 2) - ds;
                col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, na);
            }
            if (odl + 1 < cd)
                col_reduce<T, MAXKD>(wb, nb, pv + (odl + 1) * HW + gi * VE,
                                     pd + (odl + 1) * HW + gi * VE);
        }
    }
    __syncthreads();

    // stage HW
    const int32_t per_slice = B.O * Cw.O;
    const int32_t nout = cd * per_slice;
    const int64_t obase = (int64_t)plane * p.g.out_plane + (int64_t)od0 * per_slice;
    for (int32_t e = tid; e < nout; e += kBlock) {
        const uint32_t q = p.ow_div.div((uint32_t)e);
        const int32_t ow = e - (int32_t)q * Cw.O;
        const uint32_t odl = p.oh_div.div(q);
        const int32_t oh = (int32_t)(q - odl * (uint32_t)B.O);
        const int2 wh = tab[oh], ww = tab[B.O + ow];
        const float *sv = pv + odl * HW;
        const uint8_t *sd = pd + odl * HW;
        int32_t bi = wh.x * W + ww.x;
        float best = sv[bi];
        int32_t bd = sd[bi];
        for (int32_t h = wh.x; h < wh.y; ++h) {
#pragma unroll 4
            for (int32_t w = ww.x; w < ww.y; ++w) {
                const int32_t i = h * W + w;
                const float v = sv[i];
                const int32_t d = sd[i];
                const bool vnan = v != v, bnan = best != best;
                // larger value; or an equal value (or NaN against a NaN best)
                // from an earlier slice; or the first NaN
                const bool take = (v > best) || ((v == best || (vnan && bnan)) && d < bd) ||
                                  (vnan && !bnan);
                best = take ? v : best;
                bd = take ? d : bd;
                bi = take ? i : bi;
            }
        }
        const int32_t dwin = A.start(od0 + (int32_t)odl) + bd;
        const int32_t pos = dwin * HW + bi;
        R raw;
        if (T::exact_nan || best == best)
            raw = T::back(best);
        else
            raw = xp[pos];            // NaN: copy the element's own bits
        st_stream(y + obase + e, raw);
        st_stream(idx + obase + e, pos);
    }
}

template <typename T, int MAXKD>
hipError_t launch_col(const void *x, void *y, int32_t *idx, const ColPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    hipLaunchKernelGGL((fwd_col_kernel<T, MAXKD>), dim3(p.ntiles), dim3(kBlock), p.lds_bytes, s,
                       (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_forward_col(const void *x, void *y, int32_t *idx, const ColPlan &p,
                              hipStream_t s)
{
    if (p.maxkd <= 4) return launch_col<T, 4>(x, y, idx, p, s);
    return launch_col<T, 8>(x, y, idx, p, s);
}

template hipError_t launch_forward_col<F32>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<F16>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);
template hipError_t launch_forward_col<BF16>(const void *, void *, int32_t *, const ColPlan &, hipStream_t);

}  // namespace mp3d
