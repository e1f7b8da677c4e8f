// forward_col.hip -- forward for any window rule (fixed or adaptive) when
// whole H*W slices can be read as 16-byte vectors, the windows along D are
// at most 8 wide, and a tile's D-partials fit in LDS.
//
// Same definition as the other forward kernels ("Struct Maxpool3dForward",
// teenygrad, description; PR #308 page, Summary): per window, the first
// maximum in d, h, w scan order, NaN ranking above every number.
//
// A workgroup owns one plane and a run of output slices od.  The reduction
// is split by axis so that every memory access is coalesced:
//  stage D (registers): thread i owns the 16-byte column groups i,
//    i + NT, ... of the H*W slice (NT threads: 256, or 512 when the tile's
//    D-partials need much LDS and few workgroups fit on a CU).  For each od it loads the window's
//    slices of its column (the next window's loads are issued before the
//    current window is reduced; a slice shared by two windows is read
//    twice, the second time from L2), and reduces them element-wise to the
//    first maximum over d, written to LDS as the value and its d offset.
//  stage HW (LDS): each output scans the D-partials of its h, w window once,
//    keeping the running maximum and the smallest key d << 24 | (h * W + w)
//    among the partials equal to it: the smallest d, then the first (h, w)
//    in scan order, which is the first maximum in (d, h, w) order.
// Stage D finds a maximum first (IEEE 754-2019 maximum, NaN when an operand
// is NaN) and its first slot second; stage HW keeps the running maximum and
// the smallest key among the elements equal to it in one pass, and the
// smallest key among NaNs apart (a window holding a NaN takes its first NaN).
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// One window's slices of one column group: slot j holds slice ds + j for
// j < n and repeats slice ds + n - 1 beyond.  The loads carry no branch, so
// that every load of a tile is in flight at once; a repeated slice never
// comes first among equal values.  Plain (cached) loads: a slice shared by
// two neighbouring windows is served from L2 the second time.
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
        w.q[j] = *reinterpret_cast<const u32x4 *>(col + (int64_t)min(j, n - 1) * hw);
}

// Element-wise first maximum over the window's slots: writes the values and
// the winning slot (the d offset in the window) to LDS.
template <typename T, int MAXKD>
__device__ __forceinline__ void col_reduce(const ColWin<MAXKD> &w, typename T::acc *pv, uint8_t *pd)
{
    using A = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(typename T::raw);
    A v[MAXKD][VE];
#pragma unroll
    for (int j = 0; j < MAXKD; ++j) T::unpack(w.q[j], v[j]);
#pragma unroll
    for (int i = 0; i < VE; ++i) {
        A m = v[0][i];
#pragma unroll
        for (int j = 1; j < MAXKD; ++j) m = __builtin_elementwise_maximum(m, v[j][i]);
        // the first slot equal to the maximum (the first NaN when it is
        // NaN), found from the last slot back; the value is taken from the
        // slot itself, which keeps the sign of a zero and a NaN's bits
        int32_t jd = MAXKD - 1;
        A val = v[MAXKD - 1][i];
        if (m == m) {
#pragma unroll
            for (int j = MAXKD - 2; j >= 0; --j) {
                const bool hit = v[j][i] == m;
                jd = hit ? j : jd;
                val = hit ? v[j][i] : val;
            }
        } else {
#pragma unroll
            for (int j = MAXKD - 2; j >= 0; --j) {
                const bool hit = v[j][i] != v[j][i];
                jd = hit ? j : jd;
                val = hit ? v[j][i] : val;
            }
        }
        pv[i] = val;
        pd[i] = (uint8_t)jd;
    }
}

template <typename T, typename IT, int MAXKD, int NT>
__global__ void __launch_bounds__(NT)
fwd_col_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
               IT *__restrict__ idx, ColPlan p)
{
    using R = typename T::raw;
    using Acc = typename T::acc;
    constexpr int VE = 16 / (int)sizeof(R);
    extern __shared__ __align__(16) unsigned char smem[];
    const Axis A = p.g.ax[0], B = p.g.ax[1], Cw = p.g.ax[2];
    const int32_t H = B.X, W = Cw.X, HW = H * W;
    const int32_t tid = threadIdx.x;

    // LDS: window table (oh then ow) | D-partial values | D-partial d offsets
    int2 *tab = reinterpret_cast<int2 *>(smem);
    Acc *pv = reinterpret_cast<Acc *>(smem + p.tab_bytes);
    uint8_t *pd = reinterpret_cast<uint8_t *>(smem + p.tab_bytes + p.pv_bytes);

    const uint32_t t = xcd_local_block(blockIdx.x, gridDim.x);
    const uint32_t plane = p.ntd_div.div(t);
    const int32_t td = (int32_t)(t - plane * (uint32_t)p.ntd);
    const int32_t od0 = td * p.tod, od1 = min(od0 + p.tod, A.O);
    const int32_t cd = od1 - od0;
    const R *xp = x + (int64_t)plane * p.g.in_plane;

    for (int32_t j = tid; j < B.O + Cw.O; j += NT)
        tab[j] = j < B.O ? make_int2(B.start(j), B.end(j))
                         : make_int2(Cw.start(j - B.O), Cw.end(j - B.O));

    // stage D: the loads of two windows in flight while the previous one
    // is reduced
    const int32_t ngroups = HW / VE;
    for (int32_t gi = tid; gi < ngroups; gi += NT) {
        const R *col = xp + gi * VE;
        ColWin<MAXKD> wa, wb;
        int32_t ds = A.start(od0);
        col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, A.end(od0) - ds);
        for (int32_t odl = 0; odl < cd; odl += 2) {
            if (odl + 1 < cd) {
                ds = A.start(od0 + odl + 1);
                col_load<R, MAXKD>(wb, col + (int64_t)ds * HW, HW, A.end(od0 + odl + 1) - ds);
            }
            col_reduce<T, MAXKD>(wa, pv + odl * HW + gi * VE, pd + odl * HW + gi * VE);
            if (odl + 2 < cd) {
                ds = A.start(od0 + odl + 2);
                col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, A.end(od0 + odl + 2) - ds);
            }
            if (odl + 1 < cd)
                col_reduce<T, MAXKD>(wb, pv + (odl + 1) * HW + gi * VE, pd + (odl + 1) * HW + gi * VE);
        }
    }
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
        const int2 wh = tab[oh], ww = tab[B.O + ow];
        const Acc *sv = pv + odl * HW;
        const uint8_t *sd = pd + odl * HW;
        // one pass: the running maximum and the smallest key among the
        // elements equal to it; NaNs tracked apart (the first NaN wins)
        Acc m = sv[wh.x * W + ww.x];
        uint32_t bk = 0xffffffffu, nk = 0xffffffffu;
        for (int32_t h = wh.x; h < wh.y; ++h) {
#pragma unroll 4
            for (int32_t w = ww.x; w < ww.y; ++w) {
                const int32_t i = h * W + w;
                const Acc v = sv[i];
                const uint32_t k = ((uint32_t)sd[i] << 24) | (uint32_t)i;
                const bool gt = v > m;
                bk = gt ? k : (v == m ? min(bk, k) : bk);
                m = gt ? v : m;
                nk = v != v ? min(nk, k) : nk;
            }
        }
        if (nk != 0xffffffffu) bk = nk;
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
    int64_t grid = p.ntiles;
    if (p.lds_bytes > kColBigLds)
        hipLaunchKernelGGL((fwd_col_kernel<T, IT, MAXKD, kColBigThreads>), dim3((uint32_t)grid),
                           dim3(kColBigThreads), p.lds_bytes, s, (const R *)x, (R *)y, idx, p);
    else
        hipLaunchKernelGGL((fwd_col_kernel<T, IT, MAXKD, kBlock>), dim3((uint32_t)grid),
                           dim3(kBlock), p.lds_bytes, s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
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
