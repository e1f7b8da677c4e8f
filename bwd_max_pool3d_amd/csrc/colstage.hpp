// colstage.hpp -- the two stages of the column forward, shared by the
// forward (forward_col.hip) and the index-free backward, which recomputes
// each window's first maximum the same way (backward.hip).
//
// Definition ("Struct Maxpool3dForward", teenygrad, description; PR #308
// page, Summary): per window, the first maximum in d, h, w scan order, NaN
// ranking above every number.
//  stage D (registers): a thread owns 16-byte column groups of an H*W
//    slice; for each output slice od it loads the window's slices of its
//    column group and reduces them element-wise to the first maximum over d
//    (IEEE 754-2019 maximum first, NaN when an operand is NaN, then its
//    first slot), written to LDS as the value and its d offset.
//  stage HW (LDS): a window scans the D-partials of its h, w span once,
//    keeping the running maximum and the smallest key d << 24 | (h * W + w)
//    among the partials equal to it (the smallest d, then the first (h, w):
//    the first maximum in d, h, w order), and the smallest key among NaNs
//    apart (a window holding a NaN takes its first NaN).
#pragma once

#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

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

// Where stage D writes a slice's D-partials and stage HW reads them.
// PartSplit: the values (binary32, or binary64 for float64) and their 8-bit
// d offsets in two arrays.
template <typename T>
struct PartSplit {
    using Acc = typename T::acc;
    Acc *pv;
    uint8_t *pd;
    __device__ __forceinline__ void put(int32_t i, Acc v, int32_t jd) const {
        pv[i] = v;
        pd[i] = (uint8_t)jd;
    }
    __device__ __forceinline__ Acc value(int32_t i) const { return pv[i]; }
    __device__ __forceinline__ uint32_t dof(int32_t i) const { return pd[i]; }
    __device__ __forceinline__ PartSplit at(int32_t off) const { return {pv + off, pd + off}; }
};

// PartPacked (16-bit storage types): one 32-bit word per partial, the value
// narrowed back to its storage bits in the low half (exact for every
// number; a NaN stays a NaN) and the d offset in the high half.
template <typename T>
struct PartPacked {
    using Acc = typename T::acc;
    uint32_t *pk;
    __device__ __forceinline__ void put(int32_t i, Acc v, int32_t jd) const {
        pk[i] = (uint32_t)T::narrow(v) | ((uint32_t)jd << 16);
    }
    __device__ __forceinline__ Acc value(int32_t i) const {
        return T::widen((typename T::raw)(pk[i] & 0xffffu));
    }
    __device__ __forceinline__ uint32_t dof(int32_t i) const { return pk[i] >> 16; }
    __device__ __forceinline__ PartPacked at(int32_t off) const { return {pk + off}; }
};

// Element-wise first maximum over the window's slots: stores the values and
// the winning slot (the d offset in the window) through the partial store.
template <typename T, int MAXKD, typename P>
__device__ __forceinline__ void col_reduce(const ColWin<MAXKD> &w, const P &part)
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
        part.put(i, val, jd);
    }
}

// Stage D for output slices [od0, od0 + cd) of one plane (xp): the
// D-partials of slice odl go to part.at(odl * HW).  The loads of two
// windows are in flight while the previous one is reduced; a slice shared
// by two windows is read twice, the second time from L2.
template <typename T, int MAXKD, int NT, typename P>
__device__ __forceinline__ void col_stage_d(const typename T::raw *__restrict__ xp, const Axis &A,
                                            int32_t HW, int32_t od0, int32_t cd, const P &part)
{
    using R = typename T::raw;
    constexpr int VE = 16 / (int)sizeof(R);
    const int32_t ngroups = HW / VE;
    for (int32_t gi = (int32_t)threadIdx.x; gi < ngroups; gi += NT) {
        const R *col = xp + gi * VE;
        ColWin<MAXKD> wa, wb;
        int32_t ds = A.start(od0);
        col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, A.end(od0) - ds);
        for (int32_t odl = 0; odl < cd; odl += 2) {
            if (odl + 1 < cd) {
                ds = A.start(od0 + odl + 1);
                col_load<R, MAXKD>(wb, col + (int64_t)ds * HW, HW, A.end(od0 + odl + 1) - ds);
            }
            col_reduce<T, MAXKD>(wa, part.at(odl * HW + gi * VE));
            if (odl + 2 < cd) {
                ds = A.start(od0 + odl + 2);
                col_load<R, MAXKD>(wa, col + (int64_t)ds * HW, HW, A.end(od0 + odl + 2) - ds);
            }
            if (odl + 1 < cd)
                col_reduce<T, MAXKD>(wb, part.at((odl + 1) * HW + gi * VE));
        }
    }
}

// Stage HW for one window: rows [wh.x, wh.y), columns [ww.x, ww.y) of one
// slice's D-partials.  Returns the key of the first maximum (the first NaN
// when there is one) and sets m to the maximum.
template <typename P, typename Acc>
__device__ __forceinline__ uint32_t col_scan(const P &sp, int32_t W, int2 wh, int2 ww, Acc &m)
{
    m = sp.value(wh.x * W + ww.x);
    uint32_t bk = 0xffffffffu, nk = 0xffffffffu;
    for (int32_t h = wh.x; h < wh.y; ++h) {
#pragma unroll 4
        for (int32_t w = ww.x; w < ww.y; ++w) {
            const int32_t i = h * W + w;
            const Acc v = sp.value(i);
            const uint32_t k = (sp.dof(i) << 24) | (uint32_t)i;
            const bool gt = v > m;
            bk = gt ? k : (v == m ? min(bk, k) : bk);
            m = gt ? v : m;
            nk = v != v ? min(nk, k) : nk;
        }
    }
    return nk != 0xffffffffu ? nk : bk;
}

// Stage HW for windows of at most K rows and K columns, every load issued
// at once: row and column numbers are clamped to the window's span, and a
// clamped tap repeats an element of the window with its own key, which
// changes neither the maximum nor the smallest key.
template <int K, typename P, typename Acc>
__device__ __forceinline__ uint32_t col_scan_k(const P &sp, int32_t W, int2 wh, int2 ww, Acc &m)
{
    int32_t at[K * K];
    Acc v[K * K];
    uint32_t dd[K * K];
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
        for (int c = 0; c < K; ++c)
            at[j * K + c] = min(wh.x + j, wh.y - 1) * W + min(ww.x + c, ww.y - 1);
#pragma unroll
    for (int q = 0; q < K * K; ++q) {
        v[q] = sp.value(at[q]);
        dd[q] = sp.dof(at[q]);
    }
    m = v[0];
    uint32_t bk = 0xffffffffu, nk = 0xffffffffu;
#pragma unroll
    for (int q = 0; q < K * K; ++q) {
        const uint32_t k = (dd[q] << 24) | (uint32_t)at[q];
        const bool gt = v[q] > m;
        bk = gt ? k : (v[q] == m ? min(bk, k) : bk);
        m = gt ? v[q] : m;
        nk = v[q] != v[q] ? min(nk, k) : nk;
    }
    return nk != 0xffffffffu ? nk : bk;
}

// Stage HW for windows of at most K rows and K columns, reading each
// partial's value once and its d offset only for the winner: the window's
// maximum first (every value load issued at once; rows and columns clamped
// to the span, so a clamped tap repeats an element of the window), then the
// first tap in (h, w) order equal to it.  When that tap is the only one
// equal to the maximum, its key is the smallest; a tie (several taps, or
// -0 and +0) or a NaN maximum takes col_scan, which reads every key.
template <int K, typename P, typename Acc>
__device__ __forceinline__ uint32_t col_scan_max(const P &sp, int32_t W, int2 wh, int2 ww, Acc &m)
{
    int32_t at[K * K];
    Acc v[K * K];
    const int32_t nh = wh.y - wh.x, nw = ww.y - ww.x;
#pragma unroll
    for (int j = 0; j < K; ++j)
#pragma unroll
        for (int c = 0; c < K; ++c)
            at[j * K + c] = min(wh.x + j, wh.y - 1) * W + min(ww.x + c, ww.y - 1);
#pragma unroll
    for (int q = 0; q < K * K; ++q) v[q] = sp.value(at[q]);
    Acc mx = v[0];
#pragma unroll
    for (int q = 1; q < K * K; ++q) mx = __builtin_elementwise_maximum(mx, v[q]);
    int32_t first = 0, hits = 0;
#pragma unroll
    for (int q = K * K - 1; q >= 0; --q) {
        // clamped taps repeat an element: count each element once
        const bool own = (q / K) < nh && (q % K) < nw;
        const bool hit = v[q] == mx;
        first = hit ? q : first;
        hits += (hit && own) ? 1 : 0;
    }
    if (hits == 1) {
        // the winner's position from its tap number (no indexing of at[]
        // by a run-time value, which would put it in scratch memory)
        const int32_t i = min(wh.x + first / K, wh.y - 1) * W + min(ww.x + first % K, ww.y - 1);
        m = mx;
        return (sp.dof(i) << 24) | (uint32_t)i;
    }
    return col_scan(sp, W, wh, ww, m);
}

}  // namespace mp3d
