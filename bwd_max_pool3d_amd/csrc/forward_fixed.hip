// forward_fixed.hip -- forward for fixed windows whose kernel and stride
// are compile-time constants, as teenygrad's Maxpool3dForward makes kd, kh,
// kw and the strides const generics ("Struct Maxpool3dForward", Fields).
//
// One thread computes V consecutive outputs of one output row (a
// block_ow-style split of the row, same page, description).  It loads the
// KD*KH input row segments under those outputs straight from HBM with
// 16-byte vector loads, plus the few columns that spill past the last
// vector, widens them to binary32 in registers, and scans each window d, h,
// w ascending with the strict-greater / NaN-first rule.  There is no LDS
// and no barrier: input rows shared by neighbouring output rows are re-read
// from L1/L2, and blocks are mapped so that neighbouring blocks run on the
// same XCD and share its L2.
//
// Padding of one position per side (PAD): a row index past an axis end is
// clamped to the nearest row, which repeats that row next to itself in scan
// order; along w the thread's span starts one column left of its vectors
// (PW = 1) -- the left neighbour lane's last column, or at a row start a
// copy of column 0.  When the last windows of a row reach past its end, the
// row's last group has its vectors wholly past the row (the plan admits no
// other case): it loads nothing and its span holds copies of the row's last
// column, its left column.  A copy is equal to the element it repeats and
// sits beside it on the far side from the window's first tap, so the first
// maximum is the same and, with its coordinates clamped back into the axes,
// so is its position.
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// Binary16 windows without NaN, in two passes over the registers: each
// window's maximum first, then the first element equal to it, found by
// scanning from the last element back to the first.  The maxima use the
// packed IEEE 754-2019 maximum (NaN when an operand is NaN) on the loaded
// dwords as they are, two columns per instruction; the compares read either
// half of a dword directly.  The scan carries the code dd << 4 | hh << 2 |
// ww, small enough to be an inline constant of the select.  Returns false,
// computing nothing, when a window holds a NaN.
template <int KD, int KH, int KW, int SW, int SPAN, int V, int NQ, typename Pos>
__device__ __forceinline__ bool f16_first_max(const uint32_t (&q)[KD][KH][NQ], Pos pos,
                                              const uint16_t *__restrict__ xp, int32_t nvalid,
                                              int32_t (&io)[V], uint16_t (&yo)[V])
{
    static_assert(KD <= 4 && KH <= 4 && KW <= 4, "window code fields are 2 bits");
    constexpr int KN = KD * KH * KW;
    constexpr int LAST = ((KD - 1) << 4) | ((KH - 1) << 2) | (KW - 1);
    constexpr int NC = (SPAN + 1) / 2;            // dwords holding the SPAN columns
    static_assert(NC <= NQ, "columns beyond the loaded dwords");
    auto h2 = [&](int dd, int hh, int i) { return __builtin_bit_cast(half2_t, q[dd][hh][i]); };
    auto hv = [&](int dd, int hh, int j) { return h2(dd, hh, j / 2)[j % 2]; };

    // column maxima over the KD*KH rows, then each window's KW columns
    half2_t cm[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        half2_t m = h2(0, 0, i);
#pragma unroll
        for (int r = 1; r < KD * KH; ++r) m = __builtin_elementwise_maximum(m, h2(r / KH, r % KH, i));
        cm[i] = m;
    }
    _Float16 mx[V];
    bool nan = false;
#pragma unroll
    for (int o = 0; o < V; ++o) {
        _Float16 m = cm[(o * SW) / 2][(o * SW) % 2];
#pragma unroll
        for (int ww = 1; ww < KW; ++ww) {
            const int j = o * SW + ww;
            m = __builtin_elementwise_maximum(m, cm[j / 2][j % 2]);
        }
        mx[o] = m;
        nan |= m != m;
    }
    if (nan) return false;

    int32_t c4[V];
#pragma unroll
    for (int o = 0; o < V; ++o) c4[o] = LAST;
#pragma unroll
    for (int k = KN - 2; k >= 0; --k) {
        const int dd = k / (KH * KW), hh = (k / KW) % KH, ww = k % KW;
#pragma unroll
        for (int o = 0; o < V; ++o)
            c4[o] = hv(dd, hh, o * SW + ww) == mx[o] ? ((dd << 4) | (hh << 2) | ww) : c4[o];
    }
#pragma unroll
    for (int o = 0; o < V; ++o) {
        io[o] = pos(o, c4[o] >> 4, (c4[o] >> 2) & 3, c4[o] & 3);
        yo[o] = __builtin_bit_cast(uint16_t, mx[o]);
        // -0 and +0 compare equal, so c4 names the first zero; its sign comes
        // from the element itself (an L1/L2 hit).  Only outputs that exist
        // read it: a window past the row end can name a column past it.
        if (mx[o] == (_Float16)0 && o < nvalid) yo[o] = xp[io[o]];
    }
    return true;
}

// Scan the window of output o (0 <= o < V) over the thread's registers:
// first maximum in d, h, w order, NaN ranking above every number.  Returns
// the value and the window-relative code (dd * KH + hh) * KW + ww.
template <typename T, int KD, int KH, int KW, int SW, typename El>
__device__ __forceinline__ float scan_window(El el, int o, int &code)
{
    float best = T::widen(el(0, 0, o * SW));
    code = 0;
#pragma unroll
    for (int dd = 0; dd < KD; ++dd)
#pragma unroll
        for (int hh = 0; hh < KH; ++hh)
#pragma unroll
            for (int ww = 0; ww < KW; ++ww) {
                if (dd == 0 && hh == 0 && ww == 0) continue;
                const float c = T::widen(el(dd, hh, o * SW + ww));
                // strictly greater, or NaN over a non-NaN best
                const bool take = (best == best) && !(c <= best);
                best = take ? c : best;
                code = take ? (dd * KH + hh) * KW + ww : code;
            }
    return best;
}

// Outputs are written with streaming stores: they leave the caches clean
// for the kernels that follow (measured about 1 % faster over the whole
// forward + backward sequence than cached stores).
template <typename T, typename IT, int KD, int KH, int KW, int SD, int SH, int SW, int V, bool PAD,
          int PW>
__global__ void __launch_bounds__(kBlock)
fwd_fixed_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                 IT *__restrict__ idx, FixedPlan p)
{
    using R = typename T::raw;
    constexpr int SPAN = (V - 1) * SW + KW;      // input columns per thread (taps' span)
    constexpr int VE = 16 / (int)sizeof(R);      // elements per 16-byte vector
    constexpr int OWNC = SPAN - PW;              // span columns from the thread's own vectors
    // PW = 1: whole vectors cover the own columns (no spill past them)
    constexpr int NV = PW ? (OWNC + VE - 1) / VE : SPAN / VE;  // vectors per row
    constexpr int NX = PW ? 0 : SPAN - NV * VE;  // columns past the last vector
    constexpr int NWAVE = kBlock / 64;
    static_assert(PW == 0 || PW == 1, "one column of padding at most");
    static_assert(PW == 0 || PAD, "column padding is padding");
    static_assert(PW == 0 || NV * VE == V * SW, "the left lane's vectors end at its last column");
    static_assert(NX == 0 || V * SW == NV * VE, "the next group must hold the spill columns");
    static_assert(NX <= 4 / (int)sizeof(R), "the spill columns fit one dword");
    const int32_t D = p.g.ax[0].X, H = p.g.ax[1].X, W = p.g.ax[2].X;
    const int32_t OD = p.g.ax[0].O, OH = p.g.ax[1].O, OW = p.g.ax[2].O;
    const int32_t G = p.G;
    const int32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint32_t blk = xcd_local_block(blockIdx.x, gridDim.x);

    // Work split.  rpw > 0: each wave owns rpw whole output rows (G lanes per
    // row), so the lane holding a group's spill columns is in the same wave.
    // rpw == 0: threads run over groups in order (rows may straddle waves).
    uint32_t row;
    int32_t g, lr = 0;
    bool active;
    if (p.rpw > 0) {
        lr = (int32_t)p.groups.div((uint32_t)lane);
        g = lane - lr * G;
        row = (blk * NWAVE + wv) * (uint32_t)p.rpw + lr;
        active = lr < p.rpw && row < p.nrows;
    } else {
        const uint32_t t = blk * kBlock + threadIdx.x;
        row = p.groups.div(t);
        g = (int32_t)(t - row * (uint32_t)G);
        active = t < p.nthreads;
    }
    const uint32_t r2 = p.oh.div(row);
    const int32_t oh = (int32_t)(row - r2 * (uint32_t)OH);
    const uint32_t plane = p.od.div(r2);
    const int32_t od = (int32_t)(r2 - plane * (uint32_t)OD);
    const int32_t ow0 = g * V;
    // first window's first tap row / column; w0 is where the thread's
    // vectors start (16-byte aligned), PW columns right of its span start
    const int32_t d0 = od * SD - (PAD ? p.pd : 0), h0 = oh * SH - (PAD ? p.ph : 0);
    const int32_t w0 = ow0 * SW;
    const R *xp = x + (int64_t)plane * p.g.in_plane;
    // offsets of the KD*KH rows (clamped into the axes under padding)
    int32_t roff[KD][KH];
#pragma unroll
    for (int dd = 0; dd < KD; ++dd)
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
            int32_t d = d0 + dd, h = h0 + hh;
            if constexpr (PAD) {
                d = min(max(d, 0), D - 1);
                h = min(max(h, 0), H - 1);
            }
            roff[dd][hh] = (d * H + h) * W + w0;
        }

    // The thread's span as raw dwords, NQ per row: element j of a row is
    // column w0 - PW + j.  With NX > 0 the last dword of a row holds the
    // spill columns.
    constexpr int EPD = 4 / (int)sizeof(R);      // elements per dword
    constexpr int NQO = NV * 4;                  // dwords of the own vectors
    constexpr int NQ = NQO + (PW || NX > 0 ? 1 : 0);
    uint32_t q[KD][KH][NQ];
    // every row's vector loads first, so that all of them are in flight
    // together (the spill handling below waits for them)
    u32x4 vq[KD][KH][NV];
#pragma unroll
    for (int dd = 0; dd < KD; ++dd)
#pragma unroll
        for (int hh = 0; hh < KH; ++hh)
#pragma unroll
            for (int j = 0; j < NV; ++j) vq[dd][hh][j] = u32x4{0u, 0u, 0u, 0u};
    // idle lanes, and a group whose vectors lie past the row end, load
    // nothing (the latter's columns are filled in below)
    const bool own_in = w0 < W;
    if (active && own_in) {
#pragma unroll
        for (int dd = 0; dd < KD; ++dd)
#pragma unroll
            for (int hh = 0; hh < KH; ++hh)
#pragma unroll
                for (int j = 0; j < NV; ++j)
                    vq[dd][hh][j] = *reinterpret_cast<const u32x4 *>(xp + roff[dd][hh] + j * VE);
    }
    uint32_t own[KD][KH][NQO];
#pragma unroll
    for (int dd = 0; dd < KD; ++dd) {
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const u32x4 t = vq[dd][hh][j];
                own[dd][hh][4 * j] = t.x;
                own[dd][hh][4 * j + 1] = t.y;
                own[dd][hh][4 * j + 2] = t.z;
                own[dd][hh][4 * j + 3] = t.w;
            }
        }
    }
    if constexpr (PW == 0) {
#pragma unroll
        for (int dd = 0; dd < KD; ++dd)
#pragma unroll
            for (int hh = 0; hh < KH; ++hh)
#pragma unroll
                for (int j = 0; j < NQO; ++j) q[dd][hh][j] = own[dd][hh][j];
    } else {
        // column w0 - 1: the left lane's last column (the previous group of
        // the same row), from memory when that group is in another wave,
        // and padding -- a copy of column 0 -- at a row start
        const bool row_start = g == 0;
        const bool left_lane = !row_start && (p.rpw > 0 || lane != 0);
        const bool left_mem = !row_start && !left_lane && active;
#pragma unroll
        for (int dd = 0; dd < KD; ++dd) {
#pragma unroll
            for (int hh = 0; hh < KH; ++hh) {
                const uint32_t nb = __shfl_up(own[dd][hh][NQO - 1], 1);
                uint32_t lw;                       // the left column in the top element of a dword
                if constexpr (EPD == 1) {
                    lw = left_lane ? nb : own[dd][hh][0];
                    if (left_mem) lw = __builtin_bit_cast(uint32_t, xp[roff[dd][hh] - 1]);
                } else {
                    lw = left_lane ? nb : own[dd][hh][0] << 16;
                    if (left_mem) lw = (uint32_t)xp[roff[dd][hh] - 1] << 16;
                }
                if (!own_in) {
                    // right padding: every own column is a copy of the left
                    // column, the row's last
                    const uint32_t c = EPD == 1 ? lw : ((lw & 0xffff0000u) | (lw >> 16));
#pragma unroll
                    for (int j = 0; j < NQO; ++j) own[dd][hh][j] = c;
                }
                if constexpr (EPD == 1) {
                    q[dd][hh][0] = lw;
#pragma unroll
                    for (int j = 0; j < NQO; ++j) q[dd][hh][j + 1] = own[dd][hh][j];
                } else {
                    // re-pair the columns one element later: dword i holds
                    // span elements 2i, 2i + 1 = columns w0 - 1 + 2i, w0 + 2i
                    q[dd][hh][0] = (own[dd][hh][0] << 16) | (lw >> 16);
#pragma unroll
                    for (int j = 1; j < NQO; ++j)
                        q[dd][hh][j] = (own[dd][hh][j] << 16) | (own[dd][hh][j - 1] >> 16);
                    q[dd][hh][NQO] = own[dd][hh][NQO - 1] >> 16;
                }
            }
        }
    }
    if constexpr (NX > 0) {
        // the next group's first columns, across lanes (ds_bpermute); at a
        // row end, or in the wave's last lane, from memory
        const bool from_lane = g + 1 < G && (p.rpw > 0 || lane != 63);
        const bool from_mem = !from_lane && p.spill_load && active;
#pragma unroll
        for (int dd = 0; dd < KD; ++dd) {
#pragma unroll
            for (int hh = 0; hh < KH; ++hh) {
                const uint32_t nb = __shfl_down(q[dd][hh][0], 1);
                uint32_t sp = from_lane ? nb : 0u;
                if (from_mem) {
                    const R *row_p = xp + roff[dd][hh];
#pragma unroll
                    for (int j = 0; j < NX; ++j) {
                        if (w0 + NV * VE + j < W) {
                            const R r = row_p[NV * VE + j];
                            uint32_t b;
                            if constexpr (EPD == 1) b = __builtin_bit_cast(uint32_t, r);
                            else b = (uint32_t)r;
                            sp |= b << (16 * j);
                        }
                    }
                }
                q[dd][hh][NV * 4] = sp;
            }
        }
    }
    // element j of row (dd, hh)
    auto el = [&](int dd, int hh, int j) -> R {
        if constexpr (EPD == 1) return __builtin_bit_cast(float, q[dd][hh][j]);
        else return (R)(q[dd][hh][j / 2] >> (16 * (j % 2)));
    };

    // plane position of element (dd, hh, ww) of output o's window, its
    // coordinates clamped into the axes (a copy stands for the element it
    // repeats)
    auto pos = [&](int o, int dd, int hh, int ww) -> int32_t {
        int32_t d = d0 + dd, h = h0 + hh, w = w0 - PW + o * SW + ww;
        if constexpr (PAD) {
            d = min(max(d, 0), D - 1);
            h = min(max(h, 0), H - 1);
            w = min(max(w, 0), W - 1);
        }
        return (d * H + h) * W + w;
    };

    R yo[V];
    int32_t io[V];
    bool done = false;
    // outputs of this group that exist (none on an idle lane)
    const int32_t nvalid = active ? OW - ow0 : 0;
    if constexpr (T::code == F16::code) done = f16_first_max<KD, KH, KW, SW, SPAN, V, NQ>(q, pos, xp, nvalid, io, yo);
    if (!done) {
#pragma unroll
        for (int o = 0; o < V; ++o) {
            int code;
            const float best = scan_window<T, KD, KH, KW, SW>(el, o, code);
            io[o] = pos(o, code / (KH * KW), (code / KW) % KH, code % KW);
            if (T::exact_nan || best == best || o >= nvalid)
                yo[o] = T::back(best);
            else
                yo[o] = xp[io[o]];            // NaN: copy the element's own bits
        }
    }

    const int64_t obase = (int64_t)row * OW + ow0;    // rows are consecutive in y / idx
    if (p.rpw > 0) {
        // Stage the wave's rows in LDS and write them out as 16-byte vectors.
        __shared__ int32_t s_idx[NWAVE][64 * V];
        __shared__ R s_y[NWAVE][64 * V];
        if (active) {
#pragma unroll
            for (int o = 0; o < V; ++o) {
                if (ow0 + o < OW) {
                    const int32_t k = lr * OW + ow0 + o;
                    s_idx[wv][k] = io[o];
                    s_y[wv][k] = yo[o];
                }
            }
        }
        // the wave reads back what its other lanes wrote: LDS operations of a
        // wave complete in order; keep the compiler from reordering them
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t row0 = (blk * NWAVE + wv) * (uint32_t)p.rpw;
        const int32_t nrow = row0 < p.nrows ? (int32_t)min((uint32_t)p.rpw, p.nrows - row0) : 0;
        const int32_t cnt = nrow * OW;
        const int64_t first = (int64_t)row0 * OW;
        // idx: IVE per 16-byte vector
        if (idx) {
            constexpr int IVE = 16 / (int)sizeof(IT);
            const int32_t head = min((int32_t)((IVE - first % IVE) % IVE), cnt);
            const int32_t nvec = (cnt - head) / IVE, tail0 = head + nvec * IVE;
            if (lane < head) idx[first + lane] = s_idx[wv][lane];
            for (int32_t i = lane; i < nvec; i += 64) {
                const int32_t k = head + IVE * i;
                if constexpr (sizeof(IT) == 4)
                    st_stream(reinterpret_cast<i32x4 *>(idx + first + k),
                              i32x4{s_idx[wv][k], s_idx[wv][k + 1], s_idx[wv][k + 2], s_idx[wv][k + 3]});
                else
                    st_stream(reinterpret_cast<i64x2 *>(idx + first + k),
                              i64x2{s_idx[wv][k], s_idx[wv][k + 1]});
            }
            if (lane < cnt - tail0) idx[first + tail0 + lane] = s_idx[wv][tail0 + lane];
        }
        // y: VE per vector
        {
            const int32_t head = min((int32_t)((VE - first % VE) % VE), cnt);
            const int32_t nvec = (cnt - head) / VE, tail0 = head + nvec * VE;
            if (lane < head) y[first + lane] = s_y[wv][lane];
            for (int32_t i = lane; i < nvec; i += 64) {
                const int32_t k = head + VE * i;
                uint32_t w4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if constexpr (sizeof(R) == 4)
                        w4[q] = __builtin_bit_cast(uint32_t, s_y[wv][k + q]);
                    else
                        w4[q] = (uint32_t)s_y[wv][k + 2 * q] | ((uint32_t)s_y[wv][k + 2 * q + 1] << 16);
                }
                st_stream(reinterpret_cast<u32x4 *>(y + first + k), u32x4{w4[0], w4[1], w4[2], w4[3]});
            }
            if (lane < cnt - tail0) y[first + tail0 + lane] = s_y[wv][tail0 + lane];
        }
    } else if (active) {
        if (p.vec_store && ow0 + V <= OW) {
            static_assert(V == 4, "vector store assumes four outputs");
            if (idx) {
                if constexpr (sizeof(IT) == 4) {
                    st_stream(reinterpret_cast<i32x4 *>(idx + obase), i32x4{io[0], io[1], io[2], io[3]});
                } else {
                    st_stream(reinterpret_cast<i64x2 *>(idx + obase), i64x2{io[0], io[1]});
                    st_stream(reinterpret_cast<i64x2 *>(idx + obase + 2), i64x2{io[2], io[3]});
                }
            }
            if constexpr (sizeof(R) == 4) {
                st_stream(reinterpret_cast<u32x4 *>(y + obase),
                          u32x4{__builtin_bit_cast(uint32_t, yo[0]), __builtin_bit_cast(uint32_t, yo[1]),
                                __builtin_bit_cast(uint32_t, yo[2]), __builtin_bit_cast(uint32_t, yo[3])});
            } else {
                st_stream(reinterpret_cast<u32x2 *>(y + obase),
                          u32x2{(uint32_t)yo[0] | ((uint32_t)yo[1] << 16),
                                (uint32_t)yo[2] | ((uint32_t)yo[3] << 16)});
            }
        } else {
#pragma unroll
            for (int o = 0; o < V; ++o) {
                if (ow0 + o < OW) {
                    y[obase + o] = yo[o];
                    if (idx) idx[obase + o] = io[o];
                }
            }
        }
    }
}

template <typename T, typename IT, int KD, int KH, int KW, int SD, int SH, int SW, bool PAD, int PW>
hipError_t launch_fixed(const void *x, void *y, IT *idx, const FixedPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    uint32_t grid;
    if (p.rpw > 0) {
        const uint32_t waves = (p.nrows + p.rpw - 1) / p.rpw;
        grid = (waves + kBlock / 64 - 1) / (kBlock / 64);
    } else {
        grid = (uint32_t)((p.nthreads + kBlock - 1) / kBlock);
    }
    grid = (grid + 7u) & ~7u;
    launch_kernel((fwd_fixed_kernel<T, IT, KD, KH, KW, SD, SH, SW, FixedPlan::V, PAD, PW>), dim3(grid),
                       dim3(kBlock), 0, s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

}  // namespace

template <typename T, typename IT, int K>
hipError_t launch_fixed_k(const void *x, void *y, IT *idx, const FixedPlan &p, hipStream_t s)
{
    if (p.pw) return launch_fixed<T, IT, K, K, K, 2, 2, 2, true, 1>(x, y, idx, p, s);
    // the row clamp serves padding on d or h, and also a last window past
    // the end of d or h without padding (ceil-mode extents)
    if (p.pd || p.ph || !p.g.plain())
        return launch_fixed<T, IT, K, K, K, 2, 2, 2, true, 0>(x, y, idx, p, s);
    return launch_fixed<T, IT, K, K, K, 2, 2, 2, false, 0>(x, y, idx, p, s);
}

template <typename T, typename IT>
hipError_t launch_forward_fixed(const void *x, void *y, IT *idx, const FixedPlan &p,
                                hipStream_t s)
{
    if (p.g.ax[0].k == 2) return launch_fixed_k<T, IT, 2>(x, y, idx, p, s);
    return launch_fixed_k<T, IT, 3>(x, y, idx, p, s);
}

template hipError_t launch_forward_fixed<F32, int32_t>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<F16, int32_t>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<BF16, int32_t>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<F32, int64_t>(const void *, void *, int64_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<F16, int64_t>(const void *, void *, int64_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<BF16, int64_t>(const void *, void *, int64_t *, const FixedPlan &, hipStream_t);

}  // namespace mp3d
