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
#include "dtype.hpp"
#include "kernels.hpp"

namespace mp3d {

namespace {

// Blocks are dealt to the 8 XCDs round-robin by block id; renumber them so
// that each XCD walks one contiguous run of the work.
__device__ inline uint32_t xcd_local_block(uint32_t b, uint32_t nblocks)
{
    if (nblocks % 8u) return b;
    return (b % 8u) * (nblocks / 8u) + b / 8u;
}

// Scan the window of output o (0 <= o < V) over the thread's registers:
// first maximum in d, h, w order, NaN ranking above every number.  Returns
// the value and the window-relative code (dd * KH + hh) * KW + ww.
template <int KD, int KH, int KW, int SW, int SPAN>
__device__ __forceinline__ float scan_window(const float (&v)[KD][KH][SPAN], int o, int &code)
{
    float best = v[0][0][o * SW];
    code = 0;
#pragma unroll
    for (int dd = 0; dd < KD; ++dd)
#pragma unroll
        for (int hh = 0; hh < KH; ++hh)
#pragma unroll
            for (int ww = 0; ww < KW; ++ww) {
                if (dd == 0 && hh == 0 && ww == 0) continue;
                const float c = v[dd][hh][o * SW + ww];
                // strictly greater, or NaN over a non-NaN best
                const bool take = (best == best) && !(c <= best);
                best = take ? c : best;
                code = take ? (dd * KH + hh) * KW + ww : code;
            }
    return best;
}

template <typename T, int KD, int KH, int KW, int SD, int SH, int SW, int V>
__global__ void __launch_bounds__(kBlock)
fwd_fixed_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                 int32_t *__restrict__ idx, FixedPlan p)
{
    using R = typename T::raw;
    constexpr int SPAN = (V - 1) * SW + KW;      // input columns per thread
    constexpr int VE = 16 / (int)sizeof(R);      // elements per 16-byte vector
    constexpr int NV = SPAN / VE;                // whole vectors per row
    constexpr int NX = SPAN - NV * VE;           // columns past the last vector
    constexpr int NWAVE = kBlock / 64;
    static_assert(NX == 0 || V * SW == NV * VE, "the next group must hold the spill columns");
    static_assert(NX <= 4 / (int)sizeof(R), "the spill columns fit one dword");
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
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
    const int32_t d0 = od * SD, h0 = oh * SH, w0 = ow0 * SW;
    const R *xp = x + (int64_t)plane * p.g.in_plane;
    const R *base = xp + (d0 * H + h0) * W + w0;

    float v[KD][KH][SPAN];
#pragma unroll
    for (int dd = 0; dd < KD; ++dd) {
#pragma unroll
        for (int hh = 0; hh < KH; ++hh) {
            const R *row_p = base + (dd * H + hh) * W;
            u32x4 q[NV];
#pragma unroll
            for (int j = 0; j < NV; ++j) q[j] = u32x4{0u, 0u, 0u, 0u};
            if (active) {                 // idle lanes load nothing and scan zeros
#pragma unroll
                for (int j = 0; j < NV; ++j) q[j] = *reinterpret_cast<const u32x4 *>(row_p + j * VE);
            }
#pragma unroll
            for (int j = 0; j < NV; ++j) T::unpack(q[j], &v[dd][hh][j * VE]);
            const u32x4 q0 = q[0];
            if constexpr (NX > 0) {
                // the next group's first columns, across lanes (ds_bpermute)
                const uint32_t nb = __shfl_down((uint32_t)q0.x, 1);
                const bool in_wave = p.rpw > 0 || lane != 63;
#pragma unroll
                for (int j = 0; j < NX; ++j) {
                    float f = 0.0f;
                    if (g + 1 < G && in_wave) {
                        if constexpr (sizeof(R) == 4)
                            f = __builtin_bit_cast(float, nb);
                        else
                            f = T::widen((R)(j == 0 ? (nb & 0xffffu) : (nb >> 16)));
                    } else if (p.spill_load && active && w0 + NV * VE + j < W) {
                        f = T::widen(row_p[NV * VE + j]);   // row end, or the wave's last lane
                    }
                    v[dd][hh][NV * VE + j] = f;
                }
            }
        }
    }

    R yo[V];
    int32_t io[V];
#pragma unroll
    for (int o = 0; o < V; ++o) {
        int code;
        const float best = scan_window<KD, KH, KW, SW, SPAN>(v, o, code);
        const int dd = code / (KH * KW), hh = (code / KW) % KH, ww = code % KW;
        io[o] = ((d0 + dd) * H + h0 + hh) * W + w0 + o * SW + ww;
        if (T::exact_nan || best == best || !active)
            yo[o] = T::back(best);
        else
            yo[o] = xp[io[o]];            // NaN: copy the element's own bits
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
        // idx: 4 per vector
        {
            const int32_t head = min((int32_t)((4 - first % 4) % 4), cnt);
            const int32_t nvec = (cnt - head) / 4, tail0 = head + nvec * 4;
            if (lane < head) idx[first + lane] = s_idx[wv][lane];
            for (int32_t i = lane; i < nvec; i += 64) {
                const int32_t k = head + 4 * i;
                *reinterpret_cast<i32x4 *>(idx + first + k) =
                    i32x4{s_idx[wv][k], s_idx[wv][k + 1], s_idx[wv][k + 2], s_idx[wv][k + 3]};
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
                *reinterpret_cast<u32x4 *>(y + first + k) = u32x4{w4[0], w4[1], w4[2], w4[3]};
            }
            if (lane < cnt - tail0) y[first + tail0 + lane] = s_y[wv][tail0 + lane];
        }
    } else if (active) {
        if (p.vec_store && ow0 + V <= OW) {
            static_assert(V == 4, "vector store assumes four outputs");
            *reinterpret_cast<i32x4 *>(idx + obase) = i32x4{io[0], io[1], io[2], io[3]};
            if constexpr (sizeof(R) == 4) {
                *reinterpret_cast<u32x4 *>(y + obase) =
                    u32x4{__builtin_bit_cast(uint32_t, yo[0]), __builtin_bit_cast(uint32_t, yo[1]),
                          __builtin_bit_cast(uint32_t, yo[2]), __builtin_bit_cast(uint32_t, yo[3])};
            } else {
                *reinterpret_cast<u32x2 *>(y + obase) =
                    u32x2{(uint32_t)yo[0] | ((uint32_t)yo[1] << 16),
                          (uint32_t)yo[2] | ((uint32_t)yo[3] << 16)};
            }
        } else {
#pragma unroll
            for (int o = 0; o < V; ++o) {
                if (ow0 + o < OW) {
                    y[obase + o] = yo[o];
                    idx[obase + o] = io[o];
                }
            }
        }
    }
}

template <typename T, int KD, int KH, int KW, int SD, int SH, int SW>
hipError_t launch_fixed(const void *x, void *y, int32_t *idx, const FixedPlan &p, hipStream_t s)
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
    hipLaunchKernelGGL((fwd_fixed_kernel<T, KD, KH, KW, SD, SH, SW, FixedPlan::V>), dim3(grid),
                       dim3(kBlock), 0, s, (const R *)x, (R *)y, idx, p);
    return hipGetLastError();
}

}  // namespace

// The window shapes with a compiled kernel: 2x2x2 / stride 2 and
// 3x3x3 / stride 2, the two fixed-window workloads' shapes.
bool fixed_shape_supported(const Geom &g)
{
    const Axis &a = g.ax[0], &b = g.ax[1], &c = g.ax[2];
    if (!a.k || a.k != b.k || a.k != c.k || a.s != b.s || a.s != c.s) return false;
    return (a.k == 2 && a.s == 2) || (a.k == 3 && a.s == 2);
}

template <typename T>
hipError_t launch_forward_fixed(const void *x, void *y, int32_t *idx, const FixedPlan &p,
                                hipStream_t s)
{
    if (p.g.ax[0].k == 2) return launch_fixed<T, 2, 2, 2, 2, 2, 2>(x, y, idx, p, s);
    return launch_fixed<T, 3, 3, 3, 2, 2, 2>(x, y, idx, p, s);
}

template hipError_t launch_forward_fixed<F32>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<F16>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);
template hipError_t launch_forward_fixed<BF16>(const void *, void *, int32_t *, const FixedPlan &, hipStream_t);

}  // namespace mp3d
