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

template <typename T, int KD, int KH, int KW, int SD, int SH, int SW, int V>
__global__ void __launch_bounds__(kBlock)
fwd_fixed_kernel(const typename T::raw *__restrict__ x, typename T::raw *__restrict__ y,
                 int32_t *__restrict__ idx, FixedPlan p)
{
    using R = typename T::raw;
    constexpr int SPAN = (V - 1) * SW + KW;      // input columns per thread
    constexpr int VE = 16 / (int)sizeof(R);      // elements per 16-byte vector
    constexpr int NV = SPAN / VE;                // whole vectors per row
    const int32_t H = p.g.ax[1].X, W = p.g.ax[2].X;
    const int32_t OD = p.g.ax[0].O, OH = p.g.ax[1].O, OW = p.g.ax[2].O;

    const uint32_t blk = xcd_local_block(blockIdx.x, gridDim.x);
    const uint32_t t = blk * kBlock + threadIdx.x;
    if (t >= p.nthreads) return;
    const uint32_t r = p.groups.div(t);
    const int32_t g = (int32_t)(t - r * (uint32_t)p.G);
    const uint32_t r2 = p.oh.div(r);
    const int32_t oh = (int32_t)(r - r2 * (uint32_t)OH);
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
            const R *row = base + (dd * H + hh) * W;
#pragma unroll
            for (int j = 0; j < NV; ++j)
                T::unpack(*reinterpret_cast<const u32x4 *>(row + j * VE), &v[dd][hh][j * VE]);
#pragma unroll
            for (int j = NV * VE; j < SPAN; ++j)
                v[dd][hh][j] = (w0 + j < W) ? T::widen(row[j]) : 0.0f;
        }
    }

    const int64_t obase = (int64_t)plane * p.g.out_plane + (od * OH + oh) * OW + ow0;
    R yo[V];
    int32_t io[V];
#pragma unroll
    for (int o = 0; o < V; ++o) {
        float best = v[0][0][o * SW];
        int code = 0;
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
        const int dd = code / (KH * KW), hh = (code / KW) % KH, ww = code % KW;
        io[o] = ((d0 + dd) * H + h0 + hh) * W + w0 + o * SW + ww;
        if (T::exact_nan || best == best)
            yo[o] = T::back(best);
        else
            yo[o] = xp[io[o]];            // NaN: copy the element's own bits
    }
    if (p.vec_store && ow0 + V <= OW) {
        static_assert(V == 4, "vector store assumes four outputs");
        *reinterpret_cast<int4 *>(idx + obase) = make_int4(io[0], io[1], io[2], io[3]);
        if constexpr (sizeof(R) == 4) {
            *reinterpret_cast<float4 *>(y + obase) =
                make_float4(__builtin_bit_cast(float, yo[0]), __builtin_bit_cast(float, yo[1]),
                            __builtin_bit_cast(float, yo[2]), __builtin_bit_cast(float, yo[3]));
        } else {
            *reinterpret_cast<uint2 *>(y + obase) =
                make_uint2((uint32_t)yo[0] | ((uint32_t)yo[1] << 16),
                           (uint32_t)yo[2] | ((uint32_t)yo[3] << 16));
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

template <typename T, int KD, int KH, int KW, int SD, int SH, int SW>
hipError_t launch_fixed(const void *x, void *y, int32_t *idx, const FixedPlan &p, hipStream_t s)
{
    using R = typename T::raw;
    uint32_t grid = (uint32_t)((p.nthreads + kBlock - 1) / kBlock);
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
