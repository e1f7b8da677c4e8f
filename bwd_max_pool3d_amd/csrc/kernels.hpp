// kernels.hpp -- launch plans and launchers shared by the C ABI layer
// (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "geometry.hpp"

namespace mp3d {

constexpr int kBlock = 256;            // threads per workgroup (4 waves)
constexpr int kSlabThreads = 512;      // threads per backward slab workgroup
// Workgroups per launch of the one-tile-per-workgroup kernels (more tiles
// take more launches): with at most 512 threads each, 2^20 keeps a launch
// within 2^32 work-items.
constexpr int64_t kMaxTileGrid = (int64_t)1 << 20;

// Workgroups of the launch that starts at tile t0 of a one-tile-per-
// workgroup kernel over ntiles tiles (launches start at t0 = 0,
// kMaxTileGrid, 2 kMaxTileGrid, ...); rounded up to a multiple of 8, which
// lets blocks map per XCD (the surplus workgroups exit at once).
inline uint32_t tile_grid(int64_t ntiles, int64_t t0)
{
    int64_t grid = ntiles - t0 < kMaxTileGrid ? ntiles - t0 : kMaxTileGrid;
    if (grid >= 64) grid = (grid + 7) & ~(int64_t)7;
    return (uint32_t)grid;
}

// Index elements come as int32 (the library's own) or int64 (torch's).  An
// int64 value outside the int32 range reads as -1, which the backward
// ignores like any value outside the plane.
template <typename IT>
__device__ __forceinline__ int32_t ld_idx(const IT *p, int64_t o)
{
    if constexpr (sizeof(IT) == 4) {
        return p[o];
    } else {
        const int64_t v = p[o];
        return v == (int64_t)(int32_t)v ? (int32_t)v : -1;
    }
}

// Forward through LDS: each workgroup owns an output tile
// [od0,od0+tod) x [oh0,oh0+toh) x [ow0,ow0+tow) of one plane, stages the
// input box those windows cover in LDS, and reduces every window there.
struct FwdPlan {
    Geom g;
    int32_t tod, toh, tow;     // output tile extents
    int32_t ntd, nth, ntw;     // tiles per axis
    int32_t full_h, full_w;    // box spans whole rows / whole slices
    int64_t ntiles;            // planes * ntd * nth * ntw
    TileSplit split;           // tile number -> (plane, td, th, tw)
    uint32_t tab_bytes;        // LDS: window table, 16-byte aligned
    uint32_t part_bytes;       // LDS: each of the two row-partial arrays
    uint32_t lds_bytes;        // dynamic LDS per workgroup
};

// Backward accumulate path: each workgroup owns an input box
// [d0,d0+td) x [h0,h0+th) x [w0,w0+tw) of one plane, zero-fills a binary32
// accumulator for it in LDS, adds every gy whose idx lands in the box with
// an LDS compare-and-swap loop, and stores the rounded box once.
//
// Ordered variant (nphase > 0, slabs only): every window reaching a slab is
// held in registers at once (one round), each gets a class -- its rank
// among the windows that contain its argmax, lexicographic over (d, h, w)
// -- and the classes are added one phase at a time with a barrier between
// phases.  Two outputs of one class never share an input, so a phase needs
// no atomics, and every element's fold runs in ascending output order.
struct BwdPlan {
    Geom g;
    int32_t td, th, tw;        // input tile extents
    int32_t ntd, nth, ntw;
    int64_t ntiles;
    TileSplit split;           // tile number -> (plane, td, th, tw)
    int32_t slab;              // boxes are whole H*W slices
    uint32_t lds_bytes;
    int32_t nphase;            // ordered: md*mh*mw phases; 0: compare-and-swap scatter
    int32_t md, mh, mw;        // ordered: most windows containing a position, per axis
    FastDiv hw_div, w_div;     // by H*W and W (input positions)
    FastDiv ohw_div, ow_div;   // by OH*OW and OW (outputs)
};
constexpr int kBwdRound = 8;               // slab: windows per thread fetched per round
constexpr int kOrdThreads = 256;           // threads per ordered slab workgroup
// Column forward: a workgroup whose slice partials take more LDS than this
// runs with more threads (fewer workgroups fit on a CU, so each needs more
// waves to keep loads in flight).
constexpr uint32_t kColBigLds = 40 * 1024;
constexpr int kColBigThreads = 512;
constexpr int kOrdRound = 8;               // ordered slab: windows per thread (one round)
constexpr int kMaxPhase = 64;              // ordered slab: at most this many phases

// Index-free backward by column stages (backward.hip): each workgroup owns
// a slab of whole slices [d0, d0 + td) of one plane's gx.  It recomputes the
// first maximum of every window reaching the slab with the column forward's
// two stages, takes it as the argmax where it equals y[o] (else scans the
// window in memory), then reuses the same LDS as the slab's accumulator.
constexpr int kRcSlots = 16;               // at most this many windows per thread (one round)
struct RcPlan {
    Geom g;
    int32_t td, ntd;           // slices per slab, slabs per plane
    FastDiv ntd_div;
    uint32_t ntiles;           // planes * ntd
    int32_t maxkd;             // widest window along D
    FastDiv ow_div, oh_div;    // window number in the slab -> (odl, oh, ow)
    uint32_t tab_bytes;        // LDS: window table, 16-byte aligned
    uint32_t lds_bytes;        // table + the larger of D-partials and accumulator
    int32_t slots;             // windows per thread: most windows reaching a slab / threads
    int32_t small3;            // every window has at most 3 taps per axis
};

// Owner-gather backward (backward_owner.hip): each workgroup owns a slab
// [d0, d0 + td) of whole slices of one plane's gx, staged in LDS in the
// storage type, with the (idx, gy) of the windows reaching the slab; the
// first window (in output order) whose argmax is an element sums every
// window's gy there, in ascending output order, and writes it.
constexpr int kOwnerSlots = 8;             // windows per thread per fetch round (512 threads)
struct OwnerPlan {
    Geom g;
    int32_t td, ntd;           // slices per slab, slabs per plane
    FastDiv ntd_div;           // slab number -> plane (when fast)
    int32_t fast;              // slab numbers fit 31 bits
    int64_t ntiles;            // planes * ntd
    int32_t threads;           // 256 or 512
    uint32_t st_bytes;         // LDS: staged slab, 16-byte aligned
    uint32_t ti_bytes;         // LDS: window idx table, 16-byte aligned
    uint32_t lds_bytes;        // + window gy table
    FastDiv hw_div, w_div;     // by H*W, by W (plane positions)
    int32_t depth2;            // every position in at most two windows per axis
};

// General forward (forward_ex.hip): one thread per output, any geometry.
struct ExPlan {
    Geom g;
    int64_t total;             // outputs
    int32_t km;                // 3: at most three taps per window and axis; 0: any
    int32_t fast32;            // total < 2^31: plane_div applies
    FastDiv plane_div;         // by out_plane
    FastDiv ow_div, oh_div;    // by OW, then by OH
};

// Ordered gather for any geometry (small.hip): one thread per input
// element visits every window containing it in ascending output order.
struct OrdPlan {
    Geom g;
    int64_t total;             // input elements
    FastDiv a2_div, a1_div;    // by W, then by H
};

// Small tensors with small windows (small.hip): one thread per output
// (forward) or per input element (backward).  total < 2^31 threads.
constexpr int kSmallK = 3;                 // forward: widest window per axis
constexpr int64_t kSmallFwd = 1 << 18;     // forward: at most this many outputs
constexpr int64_t kSmallBwd = 1 << 20;     // backward: at most this many input elements
constexpr int64_t kTinyInputs = 1 << 16;   // forward: the small kernel first up to this many inputs
struct SmallPlan {
    Geom g;
    uint32_t total;            // threads
    FastDiv plane_div;         // by out_plane (forward) or in_plane (backward)
    FastDiv a2_div, a1_div;    // by the W extent, then the H extent (outputs or inputs)
};

// Backward gather path (windows tile every axis): q = X / O per axis.
struct GatherPlan {
    Geom g;
    int32_t qd, qh, qw;
    int32_t fast;              // thread count < 2^31: the FastDivs below apply
    FastDiv grp_div;           // by the window groups per output row
    FastDiv oh_div, od_div;    // by OH, by OD
    int32_t vec_in;            // idx (and gy) may be read as vectors of 4 windows
    uint32_t grid;             // workgroups (threads are strided over them)
    // the chunk kernel: thread -> (plane, od, chunk c of a slice), c -> (h, w)
    int32_t nc;                // 16-byte chunks per H*W slice (set by the launcher)
    int32_t fast_col;          // N*C*OD*nc < 2^31: nc_div and od_div apply
    FastDiv nc_div, w_div, qh_div;
};

// Forward with compile-time window shape: one thread per V consecutive
// outputs of a row, input rows loaded straight into registers.
struct FixedPlan {
    static constexpr int V = 4;
    Geom g;
    FastDiv groups, oh, od;    // divide by G, OH, OD
    int32_t G;                 // thread groups per output row: ceil(OW / V)
    uint32_t nthreads;         // planes * OD * OH * G
    uint32_t nrows;            // output rows: planes * OD * OH
    int32_t rpw;               // whole rows per wave (0: rows may straddle waves)
    int32_t spill_load;        // some group loads its spill columns itself
    int32_t vec_store;         // outputs may be stored as 4-wide vectors
    int32_t pd, ph, pw;        // padding per axis (0 or 1)
};

// Forward by axis: D-reduce in registers from coalesced column loads, then
// an H*W reduce out of LDS.  One workgroup per (plane, run of tod output
// slices).
struct ColPlan {
    Geom g;
    int32_t tod, ntd;          // output slices per tile, tiles per plane
    FastDiv ntd_div, ow_div, oh_div;
    uint32_t ntiles;           // planes * ntd
    int32_t maxkd;             // widest window along D
    int32_t khw;               // most taps of one window along h or w
    uint32_t tab_bytes, pv_bytes, lds_bytes;
};

// Workgroups are dealt to the 8 XCDs round-robin by workgroup id; renumber
// them so that each XCD walks one contiguous run of the work (and shares
// its L2 across neighbouring tiles).
__host__ __device__ __forceinline__ uint32_t xcd_local_block(uint32_t b, uint32_t nblocks)
{
    if (nblocks % 8u) return b;
    return (b % 8u) * (nblocks / 8u) + b / 8u;
}

// Kernel-time events armed for the next C-ABI call on this thread (see
// mp3d_time_next_call): the call's first kernel records `start` at its
// start, each kernel records `stop` at its end (the last one's stands).
struct LaunchTiming {
    hipEvent_t start, stop;
};
LaunchTiming &launch_timing();

// Every kernel of the library is launched through here.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds,
                          hipStream_t s, Args... args)
{
    LaunchTiming &t = launch_timing();
    if (t.stop) {
        hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t.start, t.stop, 0u,
                              static_cast<KArgs>(args)...);
        t.start = nullptr;
    } else {
        hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
    }
}

size_t lds_limit();
int device_cus();      // compute units of the current device

bool fixed_shape_supported(const Geom &g);
bool plan_fixed(const Geom &g, int elem_bytes, const void *x, const void *y,
                const void *idx, FixedPlan *p);

bool plan_forward(const Geom &g, int elem_bytes, FwdPlan *p);
bool plan_col(const Geom &g, int elem_bytes, const void *x, ColPlan *p);
// cell_bytes: the accumulator cell, 4 (binary32) or 8 (binary64).
// plan_backward with ordered = false always succeeds; with ordered = true
// it fails when the ordered slab cannot hold the geometry (slices larger
// than the accumulator, a slab reached by more windows than one round
// holds, or more than kMaxPhase phases): the ordered gather serves then.
bool plan_backward(const Geom &g, bool ordered, int cell_bytes, BwdPlan *p);
bool plan_small_forward(const Geom &g, SmallPlan *p);
bool plan_small_backward(const Geom &g, SmallPlan *p);
void plan_ordered(const Geom &g, OrdPlan *p);
// windows that tile every axis (q = X / O per axis)
void plan_gather(const Geom &g, GatherPlan *p);
// es: storage element bytes; acc_bytes: accumulator cell bytes
bool plan_rc(const Geom &g, int es, int acc_bytes, const void *x, RcPlan *p);
void plan_ex(const Geom &g, ExPlan *p);
// es: storage element bytes.  Fails when a slab's staging and window table
// do not fit LDS or a position lies in too many windows.
bool plan_owner(const Geom &g, int es, OwnerPlan *p);
int64_t max_taps(const Axis &a);         // most taps of one window on the axis

template <typename T, typename IT>
hipError_t launch_forward_tile(const void *x, void *y, IT *idx, const FwdPlan &p, hipStream_t s);
template <typename T, typename IT>
hipError_t launch_forward_fixed(const void *x, void *y, IT *idx, const FixedPlan &p, hipStream_t s);
template <typename T, typename IT>
hipError_t launch_forward_col(const void *x, void *y, IT *idx, const ColPlan &p, hipStream_t s);
template <typename T, typename IT>
hipError_t launch_forward_direct(const void *x, void *y, IT *idx, const Geom &p, hipStream_t s);
template <typename T, typename IT>
hipError_t launch_forward_ex(const void *x, void *y, IT *idx, const ExPlan &p, hipStream_t s);
template <typename T, typename Src>
hipError_t launch_backward_tile(const void *gy, const Src &src, void *gx, const BwdPlan &p,
                                hipStream_t s);
template <typename T, typename IT>
hipError_t launch_forward_small(const void *x, void *y, IT *idx, const SmallPlan &p, hipStream_t s);
template <typename T, typename Src>
hipError_t launch_backward_owner(const void *gy, const Src &src, void *gx, const OwnerPlan &p,
                                 hipStream_t s);
template <typename T, typename Src>
hipError_t launch_backward_small(const void *gy, const Src &src, void *gx, const SmallPlan &p,
                                 hipStream_t s);
template <typename T>
hipError_t launch_backward_rc(const void *x, const void *y, const void *gy, void *gx,
                              const RcPlan &p, hipStream_t s);
template <typename T, typename Src>
hipError_t launch_backward_gather(const void *gy, const Src &src, void *gx, const GatherPlan &p,
                                  hipStream_t s);
template <typename T, typename Src>
hipError_t launch_backward_ordered(const void *gy, const Src &src, void *gx, const OrdPlan &p,
                                   hipStream_t s);

}  // namespace mp3d
