// kernels.hpp -- launch plans and launchers shared by the C ABI layer
// (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "geometry.hpp"

namespace mp3d {

constexpr int kBlock = 256;            // threads per workgroup (4 waves)

// Forward through LDS: each workgroup owns an output tile
// [od0,od0+tod) x [oh0,oh0+toh) x [ow0,ow0+tow) of one plane, stages the
// input box those windows cover in LDS, and reduces every window there.
struct FwdPlan {
    Geom g;
    int32_t tod, toh, tow;     // output tile extents
    int32_t ntd, nth, ntw;     // tiles per axis
    int32_t full_h, full_w;    // box spans whole rows / whole slices
    int64_t ntiles;            // planes * ntd * nth * ntw
    uint32_t lds_bytes;        // dynamic LDS per workgroup
};

// Backward accumulate path: each workgroup owns an input box
// [d0,d0+td) x [h0,h0+th) x [w0,w0+tw) of one plane, zero-fills a binary32
// accumulator for it in LDS, adds every gy whose idx lands in the box with
// LDS atomics, and stores the rounded box once.
struct BwdPlan {
    Geom g;
    int32_t td, th, tw;        // input tile extents
    int32_t ntd, nth, ntw;
    int64_t ntiles;
    uint32_t lds_bytes;
};

// Backward gather path (windows tile every axis): q = X / O per axis.
struct GatherPlan {
    Geom g;
    int32_t qd, qh, qw;
};

size_t lds_limit();

bool plan_forward(const Geom &g, int elem_bytes, FwdPlan *p);
bool plan_backward(const Geom &g, BwdPlan *p);

template <typename T>
hipError_t launch_forward_tile(const void *x, void *y, int32_t *idx,
                               const FwdPlan &p, hipStream_t s);
template <typename T>
hipError_t launch_forward_direct(const void *x, void *y, int32_t *idx,
                                 const Geom &g, hipStream_t s);
template <typename T>
hipError_t launch_backward_tile(const void *gy, const int32_t *idx, void *gx,
                                const BwdPlan &p, hipStream_t s);
template <typename T>
hipError_t launch_backward_gather(const void *gy, const int32_t *idx, void *gx,
                                  const GatherPlan &p, hipStream_t s);

}  // namespace mp3d
