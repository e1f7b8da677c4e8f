// plan.hip -- host-side choice of tile shapes for the LDS kernels.
//
// Forward: a tile is a block of outputs of one plane; its input box is the
// union of their windows, and it must fit the LDS budget.  Whole H*W slices
// are preferred (the box is then one contiguous span of the plane and is
// read with 16-byte coalesced loads); only when one window's slices do not
// fit are rows, then row segments, cut.
//
// Backward: a tile is a box of one plane's gx held as binary32 in LDS,
// again whole slices where possible.
#include <algorithm>

#include "kernels.hpp"

namespace mp3d {

namespace {

constexpr int64_t kLdsCap = 64 * 1024;     // LDS per workgroup, all uses
constexpr int64_t kBoxBudget = 60 * 1024;   // of which the forward's input box
constexpr int64_t kWantTiles = 1024;        // >= 4 workgroups per CU

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest input extent covered by t consecutive windows of axis a (the
// union of windows [o0, o0+t) over every tile start o0 = 0, t, 2t, ...).
int64_t box_extent(const Axis &a, int32_t t)
{
    if (a.k) return std::min<int64_t>((int64_t)(t - 1) * a.s + a.k, a.X);
    const int64_t ntiles = cdiv(a.O, t);
    if (ntiles > 65536)   // bound instead of scanning every tile
        return std::min<int64_t>(cdiv((int64_t)t * a.X, a.O) + 1, a.X);
    int64_t m = 0;
    for (int64_t o0 = 0; o0 < a.O; o0 += t) {
        const int32_t o1 = (int32_t)std::min<int64_t>(o0 + t, a.O) - 1;
        m = std::max<int64_t>(m, a.end(o1) - a.start((int32_t)o0));
    }
    return m;
}

// Largest t (1..O) with box_extent(a, t) * unit <= budget, or 0.
int32_t fit_tile(const Axis &a, int64_t unit, int64_t budget)
{
    int32_t best = 0;
    const int32_t cap = std::min<int32_t>(a.O, 4096);
    for (int32_t t = 1; t <= cap; ++t) {
        if (box_extent(a, t) * unit <= budget) best = t;
        else break;
    }
    return best;
}

// Even out tiles: the smallest tile size giving the same tile count.
int32_t balance(int32_t O, int32_t t) { return (int32_t)cdiv(O, cdiv(O, t)); }

}  // namespace

bool plan_forward(const Geom &g, int es, FwdPlan *p)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    const int64_t H = B.X, W = Cw.X;
    const int64_t cap = std::min<int64_t>(kLdsCap, (int64_t)lds_limit());
    const int64_t budget = std::min<int64_t>(kBoxBudget, cap - 4096);
    p->g = g;
    int32_t tod = 0, toh = B.O, tow = Cw.O;
    int full_h = 1, full_w = 1;
    int32_t t = fit_tile(A, H * W * es, budget);
    if (t > 0) {
        // enough tiles to spread over the chip when there are few planes
        const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
        const int32_t tpar = (int32_t)std::max<int64_t>(1, A.O / per_plane);
        tod = balance(A.O, std::min(t, tpar));
    } else {
        tod = 1;
        full_h = 0;
        const int64_t dext = box_extent(A, 1);
        toh = fit_tile(B, dext * W * es, budget);
        if (toh > 0) {
            toh = balance(B.O, toh);
        } else {
            toh = 1;
            full_w = 0;
            tow = fit_tile(Cw, dext * box_extent(B, 1) * es, budget);
            if (tow == 0) return false;
            tow = balance(Cw.O, tow);
        }
    }
    p->tod = tod;
    p->toh = toh;
    p->tow = tow;
    p->ntd = (int32_t)cdiv(A.O, tod);
    p->nth = (int32_t)cdiv(B.O, toh);
    p->ntw = (int32_t)cdiv(Cw.O, tow);
    p->full_h = full_h;
    p->full_w = full_w;
    p->ntiles = g.planes * p->ntd * p->nth * p->ntw;
    const int64_t lh = full_h ? H : box_extent(B, toh);
    const int64_t lw = full_w ? W : box_extent(Cw, tow);
    const int64_t box = box_extent(A, tod) * lh * lw * es;
    const int64_t tab = ((int64_t)(tod + toh + tow) * 8 + 15) & ~(int64_t)15;
    if (tab + 16 + box > cap) return false;   // e.g. O far above X: huge tables
    p->lds_bytes = (uint32_t)(tab + 16 + box);
    return true;
}

bool plan_backward(const Geom &g, BwdPlan *p)
{
    const int32_t D = g.ax[0].X, H = g.ax[1].X, W = g.ax[2].X;
    const int64_t budget = std::min<int64_t>(kLdsCap, (int64_t)lds_limit());
    const int64_t slice = (int64_t)H * W * 4;
    p->g = g;
    if (slice <= budget) {
        int32_t td = (int32_t)std::min<int64_t>(D, budget / slice);
        const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
        td = std::min<int32_t>(td, (int32_t)std::max<int64_t>(1, D / per_plane));
        p->td = (int32_t)cdiv(D, cdiv(D, td));
        p->th = H;
        p->tw = W;
    } else if ((int64_t)W * 4 <= budget) {
        p->td = 1;
        const int32_t th = (int32_t)std::min<int64_t>(H, budget / ((int64_t)W * 4));
        p->th = (int32_t)cdiv(H, cdiv(H, th));
        p->tw = W;
    } else {
        p->td = 1;
        p->th = 1;
        const int32_t tw = (int32_t)std::min<int64_t>(W, budget / 4);
        p->tw = (int32_t)cdiv(W, cdiv(W, tw));
    }
    p->ntd = (int32_t)cdiv(D, p->td);
    p->nth = (int32_t)cdiv(H, p->th);
    p->ntw = (int32_t)cdiv(W, p->tw);
    p->ntiles = g.planes * p->ntd * p->nth * p->ntw;
    p->lds_bytes = (uint32_t)((int64_t)p->td * p->th * p->tw * 4);
    return true;
}

}  // namespace mp3d
