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
#include <stdlib.h>

#include <algorithm>

#include "kernels.hpp"

namespace mp3d {

namespace {

constexpr int64_t kLdsCap = 64 * 1024;     // forward LDS per workgroup, all uses
constexpr int64_t kAccBudget = 40 * 1024;   // backward accumulator per workgroup
constexpr int32_t kColMaxTod = 2;           // column forward: output slices per tile
constexpr int64_t kOrdBudget = 40 * 1024;   // the same, ordered slabs
constexpr int64_t kWantTiles = 1024;        // >= 4 workgroups per CU
constexpr int64_t kOwnerBudget = 80 * 1024; // owner gather: LDS per workgroup (2 per CU)
constexpr int64_t kOwnerMaxCand = 64;       // owner gather: windows containing one position
constexpr int64_t kMaxGrid = (int64_t)1 << 20;       // grid-stride kernels: workgroups per launch

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

// Even out tiles: the smallest tile size giving the same tile count.
int32_t balance(int32_t O, int32_t t) { return (int32_t)cdiv(O, cdiv(O, t)); }

}  // namespace

// LDS bytes of a forward tile of tod x toh x tow outputs: window table,
// two row-partial arrays (value, column) and the input box plus 16 bytes of
// alignment slack.
static int64_t fwd_lds(const Geom &g, int es, int32_t tod, int32_t toh, int32_t tow,
                       bool full_h, bool full_w, int64_t *tab, int64_t *part)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    const int64_t ld = box_extent(A, tod);
    const int64_t lh = full_h ? B.X : box_extent(B, toh);
    const int64_t lw = full_w ? Cw.X : box_extent(Cw, tow);
    *tab = ((int64_t)(tod + toh + tow) * 8 + 15) & ~(int64_t)15;
    *part = ((ld * lh * tow * 4) + 15) & ~(int64_t)15;
    return *tab + 2 * *part + 16 + ld * lh * lw * es;
}

bool plan_forward(const Geom &g, int es, FwdPlan *p)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    const int64_t cap = std::min<int64_t>(kLdsCap, (int64_t)lds_limit());
    int64_t tab = 0, part = 0;
    p->g = g;
    int32_t tod = 0, toh = B.O, tow = Cw.O;
    bool full_h = true, full_w = true;
    // largest whole-slice tile that fits
    for (int32_t t = 1; t <= std::min<int32_t>(A.O, 4096); ++t) {
        if (fwd_lds(g, es, t, toh, tow, true, true, &tab, &part) <= cap) tod = t;
        else break;
    }
    if (tod > 0) {
        // enough tiles to spread over the chip when there are few planes
        const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
        const int32_t tpar = (int32_t)std::max<int64_t>(1, A.O / per_plane);
        tod = balance(A.O, std::min(tod, tpar));
    } else {
        tod = 1;
        full_h = false;
        toh = 0;
        for (int32_t t = 1; t <= std::min<int32_t>(B.O, 4096); ++t) {
            if (fwd_lds(g, es, 1, t, tow, false, true, &tab, &part) <= cap) toh = t;
            else break;
        }
        if (toh > 0) {
            toh = balance(B.O, toh);
        } else {
            toh = 1;
            full_w = false;
            tow = 0;
            for (int32_t t = 1; t <= std::min<int32_t>(Cw.O, 4096); ++t) {
                if (fwd_lds(g, es, 1, 1, t, false, false, &tab, &part) <= cap) tow = t;
                else break;
            }
            if (tow == 0) return false;
            tow = balance(Cw.O, tow);
        }
    }
    const int64_t lds = fwd_lds(g, es, tod, toh, tow, full_h, full_w, &tab, &part);
    if (lds > cap) return false;
    p->tod = tod;
    p->toh = toh;
    p->tow = tow;
    p->ntd = (int32_t)cdiv(A.O, tod);
    p->nth = (int32_t)cdiv(B.O, toh);
    p->ntw = (int32_t)cdiv(Cw.O, tow);
    p->full_h = full_h;
    p->full_w = full_w;
    p->ntiles = g.planes * p->ntd * p->nth * p->ntw;
    p->split = TileSplit::make(g.planes, p->ntd, p->nth, p->ntw);
    p->tab_bytes = (uint32_t)tab;
    p->part_bytes = (uint32_t)part;
    p->lds_bytes = (uint32_t)lds;
    return true;
}

// The window shapes with a compiled kernel: 2x2x2 / stride 2 and
// 3x3x3 / stride 2, the two fixed-window workloads' shapes, with no padding
// or one position of padding per side (dilation 1).  Along w a tap past the
// end needs the padding column of that axis (the plan then checks that the
// row's last group lies wholly past the end); along d and h the row clamp
// covers both ends.
bool fixed_shape_supported(const Geom &g)
{
    const Axis &a = g.ax[0], &b = g.ax[1], &c = g.ax[2];
    if (!a.k || a.k != b.k || a.k != c.k || a.s != b.s || a.s != c.s) return false;
    if (!((a.k == 2 && a.s == 2) || (a.k == 3 && a.s == 2))) return false;
    for (int i = 0; i < 3; ++i)
        if (g.ax[i].dil != 1 || g.ax[i].pad > 1) return false;
    if (g.plain()) return true;
    return c.pad == 1 || (int64_t)(c.O - 1) * c.s - c.pad + c.k <= c.X;
}

bool plan_fixed(const Geom &g, int es, const void *x, const void *y, const void *idx,
                FixedPlan *p)
{
    if (!fixed_shape_supported(g)) return false;
    const Axis &c = g.ax[2];
    const int64_t W = c.X, V = FixedPlan::V;
    const int64_t ve = 16 / es;                     // elements per 16-byte vector
    const int64_t span = (V - 1) * c.s + c.k;       // input columns per thread
    const int64_t G = cdiv(c.O, V);
    const int64_t pw = c.pad;
    // vectors per row: with a left padding column the own vectors cover the
    // rest of the span and end where the next group's start
    const int64_t nv = pw ? cdiv(span - pw, ve) : span / ve;
    if ((W * es) % 16 || (uintptr_t)x % 16 || (V * c.s * es) % 16) return false;
    if (pw && nv * ve != V * c.s) return false;
    // vectors stay in the row, but for the last group under a padding column
    // when it starts exactly at the row end (its columns are all padding)
    const int64_t last = (G - 1) * V * c.s;
    if (last + nv * ve > W && !(pw && last == W)) return false;
    // without the padding column no tap may fall past the row end
    if (!pw && (c.O - 1) * c.s - c.pad + c.k > W) return false;
    const int64_t n = g.planes * g.ax[0].O * g.ax[1].O * G;
    if (n >= ((int64_t)1 << 31)) return false;
    p->g = g;
    p->G = (int32_t)G;
    p->groups = FastDiv((uint32_t)G);
    p->oh = FastDiv((uint32_t)g.ax[1].O);
    p->od = FastDiv((uint32_t)g.ax[0].O);
    p->nthreads = (uint32_t)n;
    p->nrows = (uint32_t)(g.planes * g.ax[0].O * g.ax[1].O);
    p->vec_store = (c.O % V == 0) && ((uintptr_t)y % (V * es) == 0) && ((uintptr_t)idx % 16 == 0);
    const bool spill = !pw && span % ve != 0;   // columns beyond the thread's vectors
    p->pd = g.ax[0].pad;
    p->ph = g.ax[1].pad;
    p->pw = (int32_t)pw;
    // Windows that spill read the next group's columns across lanes, and a
    // left padding column the previous group's: give each wave whole rows
    // so that lane is in the same wave, and stage the wave's outputs to
    // write them as vectors.
    p->rpw = ((spill || pw) && G <= 64 && (uintptr_t)y % 16 == 0 && (uintptr_t)idx % 16 == 0)
                 ? (int32_t)(64 / G) : 0;
    // the last group of a row needs its spill columns when its last output
    // exists; without whole rows per wave, lane 63 needs them too
    p->spill_load = spill && (c.O % V == 0 || p->rpw == 0);
    if (p->rpw > 0) p->groups = FastDiv((uint32_t)G);
    return true;
}

bool plan_col(const Geom &g, int es, const void *x, ColPlan *p)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    const int64_t HW = (int64_t)B.X * Cw.X;
    // keys hold the offset in the slice in 24 bits
    if ((HW * es) % 16 || (uintptr_t)x % 16 || HW >= ((int64_t)1 << 24)) return false;
    // widest window along D (all windows of a fixed axis have width k)
    int64_t maxkd = A.k;
    if (!A.k) {
        if (A.O > 4096) return false;
        for (int32_t o = 0; o < A.O; ++o) maxkd = std::max<int64_t>(maxkd, A.end(o) - A.start(o));
    }
    if (maxkd > 8) return false;
    const int64_t cap = std::min<int64_t>(kLdsCap, (int64_t)lds_limit());
    const int64_t tab = ((int64_t)(B.O + Cw.O) * 8 + 15) & ~(int64_t)15;
    if (tab > 16 * 1024) return false;
    // per output slice: D-partial value (binary32, or binary64 for float64)
    // + d offset
    const int64_t ab = es == 8 ? 8 : 4;
    const int64_t per_slice = HW * (ab + 1) + 16;
    int32_t tod = (int32_t)std::min<int64_t>(A.O, (cap - tab) / per_slice);
    if (tod < 1) return false;
    const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
    tod = std::min<int32_t>(tod, (int32_t)std::max<int64_t>(1, A.O / per_plane));
    // at most two output slices per tile: measured on the adaptive f32
    // workload (5 output slices of 16), 103 us with tiles of 2, 2, 1 against
    // 107 with one tile of 5, 107 with 3 + 2 and 110 with 5 tiles of 1
    tod = balance(A.O, std::min<int32_t>(tod, kColMaxTod));
    const int64_t ntd = cdiv(A.O, tod);
    const int64_t ntiles = g.planes * ntd;
    if (ntiles >= ((int64_t)1 << 31) || (int64_t)tod * B.O * Cw.O >= ((int64_t)1 << 31))
        return false;
    p->g = g;
    p->tod = tod;
    p->ntd = (int32_t)ntd;
    p->ntd_div = FastDiv((uint32_t)ntd);
    p->ow_div = FastDiv((uint32_t)Cw.O);
    p->oh_div = FastDiv((uint32_t)B.O);
    p->ntiles = (uint32_t)ntiles;
    p->maxkd = (int32_t)maxkd;
    p->khw = (int32_t)std::min<int64_t>(std::max(max_taps(B), max_taps(Cw)), 1 << 20);
    p->tab_bytes = (uint32_t)tab;
    p->pv_bytes = (uint32_t)(((int64_t)tod * HW * ab + 15) & ~(int64_t)15);
    p->lds_bytes = (uint32_t)(tab + p->pv_bytes + (int64_t)tod * HW);
    return true;
}

// Most windows that contain one position of the axis: 1 or 2, or 0 when
// it may be more.
static int32_t axis_cover(const Axis &a)
{
    if (a.k) return a.ext <= a.s ? 1 : a.ext <= 2 * a.s ? 2 : 0;
    if (a.O > 65536) return 0;
    int32_t c = 1;
    for (int32_t o = 0; o + 1 < a.O; ++o) {
        if (a.end(o) > a.start(o + 1)) c = 2;
        if (o + 2 < a.O && a.end(o) > a.start(o + 2)) return 0;
    }
    return c;
}

static int64_t axis_widest(const Axis &a)
{
    if (a.k) return a.k;
    if (a.O > 65536) return (int64_t)1 << 31;
    int64_t m = 0;
    for (int32_t o = 0; o < a.O; ++o) m = std::max<int64_t>(m, a.end(o) - a.start(o));
    return m;
}

bool plan_small_forward(const Geom &g, SmallPlan *p)
{
    const int64_t total = g.planes * (int64_t)g.out_plane;
    if (total > kSmallFwd) return false;
    for (int a = 0; a < 3; ++a)
        if (axis_widest(g.ax[a]) > kSmallK) return false;
    p->g = g;
    p->total = (uint32_t)total;
    p->plane_div = FastDiv((uint32_t)g.out_plane);
    p->a2_div = FastDiv((uint32_t)g.ax[2].O);
    p->a1_div = FastDiv((uint32_t)g.ax[1].O);
    return true;
}

bool plan_small_backward(const Geom &g, SmallPlan *p)
{
    const int64_t total = g.planes * (int64_t)g.in_plane;
    if (total > kSmallBwd) return false;
    for (int a = 0; a < 3; ++a)
        if (!axis_cover(g.ax[a])) return false;
    p->g = g;
    p->total = (uint32_t)total;
    p->plane_div = FastDiv((uint32_t)g.in_plane);
    p->a2_div = FastDiv((uint32_t)g.ax[2].X);
    p->a1_div = FastDiv((uint32_t)g.ax[1].X);
    return true;
}

// Most windows that contain one position of the axis (0: not known, an
// adaptive axis with too many windows to scan).  The count only grows at
// a window start, so scanning the starts is enough.
static int32_t axis_depth(const Axis &a)
{
    if (a.k) return (int32_t)std::min<int64_t>(cdiv(a.ext, a.s), a.O);
    if (a.O > (1 << 20)) return 0;
    int32_t m = 1;
    for (int32_t o = 0; o < a.O; ++o) {
        const int32_t x = a.start(o);
        m = std::max(m, a.last_starting(x) - a.first_reaching(x) + 1);
    }
    return m;
}

// Most windows (output slices) reaching one slab of td slices.
static int64_t slab_reach(const Axis &a, int32_t td)
{
    int64_t m = 0;
    for (int32_t d0 = 0; d0 < a.X; d0 += td) {
        const int32_t d1 = std::min(d0 + td, a.X);
        m = std::max<int64_t>(m, a.last_starting(d1 - 1) + 1 - a.first_reaching(d0));
    }
    return m;
}

bool plan_backward(const Geom &g, bool ordered, int cell_bytes, BwdPlan *p)
{
    const int32_t D = g.ax[0].X, H = g.ax[1].X, W = g.ax[2].X;
    const int64_t budget = std::min<int64_t>(ordered ? kOrdBudget : kAccBudget,
                                             (int64_t)lds_limit() - 64);
    const int64_t cb = cell_bytes;
    const int64_t slice = (int64_t)H * W * cb;
    p->g = g;
    if (slice <= budget) {
        int32_t td = (int32_t)std::min<int64_t>(D, budget / slice);
        const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
        td = std::min<int32_t>(td, (int32_t)std::max<int64_t>(1, D / per_plane));
        p->td = (int32_t)cdiv(D, cdiv(D, td));
        p->th = H;
        p->tw = W;
    } else if ((int64_t)W * cb <= budget) {
        p->td = 1;
        const int32_t th = (int32_t)std::min<int64_t>(H, budget / ((int64_t)W * cb));
        p->th = (int32_t)cdiv(H, cdiv(H, th));
        p->tw = W;
    } else {
        p->td = 1;
        p->th = 1;
        const int32_t tw = (int32_t)std::min<int64_t>(W, budget / cb);
        p->tw = (int32_t)cdiv(W, cdiv(W, tw));
    }
    p->nphase = 0;
    p->md = p->mh = p->mw = 0;
    if (ordered) {
        if (!(p->th == H && p->tw == W)) return false;
        // the kernel ranks in 32 bits, and a rank counts windows between the
        // first one reaching a position and the window itself: all of them
        // contain the position only when windows are contiguous
        for (int a = 0; a < 3; ++a)
            if ((!g.ax[a].k && !g.ax[a].fast) || g.ax[a].dil != 1) return false;
        const Axis &A = g.ax[0];
        const int32_t md = axis_depth(A), mh = axis_depth(g.ax[1]), mw = axis_depth(g.ax[2]);
        if (!md || !mh || !mw || (int64_t)md * mh * mw > kMaxPhase) return false;
        if (D > (1 << 20)) return false;             // bounds the slab scans below
        // every window reaching a slab must fit one round of the workgroup
        const int64_t ohw = (int64_t)g.ax[1].O * g.ax[2].O;
        const int64_t cap = (int64_t)kOrdRound * kOrdThreads;
        int32_t td = p->td;
        while (td > 1 && slab_reach(A, td) * ohw > cap) td = (int32_t)cdiv(D, cdiv(D, td - 1));
        if (slab_reach(A, td) * ohw > cap) return false;
        p->td = td;
        p->nphase = md * mh * mw;
        p->md = md;
        p->mh = mh;
        p->mw = mw;
        p->hw_div = FastDiv((uint32_t)(H * W));
        p->w_div = FastDiv((uint32_t)W);
        p->ohw_div = FastDiv((uint32_t)ohw);
        p->ow_div = FastDiv((uint32_t)g.ax[2].O);
    }
    p->ntd = (int32_t)cdiv(D, p->td);
    p->nth = (int32_t)cdiv(H, p->th);
    p->ntw = (int32_t)cdiv(W, p->tw);
    p->ntiles = g.planes * p->ntd * p->nth * p->ntw;
    p->split = TileSplit::make(g.planes, p->ntd, p->nth, p->ntw);
    p->slab = p->th == H && p->tw == W;
    // + alignment shift and the rounding of the zero fill to 16 bytes
    p->lds_bytes = (uint32_t)(((int64_t)p->td * p->th * p->tw + 8) * cb);
    return true;
}

// Owner-gather backward: slabs of whole slices.  LDS per slab: the staged
// slab (storage type, plus the alignment shift) and the idx and gy tables
// of the windows reaching it.  The largest slab within the budget that
// still gives enough slabs to fill the chip; MP3D_OWNER_SLICES and
// MP3D_OWNER_THREADS override the slab depth and the workgroup size
// (tuning sweeps).
bool plan_owner(const Geom &g, int es, OwnerPlan *p)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    if (A.X > (1 << 20)) return false;                 // bounds the slab scans below
    const int32_t md = axis_depth(A), mh = axis_depth(B), mw = axis_depth(Cw);
    // positions in many windows make each owner's enumeration long
    if (!md || !mh || !mw || (int64_t)md * mh * mw > kOwnerMaxCand) return false;
    const int64_t HW = (int64_t)B.X * Cw.X, ohw = (int64_t)B.O * Cw.O;
    const int64_t ve = 16 / es;
    const int64_t budget = std::min<int64_t>(kOwnerBudget, (int64_t)lds_limit() - 64);
    auto r16 = [](int64_t b) { return (b + 15) & ~(int64_t)15; };
    auto lds = [&](int32_t td, int64_t *st, int64_t *ti) -> int64_t {
        const int64_t maxw = slab_reach(A, td) * ohw;
        *st = r16((td * HW + ve) * es);
        *ti = r16(maxw * 4);
        return *st + *ti + r16(maxw * es);
    };
    int64_t st = 0, ti = 0;
    const char *ev = getenv("MP3D_OWNER_SLICES");
    int32_t td = 0;
    if (ev && atoi(ev) > 0) {
        td = std::min<int32_t>(atoi(ev), A.X);
        if (lds(td, &st, &ti) > (int64_t)lds_limit() - 64) return false;
    } else {
        const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
        const int32_t cap = (int32_t)std::max<int64_t>(1, A.X / per_plane);
        for (int32_t t = std::min<int32_t>(A.X, cap); t >= 1; --t)
            if (lds(t, &st, &ti) <= budget) { td = t; break; }
        if (td < 1) return false;
        td = (int32_t)cdiv(A.X, cdiv(A.X, td));        // even slabs need no more LDS
    }
    const int64_t total = lds(td, &st, &ti);
    const int64_t ntd = cdiv(A.X, td);
    p->g = g;
    p->td = td;
    p->ntd = (int32_t)ntd;
    p->ntd_div = FastDiv((uint32_t)ntd);
    p->ntiles = g.planes * ntd;
    p->fast = p->ntiles < ((int64_t)1 << 31);
    // 512 threads where a slab has many windows to resolve, else 256
    // (measured: 3645 windows per slab of the 3x3x3/2 f16 workload, 245 of
    // the adaptive f32 one)
    const char *et = getenv("MP3D_OWNER_THREADS");
    const int64_t maxw = slab_reach(A, td) * ohw;
    p->threads = (et && atoi(et) == 256) ? 256 : (et && atoi(et) == 512) ? 512
                 : maxw >= 2048 ? 512 : 256;
    p->st_bytes = (uint32_t)st;
    p->ti_bytes = (uint32_t)ti;
    p->lds_bytes = (uint32_t)total;
    p->hw_div = FastDiv((uint32_t)HW);
    p->w_div = FastDiv((uint32_t)Cw.X);
    p->depth2 = md <= 2 && mh <= 2 && mw <= 2;
    return true;
}

bool plan_rc(const Geom &g, int es, int ab, const void *x, RcPlan *p)
{
    const Axis &A = g.ax[0], &B = g.ax[1], &Cw = g.ax[2];
    if (!g.contiguous() || A.X > 4096) return false;
    const int64_t HW = (int64_t)B.X * Cw.X;
    // the column stages: 16-byte column groups, keys of 24 bits, windows at
    // most 8 wide along D
    if ((HW * es) % 16 || (uintptr_t)x % 16 || HW >= ((int64_t)1 << 24)) return false;
    const int64_t maxkd = A.k ? A.k : axis_widest(A);
    if (maxkd > 8) return false;
    const int64_t ohw = (int64_t)B.O * Cw.O;
    const int64_t tab = ((int64_t)(B.O + Cw.O) * 8 + 15) & ~(int64_t)15;
    if (tab > 16 * 1024) return false;
    const int64_t budget = std::min<int64_t>(kAccBudget, (int64_t)lds_limit() - 64 - tab);
    auto r16 = [](int64_t b) { return (b + 15) & ~(int64_t)15; };
    // LDS of slabs of td slices: the larger of the D-partials of the output
    // slices reaching a slab (value + d offset) and the slab's accumulator
    // (+ alignment shift); 0 when some slab's windows exceed one round
    int64_t cdmax = 0;
    auto region = [&](int32_t td) -> int64_t {
        cdmax = 0;
        for (int32_t d0 = 0; d0 < A.X; d0 += td) {
            const int32_t d1 = std::min(d0 + td, A.X);
            const int64_t cd = (int64_t)A.last_starting(d1 - 1) + 1 - A.first_reaching(d0);
            cdmax = std::max(cdmax, cd);
        }
        if (cdmax * ohw > (int64_t)kRcSlots * kBlock) return 0;
        // partials: one packed word for 16-bit storage, else value + d byte
        const int64_t part = es == 2 ? r16(cdmax * HW * 4) : r16(cdmax * HW * ab) + cdmax * HW;
        return std::max(part, r16(((int64_t)td * HW + 8) * ab));
    };
    const int64_t per_plane = cdiv(kWantTiles, std::max<int64_t>(g.planes, 1));
    int32_t td = (int32_t)std::min<int64_t>(A.X, std::max<int64_t>(1, A.X / per_plane));
    int64_t rb = 0;
    for (; td >= 1; --td) {
        rb = region(td);
        if (rb > 0 && rb <= budget) break;
    }
    if (td < 1) return false;
    // even slabs: fewer slices per slab never need more LDS
    td = (int32_t)cdiv(A.X, cdiv(A.X, td));
    rb = region(td);
    if (rb <= 0 || rb > budget) return false;
    const int64_t ntd = cdiv(A.X, td);
    if (g.planes * ntd >= ((int64_t)1 << 31)) return false;
    p->g = g;
    p->td = td;
    p->ntd = (int32_t)ntd;
    p->ntd_div = FastDiv((uint32_t)ntd);
    p->ntiles = (uint32_t)(g.planes * ntd);
    p->maxkd = (int32_t)maxkd;
    p->ow_div = FastDiv((uint32_t)Cw.O);
    p->oh_div = FastDiv((uint32_t)B.O);
    p->tab_bytes = (uint32_t)tab;
    p->lds_bytes = (uint32_t)(tab + rb);
    p->slots = (int32_t)cdiv(cdmax * ohw, kBlock);
    p->small3 = maxkd <= 3 && max_taps(B) <= 3 && max_taps(Cw) <= 3;
    return true;
}

int64_t max_taps(const Axis &a)
{
    return a.k ? (int64_t)a.k : axis_widest(a);
}

void plan_ex(const Geom &g, ExPlan *p)
{
    p->g = g;
    p->total = g.planes * (int64_t)g.out_plane;
    p->km = 3;
    for (int a = 0; a < 3; ++a)
        if (max_taps(g.ax[a]) > 3) p->km = 0;
    p->fast32 = p->total < ((int64_t)1 << 31);
    p->plane_div = FastDiv((uint32_t)g.out_plane);
    p->ow_div = FastDiv((uint32_t)g.ax[2].O);
    p->oh_div = FastDiv((uint32_t)g.ax[1].O);
}

void plan_gather(const Geom &g, GatherPlan *p)
{
    constexpr int V = 4;                       // windows per thread (kGatherV)
    p->g = g;
    p->qd = g.ax[0].X / g.ax[0].O;
    p->qh = g.ax[1].X / g.ax[1].O;
    p->qw = g.ax[2].X / g.ax[2].O;
    const int64_t G = cdiv(g.ax[2].O, V);
    const int64_t threads = g.planes * g.ax[0].O * g.ax[1].O * G;
    p->fast = threads < ((int64_t)1 << 31);
    p->grp_div = FastDiv((uint32_t)G);
    p->oh_div = FastDiv((uint32_t)g.ax[1].O);
    p->od_div = FastDiv((uint32_t)g.ax[0].O);
    p->vec_in = 0;                             // set by the launcher (pointer alignment)
    p->nc = 0;                                 // set by the chunk kernel's launcher
    p->fast_col = 0;
    p->w_div = FastDiv((uint32_t)g.ax[2].X);
    p->qh_div = FastDiv((uint32_t)p->qh);
    int64_t grid = std::min<int64_t>(cdiv(threads, kBlock), kMaxGrid);
    if (grid >= 64) grid = (grid + 7) & ~(int64_t)7;
    p->grid = (uint32_t)std::max<int64_t>(grid, 1);
}

void plan_ordered(const Geom &g, OrdPlan *p)
{
    p->g = g;
    p->total = g.planes * (int64_t)g.in_plane;
    p->a2_div = FastDiv((uint32_t)g.ax[2].X);
    p->a1_div = FastDiv((uint32_t)g.ax[1].X);
}

}  // namespace mp3d
