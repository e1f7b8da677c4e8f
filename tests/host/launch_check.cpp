// Host-side check of the launch shapes the planners lead to (plan.hip):
// for geometries from one plane to tens of millions of planes, every
// launch of a one-tile-per-workgroup kernel stays within kMaxTileGrid
// workgroups (so workgroups x threads < 2^32 work-items), the launches
// together cover every tile exactly once, and the XCD renumbering of block
// ids is a permutation.  Built with hipcc as host code together with
// plan.hip; launches nothing (the two device queries plan.hip makes are
// answered here with MI355X's figures).
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../bwd_max_pool3d_amd/csrc/kernels.hpp"

namespace mp3d {
size_t lds_limit() { return 160 * 1024; }
int device_cus() { return 256; }
}  // namespace mp3d

using namespace mp3d;

static int fails = 0;
#define EXPECT(c)                                                                  \
    do {                                                                           \
        if (!(c) && fails++ < 20) std::printf("FAIL line %d: %s\n", __LINE__, #c); \
    } while (0)

struct Shape {
    int64_t N, C, D, H, W;
    int32_t od, oh, ow;      // adaptive extents (k == 0), else ignored
    int32_t k, s;            // fixed window on every axis (0: adaptive)
};

static Geom make(const Shape &sh)
{
    Geom g;
    const int64_t X[3] = {sh.D, sh.H, sh.W};
    const int32_t O[3] = {sh.od, sh.oh, sh.ow};
    for (int a = 0; a < 3; ++a)
        g.ax[a] = sh.k ? Axis::make((int32_t)X[a], (int32_t)((X[a] - sh.k) / sh.s + 1), sh.k, sh.s)
                       : Axis::make((int32_t)X[a], O[a], 0, 0);
    g.planes = sh.N * sh.C;
    g.in_plane = g.ax[0].X * g.ax[1].X * g.ax[2].X;
    g.out_plane = g.ax[0].O * g.ax[1].O * g.ax[2].O;
    return g;
}

// The launches of a one-tile-per-workgroup kernel over ntiles tiles, as the
// launchers make them: within the dispatch limit, covering every tile once.
static void check_tiles(int64_t ntiles, int threads)
{
    int64_t covered = 0, launches = 0;
    for (int64_t t0 = 0; t0 < ntiles; t0 += kMaxTileGrid) {
        const uint32_t grid = tile_grid(ntiles, t0);
        EXPECT(grid >= 1 && (int64_t)grid <= kMaxTileGrid);
        EXPECT((uint64_t)grid * (uint64_t)threads < ((uint64_t)1 << 32));
        // blocks whose tile t0 + xcd(b) < ntiles do the work, the rest exit
        int64_t live = 0;
        if (grid <= 4096) {
            for (uint32_t b = 0; b < grid; ++b) live += t0 + xcd_local_block(b, grid) < ntiles;
        } else {
            live = std::min<int64_t>(grid, ntiles - t0);
        }
        EXPECT(live == std::min<int64_t>(kMaxTileGrid, ntiles - t0));
        covered += live;
        ++launches;
    }
    EXPECT(covered == ntiles);
    EXPECT(launches == (ntiles + kMaxTileGrid - 1) / kMaxTileGrid);
}

int main()
{
    // the XCD renumbering is a permutation of the block ids
    for (uint32_t n : {1u, 7u, 8u, 64u, 72u, 1000u, 1024u, 4104u}) {
        std::vector<int> seen(n, 0);
        for (uint32_t b = 0; b < n; ++b) {
            const uint32_t t = xcd_local_block(b, n);
            EXPECT(t < n);
            if (t < n) ++seen[t];
        }
        for (uint32_t t = 0; t < n; ++t) EXPECT(seen[t] == 1);
    }
    const std::vector<Shape> shapes = {
        {2, 3, 8, 8, 8, 4, 4, 4, 0, 0},                // the five named workloads
        {4, 16, 10, 10, 10, 8, 8, 8, 0, 0},
        {16, 64, 16, 112, 112, 0, 0, 0, 2, 2},
        {8, 128, 32, 56, 56, 0, 0, 0, 3, 2},
        {32, 256, 16, 32, 32, 5, 7, 7, 0, 0},
        {4097, 4096, 3, 2, 2, 2, 1, 1, 0, 0},          // 2^24 + 2^12 planes, overlapping on d
        {8192, 1024, 4, 4, 4, 3, 3, 3, 0, 0},          // 2^23 planes
        {1 << 14, 1 << 12, 3, 3, 3, 2, 2, 2, 0, 0},    // 2^26 planes
        {1 << 15, 1 << 13, 2, 2, 2, 0, 0, 0, 2, 1},    // 2^28 planes, fixed k2 s1
        {1, 1, 1 << 12, 64, 64, 0, 0, 0, 3, 2},        // one deep plane
        {1, 1, 256, 1024, 1024, 0, 0, 0, 3, 2},        // slices beyond LDS: boxes
    };
    int planned = 0;
    for (const Shape &sh : shapes) {
        const Geom g = make(sh);
        for (int es : {2, 4, 8}) {
            const int cell = es == 8 ? 8 : 4;
            BwdPlan bp;
            for (bool ordered : {false, true}) {
                if (!plan_backward(g, ordered, cell, &bp)) continue;
                ++planned;
                if (bp.slab) {
                    check_tiles(bp.ntiles, ordered ? kOrdThreads : kSlabThreads);
                } else {
                    EXPECT(std::min<int64_t>(bp.ntiles, kMaxTileGrid) * kBlock < ((int64_t)1 << 32));
                }
            }
            OwnerPlan op;
            if (plan_owner(g, es, &op)) {
                ++planned;
                check_tiles(op.ntiles, op.threads);
                EXPECT(op.threads == 256 || op.threads == 512);
            }
            ColPlan cp;
            // a 16-byte aligned stand-in address: plan_col only checks alignment
            if (plan_col(g, es, (const void *)(uintptr_t)256, &cp)) {
                ++planned;
                check_tiles(cp.ntiles, cp.lds_bytes > kColBigLds ? kColBigThreads : kBlock);
            }
            RcPlan rp;
            if (plan_rc(g, es, cell, (const void *)(uintptr_t)256, &rp)) {
                ++planned;
                check_tiles(rp.ntiles, kBlock);
            }
            FixedPlan fp;
            if (plan_fixed(g, es, (const void *)(uintptr_t)256, (const void *)(uintptr_t)256,
                           (const void *)(uintptr_t)256, &fp)) {
                ++planned;
                // one thread per group of V outputs, fewer than 2^31 of them
                EXPECT((int64_t)fp.nthreads < ((int64_t)1 << 31));
            }
        }
        GatherPlan gp;
        bool tiles = true;
        for (int a = 0; a < 3; ++a)
            tiles = tiles && g.ax[a].X % g.ax[a].O == 0 &&
                    (g.ax[a].k == 0 || (g.ax[a].s == g.ax[a].X / g.ax[a].O && g.ax[a].k <= g.ax[a].s));
        if (tiles) {
            plan_gather(g, &gp);
            ++planned;
            EXPECT((uint64_t)gp.grid * kBlock < ((uint64_t)1 << 32));
        }
    }
    EXPECT(planned > 40);
    if (fails) {
        std::printf("%d failures\n", fails);
        return 1;
    }
    std::printf("launch: ok (%d plans)\n", planned);
    return 0;
}
