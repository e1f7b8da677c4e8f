// Host-side check of the library's geometry helpers (geometry.hpp): the
// multiply-high divisions against plain integer division, the fast and
// 64-bit paths of every window function against each other, and the tile
// split against div/mod.  Built with hipcc as host code; launches nothing.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../../bwd_max_pool3d_amd/csrc/geometry.hpp"

using mp3d::Axis;
using mp3d::FastDiv;
using mp3d::TileSplit;

static int fails = 0;
#define EXPECT(c)                                                         \
    do {                                                                  \
        if (!(c) && fails++ < 20) std::printf("FAIL line %d: %s\n", __LINE__, #c); \
    } while (0)

int main()
{
    std::mt19937_64 rng(5);
    // divisors: small, powers of two and neighbours, random, the largest
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d < 4096; ++d) ds.push_back(d);
    for (int b = 1; b < 31; ++b) {
        ds.push_back(1u << b);
        ds.push_back((1u << b) - 1);
        ds.push_back((1u << b) + 1);
    }
    for (int i = 0; i < 2000; ++i) ds.push_back((uint32_t)(rng() % 0x7fffffffu) + 1);
    ds.push_back(0x7fffffffu);
    for (uint32_t d : ds) {
        FastDiv f(d);
        const uint32_t ns[] = {0u, 1u, d - 1, d, d + 1, 2 * d - 1, 0x7ffffffeu, 0x7fffffffu};
        for (uint32_t n : ns)
            if (n < 0x80000000u) EXPECT(f.div(n) == n / d);
        for (int i = 0; i < 200; ++i) {
            const uint32_t n = (uint32_t)(rng() & 0x7fffffffu);
            EXPECT(f.div(n) == n / d);
        }
    }
    // window functions: fast path == 64-bit path
    for (int32_t X = 1; X <= 80; ++X) {
        for (int32_t O = 1; O <= 80; ++O) {
            Axis a = Axis::make(X, O, 0, 0);
            Axis b = a;
            b.fast = 0;
            EXPECT(a.fast);
            for (int32_t o = 0; o < O; ++o) {
                EXPECT(a.start(o) == b.start(o));
                EXPECT(a.end(o) == b.end(o));
            }
            for (int32_t p = 0; p < X; ++p) {
                EXPECT(a.first_reaching(p) == b.first_reaching(p));
                EXPECT(a.last_starting(p) == b.last_starting(p));
                // every window containing p lies in [first_reaching, last_starting]
                for (int32_t o = 0; o < O; ++o) {
                    const bool in = a.start(o) <= p && p < a.end(o);
                    if (in) EXPECT(o >= a.first_reaching(p) && o <= a.last_starting(p));
                }
            }
        }
    }
    for (int32_t k = 1; k <= 6; ++k)
        for (int32_t s = 1; s <= 6; ++s)
            for (int32_t X = k; X <= 60; ++X) {
                const int32_t O = (X - k) / s + 1;
                Axis a = Axis::make(X, O, k, s);
                for (int32_t p = 0; p < X; ++p) {
                    const int32_t lo = p < k ? 0 : (p - k) / s + 1;
                    EXPECT(a.first_reaching(p) == lo);
                    EXPECT(a.last_starting(p) == std::min(p / s, O - 1));
                    for (int32_t o = 0; o < O; ++o) {
                        const bool in = a.start(o) <= p && p < a.end(o);
                        if (in) EXPECT(o >= a.first_reaching(p) && o <= a.last_starting(p));
                    }
                }
            }
    // a large adaptive axis takes the 64-bit path
    Axis big = Axis::make(2000000000, 7, 0, 0);
    EXPECT(!big.fast);
    EXPECT(big.end(6) == 2000000000);
    // tile split
    TileSplit ts = TileSplit::make(1000, 7, 3, 5);
    for (int64_t t = 0; t < 1000 * 7 * 3 * 5; t += 7) {
        int64_t plane;
        int32_t i0, i1, i2;
        ts.split(t, &plane, &i0, &i1, &i2);
        EXPECT(i2 == t % 5 && i1 == (t / 5) % 3 && i0 == (t / 15) % 7 && plane == t / 105);
    }
    std::printf(fails ? "geometry: %d failures\n" : "geometry: ok\n", fails);
    return fails ? 1 : 0;
}
