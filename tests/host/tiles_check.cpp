// Host check of the tile bookkeeping in csrc/tiles.hpp: the multiply-based divisions and
// the division-free decoder against plain integer division.  Built with g++ by
// tests/test_tiles_host.py; prints "ok" or the first mismatch.
#define __host__
#define __device__
#include "tiles.hpp"

#include <cstdio>
#include <cstdint>
#include <random>
#include <vector>

using namespace diagmm;

static int check_div(uint32_t d, uint32_t n) {
    const Div32 v = make_div32(d);
    if (div32(v, n) != n / d) {
        std::printf("div32 mismatch: %u / %u -> %u (want %u)\n", n, d, div32(v, n), n / d);
        return 1;
    }
    return 0;
}

int main() {
    std::mt19937_64 rng(20261202);
    const uint32_t nmax = 0x7fffffffu;
    std::vector<uint32_t> ds;
    for (uint32_t d = 1; d <= 4096; ++d) ds.push_back(d);
    for (int e = 12; e < 31; ++e)
        for (int o = -2; o <= 2; ++o) ds.push_back(static_cast<uint32_t>((int64_t(1) << e) + o));
    for (int i = 0; i < 2000; ++i) ds.push_back(1 + static_cast<uint32_t>(rng() % nmax));
    ds.push_back(nmax);
    for (uint32_t d : ds) {
        std::vector<uint32_t> ns = {0u, 1u, d - 1, d, d + 1, nmax, nmax - 1, nmax - d + 1};
        for (uint32_t m : {2u, 3u, 1000u, 65537u})
            if (uint64_t(d) * m - 1 <= nmax) {
                ns.push_back(d * m - 1);
                ns.push_back(d * m);
            }
        for (int i = 0; i < 40; ++i) ns.push_back(static_cast<uint32_t>(rng() % (uint64_t(nmax) + 1)));
        for (uint32_t n : ns)
            if (n <= nmax && check_div(d, n)) return 1;
    }
    // decode_fast / class_len_fast / unit_range / unit_seq against the reference forms
    struct Case { int64_t b, n, h, K, s, rows, slots, nwg; };
    const Case cases[] = {{1, 4096, 12, 513, 1, 64, 513, 256}, {1, 4096, 12, 513, 3, 64, 513, 256},
                          {2, 1000, 3, 97, 7, 32, 40, 37},   {3, 5, 2, 9, 9, 64, 513, 8},
                          {1, 130, 5, 601, 2, 64, 300, 1},  {4, 77, 7, 33, 100, 32, 16, 250}};
    for (const Case& c : cases) {
        const TileGrid g = make_grid(c.b, c.n, c.h, c.K, c.s, c.rows, c.slots);
        const int64_t nwg = c.nwg < g.tiles ? c.nwg : g.tiles;
        const TileDecode dc = make_decode(g, c.h, c.n, c.s, g.tiles, nwg);
        for (int64_t t = 0; t < g.tiles; ++t) {
            const TileId a = decode_tile(g, c.h, static_cast<uint32_t>(t));
            const TileId f = decode_fast(dc, static_cast<uint32_t>(t));
            if (a.bb != f.bb || a.hh != f.hh || a.r != f.r || a.kb != f.kb || a.tb != f.tb) {
                std::printf("decode mismatch at tile %lld\n", (long long)t);
                return 1;
            }
            if (class_len(c.n, c.s, a.r) != class_len_fast(dc, a.r)) {
                std::printf("class_len mismatch r=%d\n", a.r);
                return 1;
            }
        }
        uint32_t expect = 0;
        for (uint32_t r = 0; r < static_cast<uint32_t>(nwg); ++r) {
            uint32_t b, e;
            unit_range(dc, r, &b, &e);
            const uint32_t len = e - b;
            if (b != expect || len + 1 < g.tiles / nwg + 1 || len > g.tiles / nwg + 1) {
                std::printf("unit_range bad at rank %u: [%u, %u)\n", r, b, e);
                return 1;
            }
            expect = e;
        }
        if (expect != g.tiles) {
            std::printf("unit_range covers %u of %lld\n", expect, (long long)g.tiles);
            return 1;
        }
        // unit_seq, interleaved and contiguous: every unit exactly once, each XCD's units
        // a contiguous range shared out to +-1 among its workgroups
        for (bool il : {true, false}) {
            std::vector<int> seen(static_cast<size_t>(g.tiles), 0);
            for (uint32_t wg = 0; wg < static_cast<uint32_t>(nwg); ++wg) {
                uint32_t f, cnt, st;
                unit_seq(dc, wg, static_cast<uint32_t>(nwg), il, &f, &cnt, &st);
                for (uint32_t m = 0; m < cnt; ++m) {
                    const uint64_t u = f + uint64_t(m) * st;
                    if (u >= static_cast<uint64_t>(g.tiles) || seen[u]++) {
                        std::printf("unit_seq bad at wg %u (interleave %d)\n", wg, int(il));
                        return 1;
                    }
                }
                if (il && nwg % kXcds == 0) {
                    const uint64_t lo = uint64_t(g.tiles) * (wg % kXcds) / kXcds;
                    const uint64_t hi = uint64_t(g.tiles) * (wg % kXcds + 1) / kXcds;
                    const uint64_t per = nwg / kXcds, span = hi - lo;
                    if (cnt < span / per || cnt > span / per + 1 || (cnt && (f < lo || f >= hi))) {
                        std::printf("unit_seq unbalanced at wg %u\n", wg);
                        return 1;
                    }
                }
            }
            for (int64_t t = 0; t < g.tiles; ++t)
                if (seen[t] != 1) {
                    std::printf("unit_seq misses unit %lld (interleave %d)\n", (long long)t, int(il));
                    return 1;
                }
        }
    }
    // the strip split (g workgroups per strip of whole tiles), contiguous and interleaved:
    // every unit exactly once, each workgroup's units inside one strip, counts within one
    // (g x strips <= nwg, as the planner picks g)
    struct SCase { int64_t b, n, h, K, s, nwg, g; };
    const SCase scases[] = {{1, 4096, 12, 513, 3, 256, 7}, {2, 1100, 2, 169, 2, 24, 3},
                            {1, 300, 3, 65, 4, 24, 2}, {1, 640, 1, 33, 1, 7, 7}};
    for (const SCase& c : scases) {
        const TileGrid g = make_grid(c.b, c.n, c.h, c.K, c.s, 64, c.K);
        const int64_t per_strip = g.rb, strips = g.tiles / per_strip;
        TileDecode dc = make_decode(g, c.h, c.n, c.s, g.tiles, c.nwg);
        set_strip_split(&dc, strips, per_strip, c.g);
        for (bool il : {true, false}) {
            std::vector<int> seen(static_cast<size_t>(g.tiles), 0);
            for (uint32_t wg = 0; wg < static_cast<uint32_t>(c.nwg); ++wg) {
                uint32_t f, cnt, st;
                unit_seq(dc, wg, static_cast<uint32_t>(c.nwg), il, &f, &cnt, &st);
                const uint64_t want = per_strip / c.g;
                if (cnt && (cnt < want || cnt > want + 1)) {
                    std::printf("strip unit_seq unbalanced at wg %u\n", wg);
                    return 1;
                }
                for (uint32_t m = 0; m < cnt; ++m) {
                    const uint64_t u = f + uint64_t(m) * st;
                    if (u >= static_cast<uint64_t>(g.tiles) || seen[u]++ ||
                        u / per_strip != f / per_strip) {
                        std::printf("strip unit_seq bad at wg %u (interleave %d)\n", wg, int(il));
                        return 1;
                    }
                }
            }
            for (int64_t t = 0; t < g.tiles; ++t)
                if (seen[t] != 1) {
                    std::printf("strip unit_seq misses unit %lld (interleave %d)\n",
                                (long long)t, int(il));
                    return 1;
                }
        }
    }
    std::printf("ok\n");
    return 0;
}
