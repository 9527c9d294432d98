// Tile geometry of the band-tile scheduler, shared by the host planner and the kernels.
//
// Dilation.  With stride s, slot k of row i reads key i + (k - w) s, so rows and keys of
// one residue class i = r (mod s) only meet each other: class r is an undilated band
// problem on the sub-sequence t -> r + s t of length n_r = ceil((n - r) / s).  Tiles are
// therefore cut inside one residue class, and a tile's key window is a contiguous run
// of that class (rows r + s t, stride s rows in memory) - the 128-byte key rows stay
// whole cache lines at every dilation.
//
// Tile order.  Tile ids run over (batch, head, residue, slot block, row block) with the
// row block fastest: consecutive ids form strips that slide down one residue class, each
// tile's key window overlapping the previous one in all but 64 rows.
//
// XCD placement.  Workgroup ids are handed to the 8 XCDs round-robin (id mod 8).  Ranks
// are remapped so that each XCD owns one contiguous range of tile ids, and with it a
// contiguous range of heads and rows whose operands stay in its own L2.
#pragma once

#include <stdint.h>

namespace diagmm {

constexpr int kXcds = 8;

struct TileGrid {
    int64_t res;        // residue classes enumerated: min(s, n) (classes past n are empty)
    int64_t rb;         // row blocks per residue class (of the longest class)
    int64_t nkb;        // slot blocks
    int64_t kb;         // slots per slot block (the last one may be shorter)
    int64_t tiles;      // b * h * res * nkb * rb
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Slot blocks: as few as the per-tile slot limit allows, then balanced.
__host__ __device__ inline TileGrid make_grid(int64_t b, int64_t n, int64_t h, int64_t K,
                                              int64_t s, int64_t rows_per_tile,
                                              int64_t max_slots) {
    TileGrid g;
    g.res = s < n ? s : (n > 0 ? n : 1);
    const int64_t longest = ceil_div(n, s);
    g.rb = ceil_div(longest, rows_per_tile);
    g.nkb = ceil_div(K, max_slots);
    g.kb = ceil_div(K, g.nkb);
    g.tiles = b * h * g.res * g.rb * g.nkb;
    return g;
}

struct TileId {
    int32_t bb, hh, r, kb, tb;
};

// Tile grids are planned with fewer than 2^31 tiles (the planner falls back to the
// element kernels otherwise), so the per-workgroup decode runs in 32-bit arithmetic.
constexpr int64_t kMaxTiles = (int64_t(1) << 31) - 1;

// Tile id -> coordinates (row block fastest).
__host__ __device__ inline TileId decode_tile(const TileGrid& g, int64_t h, uint32_t tile) {
    TileId t;
    uint32_t x = tile;
    const uint32_t nkb = static_cast<uint32_t>(g.nkb), rb = static_cast<uint32_t>(g.rb);
    const uint32_t s = static_cast<uint32_t>(g.res), hu = static_cast<uint32_t>(h);
    t.tb = static_cast<int32_t>(x % rb);
    x /= rb;
    t.kb = static_cast<int32_t>(x % nkb);
    x /= nkb;
    t.r = static_cast<int32_t>(x % s);
    x /= s;
    t.hh = static_cast<int32_t>(x % hu);
    t.bb = static_cast<int32_t>(x / hu);
    return t;
}

// Persistent workgroup wg of nwg -> its rank, with ranks contiguous per XCD.
__host__ __device__ inline uint32_t xcd_rank(uint32_t wg, uint32_t nwg) {
    if (nwg % kXcds != 0) return wg;
    return (wg % kXcds) * (nwg / kXcds) + wg / kXcds;
}

// Tile range [begin, end) of rank `rank` among nwg workgroups (balanced to +-1).
__host__ __device__ inline void tile_range(int64_t tiles, uint32_t rank, uint32_t nwg,
                                           int64_t* begin, int64_t* end) {
    *begin = tiles * rank / nwg;
    *end = tiles * (rank + 1) / nwg;
}

// Length of residue class r.
__host__ __device__ inline int64_t class_len(int64_t n, int64_t s, int64_t r) {
    return r < n ? (n - r + s - 1) / s : 0;
}

// Exact n / d for 0 <= n < 2^31 and 1 <= d < 2^31 by one multiply: with
// 2^(sh-1) < d <= 2^sh, k = 32 + sh and m = floor(2^k / d) + 1, m d = 2^k + e with
// 0 < e <= d, so n m / 2^k = n / d + n e / (d 2^k) and n e < 2^31 2^sh = 2^(k-1) keeps
// the excess below 1/d: the floor is unchanged (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct Div32 {
    uint64_t m;
    uint32_t d, k;
};

inline Div32 make_div32(uint32_t d) {
    uint32_t sh = 0;
    while ((uint64_t(1) << sh) < d) ++sh;
    Div32 v;
    v.d = d;
    v.k = 32 + sh;
    v.m = static_cast<uint64_t>((static_cast<unsigned __int128>(1) << v.k) / d) + 1;
    return v;
}

__host__ __device__ inline uint32_t div32(const Div32& v, uint32_t n) {
    const uint64_t lo = static_cast<uint64_t>(n) * static_cast<uint32_t>(v.m);
    const uint64_t hi = static_cast<uint64_t>(n) * static_cast<uint32_t>(v.m >> 32);
    // (hi << 32) + lo < 2^64: n < 2^31 and m < 2^33
    return static_cast<uint32_t>(((hi << 32) + lo) >> v.k);
}

// Everything a persistent workgroup needs to walk its tiles without a division on the
// device: reciprocals of the grid extents, the residue class lengths (n = q s + m, so
// class r has q + (r < m) rows) and a balanced split of `units` (tiles, or whole tiles
// of several chunks) over the workgroups.
struct TileDecode {
    Div32 rb, nkb, res, h;
    uint32_t cls_q, cls_m;
    uint32_t unit_base, unit_rem;
    // Strip split, used when strip_wgs > 0: the units form strip_count strips of
    // strip_units consecutive ids, and workgroup rank strip * strip_wgs + j takes units of
    // that strip only.  Its first strip_wgs - strip_rem workgroups take strip_q units each
    // and the others one more, so the longer ranges sit at the end of the strip, where its
    // last (possibly short) unit is.  Ranks past the strips get nothing.
    uint32_t strip_wgs, strip_count, strip_units, strip_q, strip_rem;
};

inline TileDecode make_decode(const TileGrid& g, int64_t h, int64_t n, int64_t s,
                              int64_t units, int64_t nwg) {
    TileDecode t;
    t.rb = make_div32(static_cast<uint32_t>(g.rb));
    t.nkb = make_div32(static_cast<uint32_t>(g.nkb));
    t.res = make_div32(static_cast<uint32_t>(g.res));
    t.h = make_div32(static_cast<uint32_t>(h));
    t.cls_q = static_cast<uint32_t>(n / s);
    t.cls_m = static_cast<uint32_t>(n % s);
    t.unit_base = static_cast<uint32_t>(units / nwg);
    t.unit_rem = static_cast<uint32_t>(units % nwg);
    t.strip_wgs = t.strip_count = t.strip_units = t.strip_q = t.strip_rem = 0;
    return t;
}

// Workgroups per strip for the strip split, or 0 for the flat one (units balanced over all
// workgroups to +-1), whichever leaves the busiest workgroup less work.  Strips hold
// `per_strip` units of `unit_rows` rows, the last one `last_rows` rows (a ragged class
// end); a full unit counts 1 and the short one a quarter (its fixed costs: a pass over its
// band rows, the start and end of a tile) plus its share of rows.  The flat split counts
// every unit as full, and is kept unless the strip split saves at least a quarter.
inline int64_t pick_strip_split(int64_t strips, int64_t per_strip, int64_t unit_rows,
                                int64_t last_rows, int64_t nwg) {
    if (strips < 1 || per_strip < 1 || nwg < 1) return 0;
    const int64_t g = nwg / strips;
    if (g < 2 || g > per_strip) return 0;
    const double flat = static_cast<double>(ceil_div(strips * per_strip, nwg));
    const int64_t q = per_strip / g, rem = per_strip % g;
    double last = 0.25 + static_cast<double>(last_rows) / static_cast<double>(unit_rows);
    last = last < 1.0 ? last : 1.0;
    const double split = rem == 0 ? static_cast<double>(q)
                       : rem == 1 ? static_cast<double>(q) + last
                                  : static_cast<double>(q + 1);
    return split + 0.25 <= flat ? g : 0;
}

inline void set_strip_split(TileDecode* t, int64_t strips, int64_t per_strip, int64_t g) {
    t->strip_wgs = static_cast<uint32_t>(g);
    t->strip_count = static_cast<uint32_t>(strips);
    t->strip_units = static_cast<uint32_t>(per_strip);
    t->strip_q = static_cast<uint32_t>(per_strip / g);
    t->strip_rem = static_cast<uint32_t>(per_strip % g);
}

// Tile id -> coordinates, as decode_tile (row block fastest).
__host__ __device__ inline TileId decode_fast(const TileDecode& dc, uint32_t tile) {
    TileId t;
    uint32_t x = tile, y;
    y = div32(dc.rb, x);
    t.tb = static_cast<int32_t>(x - y * dc.rb.d);
    x = y;
    y = div32(dc.nkb, x);
    t.kb = static_cast<int32_t>(x - y * dc.nkb.d);
    x = y;
    y = div32(dc.res, x);
    t.r = static_cast<int32_t>(x - y * dc.res.d);
    x = y;
    y = div32(dc.h, x);
    t.hh = static_cast<int32_t>(x - y * dc.h.d);
    t.bb = static_cast<int32_t>(y);
    return t;
}

__host__ __device__ inline int class_len_fast(const TileDecode& dc, int r) {
    return static_cast<int>(dc.cls_q) + (static_cast<uint32_t>(r) < dc.cls_m ? 1 : 0);
}

// Units [begin, end) of rank `rank`: with the strip split as set out at TileDecode, else
// balanced over all ranks (the first unit_rem ranks take one extra).
__host__ __device__ inline void unit_range(const TileDecode& dc, uint32_t rank,
                                           uint32_t* begin, uint32_t* end) {
    if (dc.strip_wgs != 0) {
        const uint32_t strip = rank / dc.strip_wgs, j = rank - strip * dc.strip_wgs;
        if (strip >= dc.strip_count) {
            *begin = *end = 0;
            return;
        }
        const uint32_t lo = dc.strip_wgs - dc.strip_rem;      // ranges of strip_q units
        *begin = strip * dc.strip_units +
                 (j < lo ? j * dc.strip_q : lo * dc.strip_q + (j - lo) * (dc.strip_q + 1));
        *end = *begin + dc.strip_q + (j < lo ? 0u : 1u);
        return;
    }
    const uint32_t extra = rank < dc.unit_rem ? rank : dc.unit_rem;
    *begin = rank * dc.unit_base + extra;
    *end = *begin + dc.unit_base + (rank < dc.unit_rem ? 1u : 0u);
}

// The units of workgroup wg as an arithmetic sequence first, first + stride, ... (count
// terms).  Interleaved (flat split, nwg a multiple of 8 only): XCD x = wg mod 8 owns the
// units [U x / 8, U (x + 1) / 8) of the U in all, and its j-th workgroup (j = wg / 8) takes
// every (nwg / 8)-th of them from the j-th on, so that at any moment the XCD's workgroups
// hold neighbouring units and read the cache lines those share while they are in its L2.
// Interleaved on the strip split: the j-th workgroup of a strip (ranks taken as in
// unit_range) takes the strip's units j, j + g, j + 2 g, ... (g workgroups per strip), so
// that a strip's neighbouring units run at the same time; a strip's workgroups are
// consecutive XCD ranks, mostly on one XCD.
// Otherwise the contiguous range of unit_range for the workgroup's XCD rank.
__host__ __device__ inline void unit_seq(const TileDecode& dc, uint32_t wg, uint32_t nwg,
                                         bool interleave, uint32_t* first, uint32_t* count,
                                         uint32_t* stride) {
    if (interleave && dc.strip_wgs == 0 && nwg % kXcds == 0) {
        const uint64_t units = static_cast<uint64_t>(dc.unit_base) * nwg + dc.unit_rem;
        const uint32_t x = wg % kXcds, j = wg / kXcds, per = nwg / kXcds;
        const uint32_t lo = static_cast<uint32_t>(units * x / kXcds);
        const uint32_t hi = static_cast<uint32_t>(units * (x + 1) / kXcds);
        *first = lo + j;
        *stride = per;
        *count = lo + j < hi ? (hi - lo - j + per - 1) / per : 0u;
        return;
    }
    if (interleave && dc.strip_wgs != 0) {
        const uint32_t rank = xcd_rank(wg, nwg);
        const uint32_t strip = rank / dc.strip_wgs, j = rank - strip * dc.strip_wgs;
        *stride = dc.strip_wgs;
        if (strip >= dc.strip_count || j >= dc.strip_units) {
            *first = 0;
            *count = 0;
            return;
        }
        *first = strip * dc.strip_units + j;
        *count = (dc.strip_units - j + dc.strip_wgs - 1) / dc.strip_wgs;
        return;
    }
    uint32_t b, e;
    unit_range(dc, xcd_rank(wg, nwg), &b, &e);
    *first = b;
    *count = e - b;
    *stride = 1;
}

}  // namespace diagmm
