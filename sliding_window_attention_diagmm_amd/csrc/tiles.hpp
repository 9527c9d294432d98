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

}  // namespace diagmm
