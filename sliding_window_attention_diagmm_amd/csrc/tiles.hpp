// Tile geometry of the band-tile scheduler, shared by the host planner and the kernels.
//
// Dilation.  With stride s, slot k of row i reads key i + (k - w) s, so rows and keys of
// one residue class i = r (mod s) only meet each other: class r is an undilated band
// problem on the sub-sequence t -> r + s t of length n_r = ceil((n - r) / s).  Tiles are
// therefore cut inside one residue class, and a tile's key window is a contiguous run
// of that class (rows r + s t, stride s rows in memory) - the 128-byte key rows stay
// whole cache lines at every dilation.
//
// Tile order.  Tile ids run over (batch, head, residue, row block, slot block) with the
// slot block fastest.  Neighbouring ids share most of their key window.
//
// XCD placement.  Workgroup ids are handed to the 8 XCDs round-robin (id mod 8).  The
// kernels remap id -> tile so that each XCD owns one contiguous range of tile ids, and
// with it a contiguous range of heads and rows whose key windows stay in its own L2.
#pragma once

#include <stdint.h>

namespace diagmm {

constexpr int kXcds = 8;

struct TileGrid {
    int64_t s;          // stride (residue classes)
    int64_t rb;         // row blocks per residue class (of the longest class)
    int64_t nkb;        // slot blocks
    int64_t kb;         // slots per slot block (the last one may be shorter)
    int64_t tiles;      // b * h * s * rb * nkb
    int64_t per_xcd;    // tiles owned by each XCD (grid = per_xcd * kXcds workgroups)
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Slot blocks: as few as the per-tile slot limit allows, then balanced.
__host__ __device__ inline TileGrid make_grid(int64_t b, int64_t n, int64_t h, int64_t K,
                                              int64_t s, int64_t rows_per_tile,
                                              int64_t max_slots) {
    TileGrid g;
    g.s = s;
    const int64_t longest = ceil_div(n, s);
    g.rb = ceil_div(longest, rows_per_tile);
    g.nkb = ceil_div(K, max_slots);
    g.kb = ceil_div(K, g.nkb);
    g.tiles = b * h * s * g.rb * g.nkb;
    g.per_xcd = ceil_div(g.tiles, kXcds);
    return g;
}

struct TileId {
    int64_t bb, hh, r, tb, kb;
};

// Workgroup id -> tile id (XCD-contiguous ranges); returns false past the last tile.
__host__ __device__ inline bool tile_of(const TileGrid& g, int64_t h, int64_t wg, TileId* t) {
    const int64_t tile = (wg % kXcds) * g.per_xcd + wg / kXcds;
    if (tile >= g.tiles) return false;
    int64_t x = tile;
    t->kb = x % g.nkb;
    x /= g.nkb;
    t->tb = x % g.rb;
    x /= g.rb;
    t->r = x % g.s;
    x /= g.s;
    t->hh = x % h;
    t->bb = x / h;
    return true;
}

// Length of residue class r.
__host__ __device__ inline int64_t class_len(int64_t n, int64_t s, int64_t r) {
    return r < n ? (n - r + s - 1) / s : 0;
}

}  // namespace diagmm
