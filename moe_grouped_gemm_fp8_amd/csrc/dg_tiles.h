// Tile ranges of the XCD-aware workgroup mapping, shared by the kernels (device code) and the
// host-side coverage test (plain C++): no HIP header is needed to use it.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define DG_HD __host__ __device__
#else
#define DG_HD
#endif

namespace dg {

struct TileRange {
    int first;  // the workgroup's first tile id
    int end;    // one past the last tile id of its XCD's range
    int step;   // stride between the workgroup's tiles (the workgroups of its XCD)
};

// Workgroup ids are dealt round-robin over the 8 XCDs, so XCD x runs ids x, x + 8, ...  The
// first `lead` ids do other work (a multiple of 8, so the XCD of an id does not change); the
// other G = grid - lead workgroups share `total` tile ids: XCD x owns the contiguous range
// [total * w_x / G, total * (w_x + p_x) / G), where p_x is its number of workgroups and w_x
// the number on XCDs before it, and its workgroups stride through that range together, so
// the tiles in flight on one XCD are neighbours.  Every tile id in [0, total) falls to exactly
// one workgroup.  The products are 64-bit: total * (w_x + p_x) reaches total * G, which
// passes 2^31 long before the grid or the tile count does.
// Preconditions: 0 < total < 2^31, lead <= id < grid, grid - lead >= 1, lead % 8 == 0.
DG_HD inline TileRange xcd_tile_range(int64_t total, int grid, int lead, int id)
{
    const int G = grid - lead, bid = id - lead;
    const int q = G >> 3, r = G & 7, x = bid & 7;
    const int px = q + (x < r ? 1 : 0);
    const int wx = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
    TileRange t;
    t.first = (int)(total * wx / G) + (bid >> 3);
    t.end = (int)(total * (wx + px) / G);
    t.step = px;
    return t;
}

// The contiguous forms' tail: of `tiles` 256 x 256 tiles whose launch keeps `busy` workgroups
// busy (the tiles, plus one per N tile for each served straddle), the tiles left to 128-row
// tiles at the end of the launch: the busy workgroups of the last partial wave over `cus` CUs
// when they number between cus / 8 and cus / 4 (and fewer than the tiles), else none.
DG_HD inline int tail_count(int64_t busy, int64_t tiles, int cus)
{
    if (cus <= 0)
        return 0;
    const int64_t r = busy % cus;
    return (8 * r >= cus && 4 * r <= cus && r < tiles) ? (int)r : 0;
}

// The inverse for one workgroup per tile (total == grid - lead): the id of the workgroup that
// xcd_tile_range gives tile `tile` to.  XCD x's range starts at w_x and its workgroups take
// one tile each in id order, so the tile w_x + j falls to workgroup lead + 8 j + x.
// Preconditions: 0 < total == grid - lead, 0 <= tile < total.
DG_HD inline int xcd_tile_owner(int total, int lead, int tile)
{
    const int q = total >> 3, r = total & 7;
    int x, j;
    if (tile < r * (q + 1)) {
        x = tile / (q + 1);
        j = tile - x * (q + 1);
    } else {
        x = r + (tile - r * (q + 1)) / q;
        j = tile - (r * (q + 1) + (x - r) * q);
    }
    return lead + 8 * j + x;
}

}  // namespace dg
