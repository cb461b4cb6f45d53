// plan.hpp -- tile geometry and the tile schedule, shared by the host planner
// and the gfx950 kernels (host + device code, no HIP runtime calls).
//
// The schedule realises the "tile coordinate swizzling" that the FLUX summary
// names (TL;DR of "FLUX: Fast Software-based Communication Overlap On GPUs
// Through Kernel Fusion") without giving details.  Chosen here:
//   - the M x N partial is cut into BM x BN tiles that never cross a row-slice
//     boundary (a slice has ceil(S/BM) tile rows; the last may be partial, as
//     may the last tile column);
//   - slot q visits destination slices in the order rank, rank+1, ... (mod tp),
//     so this rank's own slice -- the one its reducers consume -- is produced
//     first, and at every step the tp ranks target tp different destinations;
//   - inside a slice, tiles are visited in groups of group_m tile rows,
//     column-major within a group (grouped raster: concurrently running tiles
//     share rows of X and columns of W in L2).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define GRS_HD __host__ __device__ inline
#else
#define GRS_HD inline
#endif

namespace gemm_rs {

struct Geometry {
    int32_t M, N, K, S, tp, rank;
    int32_t bm, bn, bk;
    int32_t tms;      // tile rows per slice
    int32_t tnc;      // tile columns
    int32_t ts;       // tiles per slice
    int32_t tiles;    // all tiles
    int32_t group_m;  // raster group height in tile rows
};

struct TileCoord {
    int32_t d;     // destination slice (rank owning these rows)
    int32_t tml;   // tile row inside the slice
    int32_t tn;    // tile column
    int32_t flag;  // ready-flag index: d * ts + tml * tnc + tn
};

GRS_HD int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

GRS_HD Geometry make_geometry(int32_t M, int32_t N, int32_t K, int32_t tp, int32_t rank,
                              int32_t bm, int32_t bn, int32_t bk, int32_t group_m)
{
    Geometry g;
    g.M = M; g.N = N; g.K = K; g.tp = tp; g.rank = rank;
    g.S = M / tp;
    g.bm = bm; g.bn = bn; g.bk = bk;
    g.tms = g.S > 0 ? ceil_div(g.S, bm) : 0;
    g.tnc = N > 0 ? ceil_div(N, bn) : 0;
    g.ts = g.tms * g.tnc;
    g.tiles = tp * g.ts;
    g.group_m = group_m < 1 ? 1 : (group_m > g.tms && g.tms > 0 ? g.tms : group_m);
    return g;
}

// Slot q -> tile.  Destination step first (own slice at step 0), then a
// grouped raster inside the slice.
GRS_HD TileCoord decode_slot(const Geometry& g, int32_t q)
{
    TileCoord t;
    const int32_t step = q / g.ts;
    const int32_t within = q - step * g.ts;
    int32_t d = g.rank + step;
    if (d >= g.tp) d -= g.tp;
    const int32_t span = g.group_m * g.tnc;  // slots per full group
    const int32_t grp = within / span;
    int32_t rows = g.tms - grp * g.group_m;  // tile rows in this group
    if (rows > g.group_m) rows = g.group_m;
    const int32_t v = within - grp * span;
    t.d = d;
    t.tml = grp * g.group_m + v % rows;
    t.tn = v / rows;
    t.flag = d * g.ts + t.tml * g.tnc + t.tn;
    return t;
}

// Valid rows / columns of a (possibly ragged) tile.
GRS_HD int32_t tile_rows(const Geometry& g, const TileCoord& t)
{
    const int32_t r = g.S - t.tml * g.bm;
    return r < g.bm ? r : g.bm;
}

GRS_HD int32_t tile_cols(const Geometry& g, const TileCoord& t)
{
    const int32_t c = g.N - t.tn * g.bn;
    return c < g.bn ? c : g.bn;
}

// First row of the tile in the M x N partial (row of X_r).
GRS_HD int32_t tile_row0(const Geometry& g, const TileCoord& t)
{
    return t.d * g.S + t.tml * g.bm;
}

}  // namespace gemm_rs
