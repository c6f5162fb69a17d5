// expert_tiles.h -- decoding of the device-built expert-tile list (internal).
#pragma once

#include "device.h"
#include "kernels.h"

namespace moe {

struct TileInfo {
  int e;       // expert, E = the shared expert
  bool shared;
  int row0;    // first row (expert-sorted pair row, or token for the shared expert)
  int nrows;   // rows in this tile, 1..a.tile_rows
};

// tile_off[g] = tiles of "experts" 0..g-1 (the shared expert last),
// tile_off[E + 1] = total.  Returns false when `tile` is past the last tile.
__device__ __forceinline__ bool decode_tile(const ExpertArgs& a, int tile, TileInfo& ti) {
  if (tile < 0 || tile >= a.tile_off[a.E + 1]) return false;
  const int e = upper_bound_i32(a.tile_off, a.E + 2, tile) - 1;
  const int m = tile - a.tile_off[e];
  ti.e = e;
  ti.shared = (e == a.E);
  if (ti.shared) {
    ti.row0 = m * a.tile_rows;
    ti.nrows = min(a.tile_rows, a.T - ti.row0);
  } else {
    ti.row0 = a.offsets[e] + m * a.tile_rows;
    ti.nrows = min(a.tile_rows, a.offsets[e + 1] - ti.row0);
  }
  return true;
}

// Tile table entry t (two int32): {e | nrows << 16, row0}: expert (E = the
// shared expert), rows in the tile, first row (expert-sorted pair row, or
// token for the shared expert).
__device__ __forceinline__ void write_tile_entry(int32_t* tab, int32_t t, int e, int32_t first,
                                                 int32_t rows, int32_t m, int tile_rows) {
  const int32_t row0 = first + m * tile_rows;
  const int32_t nrows = min(tile_rows, rows - m * tile_rows);
  tab[2 * t] = e | (nrows << 16);
  tab[2 * t + 1] = row0;
}

// Builds tile_off and tile_tab from offsets (used when the permute kernels did not).
hipError_t launch_tiles(const ExpertArgs& a, hipStream_t s);

}  // namespace moe
