// Tile scheduling for the grouped expert GEMMs.
//
// The number of rows per expert is data dependent and stays on the device, so
// every block derives its tile from expert_offsets itself. Tiles are numbered
// expert by expert; inside an expert the m-tiles (row blocks) run fastest, so
// consecutive tile numbers share one weight n-tile. The grid is an upper
// bound (ceil(R_max/BM) + E) * NT; blocks past the real tile count exit.
//
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2. The block -> tile map therefore hands each XCD one
// contiguous run of tile numbers, so the blocks that share a weight n-tile
// (and the blocks that share a row block) meet in the same L2.
#pragma once

#include "moe_common.h"

namespace moe {

struct TileCoord {
  int e;          // expert
  int seg_start;  // first permuted row of the expert
  int seg_rows;   // kept rows of the expert
  int m0;         // first row of this tile, relative to seg_start
  int n_tile;     // output column tile
};

constexpr int kXcds = 8;

__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int BM, int NT,
                                          int bid, TileCoord& tc) {
  int total = 0;
  for (int e = 0; e < E; ++e) {
    const int cnt = offsets[e + 1] - offsets[e];
    total += ((cnt + BM - 1) / BM) * NT;
  }
  if (bid >= total) return false;
  const int q = total / kXcds, r = total % kXcds, x = bid % kXcds;
  int tile = x * q + min(x, r) + bid / kXcds;
  for (int e = 0; e < E; ++e) {
    const int lo = offsets[e];
    const int cnt = offsets[e + 1] - lo;
    const int mt = (cnt + BM - 1) / BM;
    if (tile < mt * NT) {
      tc.e = e;
      tc.seg_start = lo;
      tc.seg_rows = cnt;
      tc.m0 = (tile % mt) * BM;
      tc.n_tile = tile / mt;
      return true;
    }
    tile -= mt * NT;
  }
  return false;
}

}  // namespace moe
