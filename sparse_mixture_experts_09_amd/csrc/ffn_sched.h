// Work scheduling for the grouped expert GEMMs.
//
// The number of rows per expert is data dependent and stays on the device, so
// every block derives its work from expert_offsets itself. Tiles are numbered
// expert by expert; inside an expert the m-tiles (row blocks) run fastest, so
// consecutive tile numbers share one weight n-tile.
//
// Split tail: with P compute units, tiles beyond the last whole round of P
// would run as a partly empty round as long as a full tile. When a launch
// allows it, each of those r tail tiles is cut into s = min(P / r, max_split,
// K steps) K-slices; the slices write fp32 partial tiles and a reduce pass sums
// them in slice order (so the result does not depend on timing).
//
// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2. Block b therefore works on XCD b % 8, and the block ->
// item map hands each XCD one contiguous run of whole tiles (blocks that share
// a weight n-tile or a row block meet in the same L2) followed by an equal
// share of the tail slices. The grid is an upper bound; blocks without an
// item exit.
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

struct WorkPlan {
  int tiles;  // tiles in total
  int full;   // tiles computed whole
  int r;      // tail tiles split into K-slices
  int s;      // slices per tail tile (1 when nothing is split)
};

struct WorkItem {
  TileCoord tc;
  int slice;  // K-slice of a split tile, 0 otherwise
  int split;  // index of the split tile in [0, r), -1 for a whole tile
};

constexpr int kXcds = 8;

__device__ __forceinline__ WorkPlan make_plan(const int32_t* __restrict__ offsets, int E, int BM, int NT,
                                              int P, int max_split, int KT) {
  int tiles = 0;
  for (int e = 0; e < E; ++e) {
    const int cnt = offsets[e + 1] - offsets[e];
    tiles += ((cnt + BM - 1) / BM) * NT;
  }
  WorkPlan p{tiles, tiles, 0, 1};
  if (max_split > 1 && P > 0) {
    const int rem = tiles % P;
    if (rem > 0) {
      const int s = min(min(P / rem, max_split), KT);
      if (s >= 2) {
        p.full = tiles - rem;
        p.r = rem;
        p.s = s;
      }
    }
  }
  return p;
}

__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ offsets, int E, int BM, int NT,
                                            int tile, TileCoord& tc) {
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

// Upper bound on the blocks a launch needs (tiles_ub bounds the tile count).
inline int64_t grid_blocks(int64_t tiles_ub, int P, bool split) {
  const int64_t per_xcd = (tiles_ub + kXcds - 1) / kXcds + 1 + (split ? (P + kXcds - 1) / kXcds + 1 : 0);
  return per_xcd * kXcds;
}

__device__ __forceinline__ bool find_item(const int32_t* __restrict__ offsets, int E, int BM, int NT, int P,
                                          int max_split, int KT, int bid, WorkItem& w) {
  const WorkPlan p = make_plan(offsets, E, BM, NT, P, max_split, KT);
  const int x = bid % kXcds, l = bid / kXcds;
  const int fq = p.full / kXcds, fr = p.full % kXcds;
  const int nf = fq + (x < fr ? 1 : 0);
  int tile;
  w.slice = 0;
  w.split = -1;
  if (l < nf) {
    tile = x * fq + min(x, fr) + l;
  } else {
    const int ns = p.r * p.s, sq = ns / kXcds, sr = ns % kXcds;
    const int l2 = l - nf;
    if (l2 >= sq + (x < sr ? 1 : 0)) return false;
    const int j = x * sq + min(x, sr) + l2;
    w.split = j / p.s;
    w.slice = j % p.s;
    tile = p.full + w.split;
  }
  return locate_tile(offsets, E, BM, NT, tile, w.tc);
}

// Whole tiles only (no split tail).
__device__ __forceinline__ bool find_tile(const int32_t* __restrict__ offsets, int E, int BM, int NT, int bid,
                                          TileCoord& tc) {
  WorkItem w;
  if (!find_item(offsets, E, BM, NT, 0, 1, 1, bid, w)) return false;
  tc = w.tc;
  return true;
}

}  // namespace moe
