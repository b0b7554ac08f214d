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

// Per-XCD plan (the forward kernels). Tiles keep the order above; XCD x takes
// the contiguous run [x T / 8, (x + 1) T / 8) of the T tiles, so its blocks
// share weight n-tiles and row blocks in its L2, and its tiles past the last
// whole round of its Px compute units form its own split tail: r = n mod Px
// tiles cut into s = min(Px / r, max_split, K steps) K-slices, whose partial
// tiles take slots x Px .. x Px + r s - 1. The plan is worked out by the whole
// 256-thread block at once (one expert per thread, a block scan through a few
// LDS words), and the blocks of an XCD step through its items with the
// grid's stride. (Runs balanced by an estimated tile cost, counting a ragged
// tile of at most 64 / 128 rows as 1/4 / 1/2 of a full one, measured slower
// at the Mixtral shape: such a tile still streams a whole weight tile. Costs
// of 5/8 and 6/8 measured no better than equal counts.)
struct XcdItem {
  TileCoord tc;
  int slice;    // K-slice of a split tile, 0 otherwise
  int nslices;  // slices of the tile (1 for a whole tile)
  int slot;     // partial tile of a split slice, -1 for a whole tile
};

// Thread e < E of the block: expert e's m-tiles, first row, rows, and the
// tiles of the experts before it.
struct ExpertScan {
  int mt, lo, cnt, tb;
};

// Block-wide exclusive scan of the tile counts over the experts; the total
// into tiles. ws: 4 ints of LDS. Every thread of the 256 calls it.
__device__ __forceinline__ ExpertScan expert_scan(const int32_t* __restrict__ offsets, int E, int NT, int* ws,
                                                  int& tiles) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  ExpertScan x{0, 0, 0, 0};
  if (tid < E) {
    x.lo = offsets[tid];
    x.cnt = offsets[tid + 1] - x.lo;
    x.mt = (x.cnt + 255) / 256;
  }
  int t = x.mt * NT;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(t, o);
    if (lane >= o) t += u;
  }
  __syncthreads();   // ws may still be read by an earlier use
  if (lane == 63) ws[wave] = t;
  __syncthreads();
  int before = 0;
  tiles = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) before += ws[w];
    tiles += ws[w];
  }
  x.tb = before + t - x.mt * NT;
  return x;
}

// The coordinates of tile t (t < tiles); ws: 5 ints of LDS.
__device__ __forceinline__ TileCoord locate_tile_scan(const ExpertScan& x, int E, int NT, int t, int* ws) {
  const int tid = threadIdx.x;
  __syncthreads();
  if (tid < E && x.mt > 0 && x.tb <= t && t < x.tb + x.mt * NT) {
    const int u = t - x.tb;
    ws[0] = tid;
    ws[1] = x.lo;
    ws[2] = x.cnt;
    ws[3] = (u % x.mt) * 256;
    ws[4] = u / x.mt;
  }
  __syncthreads();
  TileCoord tc;
  tc.e = ws[0];
  tc.seg_start = ws[1];
  tc.seg_rows = ws[2];
  tc.m0 = ws[3];
  tc.n_tile = ws[4];
  return tc;
}

struct XcdRun {
  int first, full, r, s;   // first tile, tiles computed whole, split tail tiles, slices each
};

__device__ __forceinline__ XcdRun xcd_run(int tiles, int Px, int max_split, int KT, int xcd) {
  const int first = (int)((int64_t)tiles * xcd / kXcds);
  const int n = (int)((int64_t)tiles * (xcd + 1) / kXcds) - first;
  XcdRun q{first, n, 0, 1};
  if (max_split > 1 && Px > 0) {
    const int rem = n % Px;
    if (rem > 0) {
      const int sl = min(min(Px / rem, max_split), KT);
      if (sl >= 2) {
        q.full = n - rem;
        q.r = rem;
        q.s = sl;
      }
    }
  }
  return q;
}

// Item l of a run: false past its end.
__device__ __forceinline__ bool xcd_item(const XcdRun& q, int xcd, int Px, int l, int& tile, XcdItem& w) {
  w.slice = 0;
  w.nslices = 1;
  w.slot = -1;
  tile = q.first + l;
  if (l >= q.full) {
    const int l2 = l - q.full;
    if (l2 >= q.r * q.s) return false;
    tile = q.first + q.full + l2 / q.s;
    w.slice = l2 % q.s;
    w.nslices = q.s;
    w.slot = xcd * Px + l2;
  }
  return true;
}

// Blocks per XCD of a per-XCD launch: a run holds at most ceil(T / 8) tiles
// and its split tail adds at most Px - 1 items.
inline int64_t xcd_grid_blocks(int64_t tiles_ub, int P, bool split) {
  const int64_t per_xcd = (tiles_ub + kXcds - 1) / kXcds + 1 + (split ? P / kXcds : 0);
  return per_xcd * kXcds;
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
