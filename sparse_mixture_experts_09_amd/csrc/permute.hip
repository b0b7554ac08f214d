// Permutation with token-order or priority-order capacity.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts", the
// MoE-layer walkthrough: after routing, every expert's tokens are arranged
// into one matrix, and tokens beyond the capacity are dropped. "Scaling
// Vision with Sparse Mixture of Experts", section "Priority Routing": a fixed
// buffer per expert, assignments beyond it dropped once the expert is full.
// "Take a Closer Look at the MoE LLM Routing", Introduction: drops land
// towards the end of the sequence -- the buffers fill in token order.
//
// The rank of (t, e) is the number of earlier tokens that chose e. It is
// computed without atomics on the order, so the result is deterministic:
//   1. count:   per chunk of 256 tokens: inside each wavefront, for every
//               expert present, a ballot of the lanes (tokens) that chose it
//               and a popcount of the lanes below give the in-wave rank; the
//               wavefront totals in LDS give the in-chunk rank of every slot
//               and the chunk's count per expert. The in-chunk rank goes to
//               slot_row for now, packed with its chunk.
//   2. scan:    one block: per expert, the exclusive prefix of the chunk
//               counts over chunks, the demand, kept = min(demand, cap), and
//               the exclusive prefix of kept over experts (the offsets).
//   3. place:   one wavefront per token: its lanes 0..k-1 turn the packed
//               in-chunk ranks into rows (offsets + chunk prefix + rank, -1
//               past the capacity) and write slot_row and row_slot, while
//               the token's row, loaded first, is written to each kept row
//               with 16-byte stores (the copy is skipped when the grouped
//               GEMM gathers the rows itself).
// Up to 1024 tokens, steps 1-2 and the rows run as one 1024-thread workgroup
// instead (perm_layout_kernel): the same ballot ranks per wavefront, the
// per-expert prefix over the wavefronts, the demand and the offsets, all in
// LDS; the copy follows with a wavefront per 1 KB piece of a row
// (perm_scatter_kernel), for parallelism at few tokens.
//
// Batch Priority Routing ("Scaling Vision with Sparse Mixture of Experts",
// section "Priority Routing": tokens are taken by an importance score rather
// than by position): steps 1 and 3 walk the tokens in a given order instead
// of 0..T-1, so ranks count the assignments that arrive earlier in that
// order. The order (score descending as float32, equal scores by ascending
// token) comes, for T <= 16384, from counting for every token the tokens
// with a smaller 64-bit (score image, token) key, and beyond that from a
// stable least-significant-digit radix sort: four passes
// of 8 bits over an order-preserving integer image of the score, each pass a
// per-chunk digit histogram, one exclusive scan over (digit, chunk), and a
// stable scatter whose in-chunk rank comes from ballots (lanes with the same
// digit) and per-wavefront digit counts in LDS.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kChunk = 256;   // tokens per chunk = threads per block of the count kernel
// The scan folds into the place kernel while every block's share of it (the
// nchunks x E counts) is small: measured 31.0 -> 28.2 us for the Mixtral
// shape's permute stage (16 x 8 counts), but 78.7 -> 81.1 us at 32 x 64
// (fine-grained), where the separate one-block scan stays.
constexpr int64_t kInlineScanCounts = 512;

// In-wavefront ranks of the slots a lane holds: one ballot per distinct
// expert present among the wavefront's pending slots. ex[j] = -1 for a slot
// that takes no part. Returns nothing; fills rk[] and, from lane 0, the
// wavefront's count of each expert it saw into wcnt[e].
__device__ __forceinline__ void wave_ranks(const int (&ex)[8], int (&rk)[8], int* wcnt) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t pend = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) pend |= (ex[j] >= 0 ? 1u : 0u) << j;
  for (;;) {
    const uint64_t busy = __ballot(pend != 0);
    if (busy == 0) break;
    int mine = -1;
#pragma unroll
    for (int j = 7; j >= 0; --j)
      if ((pend >> j) & 1) mine = ex[j];
    const int e = __builtin_amdgcn_readlane(mine, __ffsll((long long)busy) - 1);
    bool has = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) has |= ((pend >> j) & 1) && ex[j] == e;
    const uint64_t m = __ballot(has);
    const int r = __popcll(m & below);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (((pend >> j) & 1) && ex[j] == e) {
        rk[j] = r;
        pend &= ~(1u << j);
      }
    if (lane == 0) wcnt[e] = __popcll(m);
  }
}

// Step 1 (chunks of 256 positions of the arrival sequence; order: token at
// each position, nullptr for token order). Writes chunk_counts[chunk][e] and,
// for every slot, packed[t * k + j] = (chunk << 8) | in-chunk rank (a chunk
// holds an expert at most 256 times, so the rank fits 8 bits), -1 for an
// expert id outside [0, E).
__global__ __launch_bounds__(256) void perm_count_kernel(int64_t T, int E, int k,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ order,
                                                         int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ packed) {
  extern __shared__ int wcnt[];   // [4][E]: wavefront counts, then their prefix over the wavefronts
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t p = (int64_t)blockIdx.x * kChunk + tid;
  const bool valid = p < T;
  const int64_t t = valid ? (order ? (int64_t)order[p] : p) : 0;
  int ex[8], rk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = (valid && j < k) ? idx[t * k + j] : -1;
    ex[j] = (e >= 0 && e < E) ? e : -1;
    rk[j] = 0;
  }
  for (int i = tid; i < 4 * E; i += 256) wcnt[i] = 0;
  __syncthreads();
  wave_ranks(ex, rk, wcnt + wave * E);
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = wcnt[w * E + e];
      wcnt[w * E + e] = run;
      run += c;
    }
    chunk_counts[(int64_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  if (!valid) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    packed[t * k + j] = ex[j] >= 0 ? (int32_t)((blockIdx.x << 8) | (wcnt[wave * E + ex[j]] + rk[j])) : -1;
  }
}

// Inclusive scan of one int per thread over a 256-thread block.
__device__ __forceinline__ int block_inclusive_scan(int v, int* sh_wave) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh_wave[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += sh_wave[w];
  __syncthreads();
  return v + add;
}

__global__ __launch_bounds__(256) void perm_scan_kernel(int nchunks, int E, int64_t cap,
                                                        int32_t* __restrict__ chunk_counts,
                                                        int32_t* __restrict__ expert_counts,
                                                        int32_t* __restrict__ expert_offsets) {
  __shared__ int sh_wave[4];
  const int e = threadIdx.x;
  int running = 0;
  if (e < E) {
    // 16 chunks at a time: the loads are issued together, then the prefix
    // replaces them (one memory round trip per 16 chunks, not per chunk)
    for (int b0 = 0; b0 < nchunks; b0 += 16) {
      int c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = b0 + i < nchunks ? chunk_counts[(int64_t)(b0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (b0 + i < nchunks) chunk_counts[(int64_t)(b0 + i) * E + e] = running;   // becomes the chunk base
        running += c[i];
      }
    }
  }
  const int kept = e < E ? (int)min<int64_t>(running, cap) : 0;
  const int incl = block_inclusive_scan(kept, sh_wave);
  if (e < E) {
    expert_counts[e] = running;
    expert_offsets[e] = incl - kept;
    if (e == E - 1) expert_offsets[E] = incl;
  }
}

// Step 3: one wavefront per token. The token's row (all of it, in groups of
// 8 KB) is loaded before the row arithmetic so the copy does not wait on it;
// lanes 0..k-1 then read their slot's packed in-chunk rank (written by step
// 1 into slot_row, read and replaced by the same lane here), add the chunk
// prefix and the expert's offset, apply the capacity, and write slot_row and
// row_slot; the rows are broadcast and the row is stored to each kept one.
// x_perm == nullptr: the layout only (the grouped GEMM gathers the rows).
// inline_chunks > 0 (token-order fill, few chunks x experts): step 2 is folded in.
// chunk_counts then still holds the raw counts, and every block works out,
// while its rows load, the per-expert totals, kept counts and offsets and
// the prefix of its own chunk (a block's 4 tokens share one chunk); block 0
// writes expert_counts and expert_offsets. Otherwise chunk_counts holds the
// chunk bases and expert_offsets the offsets from perm_scan_kernel.
__global__ __launch_bounds__(256) void perm_place_kernel(int64_t T, int E, int k, int64_t cap, size_t row_bytes,
                                                         int inline_chunks, const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ chunk_counts,
                                                         int32_t* __restrict__ expert_counts,
                                                         int32_t* __restrict__ expert_offsets,
                                                         int32_t* __restrict__ slot_row,
                                                         int32_t* __restrict__ row_slot,
                                                         const char* __restrict__ x, char* __restrict__ x_perm) {
  constexpr int G = 8;   // 1 KB pieces per lane group in flight
  __shared__ int sh_base[256], sh_off[256], sh_wave[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (tid >> 6);
  const bool live = t < T;
  const char* src = x + (size_t)(live ? t : 0) * row_bytes;
  const size_t first = (size_t)lane * 16;
  u32x4 v[G];
  if (live && x_perm != nullptr) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (first + (size_t)g * 1024 < row_bytes) v[g] = ld16(src + first + (size_t)g * 1024);
  }
  if (inline_chunks > 0) {
    const int chunk = (int)(((int64_t)blockIdx.x * 4) / kChunk);
    int total = 0, base = 0;
    if (tid < E) {
      for (int c0 = 0; c0 < inline_chunks; c0 += 16) {
        int c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) c[i] = c0 + i < inline_chunks ? chunk_counts[(int64_t)(c0 + i) * E + tid] : 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          total += c[i];
          base += c0 + i < chunk ? c[i] : 0;
        }
      }
    }
    const int kept = tid < E ? (int)min<int64_t>(total, cap) : 0;
    const int incl = block_inclusive_scan(kept, sh_wave);
    if (tid < E) {
      sh_base[tid] = base;
      sh_off[tid] = incl - kept;
      if (blockIdx.x == 0) {
        expert_counts[tid] = total;
        expert_offsets[tid] = incl - kept;
        if (tid == E - 1) expert_offsets[E] = incl;
      }
    }
    __syncthreads();
  }
  if (!live) return;
  int row = -1;
  if (lane < k) {
    const int e = idx[t * k + lane];
    const int pk = slot_row[t * k + lane];
    if (pk >= 0 && e >= 0 && e < E) {
      const int rank = (inline_chunks > 0 ? sh_base[e] : chunk_counts[(int64_t)(pk >> 8) * E + e]) + (pk & 255);
      if (rank < cap) {
        row = (inline_chunks > 0 ? sh_off[e] : expert_offsets[e]) + rank;
        row_slot[row] = (int32_t)(t * k + lane);
      }
    }
    slot_row[t * k + lane] = row;
  }
  if (x_perm == nullptr) return;
  int rows[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) rows[j] = j < k ? __shfl(row, j) : -1;
  for (size_t base = 0; base < row_bytes; base += (size_t)G * 1024) {
    if (base > 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
        if (base + first + (size_t)g * 1024 < row_bytes) v[g] = ld16(src + base + first + (size_t)g * 1024);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const size_t off = base + first + (size_t)g * 1024;
      if (off < row_bytes) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (rows[j] >= 0) st16(x_perm + (size_t)rows[j] * row_bytes + off, v[g]);
      }
    }
  }
}

// Steps 1-3 in one workgroup for T <= 1024: thread tid holds the token at
// position tid of the arrival sequence. LDS: wcnt[wave * E + e] = the
// wavefront's assignments to e, turned in place into their exclusive prefix
// over the wavefronts; off[E]; the per-wavefront scan totals. (Several passes
// of 1024 tokens in one workgroup measured slower than the chunked kernels at
// 4096 tokens: one CU then walks every wavefront's ballots.)
constexpr int kLayoutMaxT = 1024;

__global__ __launch_bounds__(1024) void perm_layout_kernel(int T, int E, int k, int64_t cap,
                                                           const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ order,
                                                           int32_t* __restrict__ expert_counts,
                                                           int32_t* __restrict__ expert_offsets,
                                                           int32_t* __restrict__ slot_row,
                                                           int32_t* __restrict__ row_slot) {
  extern __shared__ int sh[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int* wcnt = sh;
  int* off = sh + 16 * E;
  int* wsum = off + E;
  const int tok = tid < T ? (order ? order[tid] : tid) : -1;
  int ex[8], rk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int e = (tok >= 0 && j < k) ? idx[(int64_t)tok * k + j] : -1;
    ex[j] = (e >= 0 && e < E) ? e : -1;
    rk[j] = 0;
  }
  for (int i = tid; i < 16 * E; i += 1024) wcnt[i] = 0;
  __syncthreads();
  // in-wavefront ranks: one ballot per distinct expert present in the wavefront
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t pend = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) pend |= (ex[j] >= 0 ? 1u : 0u) << j;
  for (;;) {
    const uint64_t busy = __ballot(pend != 0);
    if (busy == 0) break;
    int mine = -1;
#pragma unroll
    for (int j = 7; j >= 0; --j)
      if ((pend >> j) & 1) mine = ex[j];
    const int e = __builtin_amdgcn_readlane(mine, __ffsll((long long)busy) - 1);
    bool has = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) has |= ((pend >> j) & 1) && ex[j] == e;
    const uint64_t m = __ballot(has);
    const int r = __popcll(m & below);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (((pend >> j) & 1) && ex[j] == e) {
        rk[j] = r;
        pend &= ~(1u << j);
      }
    if (lane == 0) wcnt[wave * E + e] = __popcll(m);
  }
  __syncthreads();
  // per expert (one wavefront each, lane w for wavefront w's count): the
  // exclusive prefix over the wavefronts in place, the demand into off[e]
  for (int e = wave; e < E; e += 16) {
    const int c = lane < 16 ? wcnt[lane * E + e] : 0;
    int v = c;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(v, o);
      if (lane >= o) v += u;
    }
    if (lane < 16) wcnt[lane * E + e] = v - c;
    if (lane == 15) off[e] = v;
  }
  __syncthreads();
  int kept = 0;
  if (tid < E) {
    const int run = off[tid];
    expert_counts[tid] = run;
    kept = (int)min<int64_t>(run, cap);
  }
  // exclusive scan of kept over the experts (E <= 256: wavefronts 0-3)
  int v = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (tid < E) {
    int add = 0;
    for (int w = 0; w < wave; ++w) add += wsum[w];
    const int excl = v + add - kept;
    off[tid] = excl;
    expert_offsets[tid] = excl;
    if (tid == E - 1) expert_offsets[E] = excl + kept;
  }
  __syncthreads();
  if (tok < 0) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = ex[j];
    int row = -1;
    if (e >= 0) {
      const int rank = wcnt[wave * E + e] + rk[j];
      if (rank < cap) {
        row = off[e] + rank;
        row_slot[row] = tok * k + j;
      }
    }
    slot_row[(int64_t)tok * k + j] = row;
  }
}

// Each wavefront copies `ppw` 1 KB pieces of one token's row (16 bytes a
// lane per piece), reading each piece once and storing it to each kept row
// of the token; a row has `pieces` pieces, split over pieces / ppw wavefronts.
__global__ __launch_bounds__(256) void perm_scatter_kernel(int64_t T, int k, size_t row_bytes, int pieces, int ppw,
                                                           const char* __restrict__ x,
                                                           const int32_t* __restrict__ slot_row,
                                                           char* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int wpt = pieces / ppw;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = wpt == 1 ? gw : gw / wpt;
  if (t >= T) return;
  int rows[8];
  bool any = false;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? slot_row[t * k + j] : -1;
    any |= rows[j] >= 0;
  }
  if (!any) return;
  const char* src = x + (size_t)t * row_bytes;
  const size_t first = (size_t)(gw - t * wpt) * ppw * 1024 + (size_t)lane * 16;
  const size_t end = min(row_bytes, first - (size_t)lane * 16 + (size_t)ppw * 1024);
#pragma unroll 2
  for (size_t off = first; off < end; off += 1024) {
    const u32x4 v = ld16(src + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (rows[j] >= 0) st16(x_perm + (size_t)rows[j] * row_bytes + off, v);
  }
}

// ---------------------------------------------------------------------------
// Priority order: stable radix sort of the positions 0..T-1 by score
// ---------------------------------------------------------------------------

// Order-preserving image of a float: larger score -> smaller key, so an
// ascending sort gives descending scores. -0 is taken as +0 (they compare
// equal as numbers, so they must tie).
__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;   // ascending image
  return ~u;
}

__global__ __launch_bounds__(256) void rsort_prep_kernel(int64_t T, const float* __restrict__ score,
                                                         int64_t stride, uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ vals) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= T) return;
  keys[p] = desc_key(score[p * stride]);
  vals[p] = (int32_t)p;
}

// hist[digit * nchunks + chunk] = elements of the chunk with that digit
__global__ __launch_bounds__(256) void rsort_hist_kernel(int64_t T, int shift, int64_t nchunks,
                                                         const uint32_t* __restrict__ keys,
                                                         int32_t* __restrict__ hist) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * 256 + tid;
  if (p < T) atomicAdd(&cnt[(keys[p] >> shift) & 255u], 1);
  __syncthreads();
  hist[(int64_t)tid * nchunks + blockIdx.x] = cnt[tid];
}

// Exclusive scan of n ints in place, one block of 1024 threads walking the
// array in coalesced tiles of 1024 with a running carry.
__global__ __launch_bounds__(1024) void rsort_scan_kernel(int64_t n, int32_t* __restrict__ a) {
  __shared__ int sh[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t i = base + tid;
    const int v = i < n ? a[i] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o);
      if (lane >= o) incl += u;
    }
    if (lane == 63) sh[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int t = sh[w];
      before += w < wave ? t : 0;
      total += t;
    }
    if (i < n) a[i] = carry + before + incl - v;
    carry += total;
    __syncthreads();   // sh is rewritten by the next tile
  }
}

// Small problems (T <= 16384): the position of token t in the order is the
// number of tokens whose 64-bit key (score image << 32 | token) is below
// t's; keys are distinct, so the positions are a permutation. Block (b, sp)
// counts, for the 256 tokens of tile b, the keys of split sp of the token
// range (staged through LDS); the per-split counts are added in split order
// by the scatter kernel, so no atomics and no zeroing are needed.
constexpr int kSmallSort = 16384;
constexpr int kCountTile = 1024;

__device__ __forceinline__ uint64_t full_key(const float* score, int64_t stride, int64_t t) {
  return ((uint64_t)desc_key(score[t * stride]) << 32) | (uint32_t)t;
}

__global__ __launch_bounds__(256) void rank_count_kernel(int64_t T, int splits, const float* __restrict__ score,
                                                         int64_t stride, int32_t* __restrict__ partial) {
  __shared__ uint64_t tile[kCountTile];
  const int tid = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * 256 + tid;
  const uint64_t mine = t < T ? full_key(score, stride, t) : 0ull;
  const int sp = blockIdx.y;
  const int64_t lo = T * sp / splits, hi = T * (sp + 1) / splits;
  int cnt = 0;
  for (int64_t base = lo; base < hi; base += kCountTile) {
    const int n = (int)min<int64_t>(kCountTile, hi - base);
    __syncthreads();
    for (int i = tid; i < n; i += 256) tile[i] = full_key(score, stride, base + i);
    __syncthreads();
    for (int i = 0; i < n; ++i) cnt += tile[i] < mine ? 1 : 0;
  }
  if (t < T) partial[(int64_t)sp * T + t] = cnt;
}

__global__ __launch_bounds__(256) void rank_scatter_kernel(int64_t T, int splits, const int32_t* __restrict__ partial,
                                                           int32_t* __restrict__ order) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int pos = 0;
  for (int sp = 0; sp < splits; ++sp) pos += partial[(int64_t)sp * T + t];
  order[pos] = (int32_t)t;
}

int small_sort_splits(int64_t T) {
  const int64_t s = T / 512;
  return s < 1 ? 1 : (s > 32 ? 32 : (int)s);
}

__global__ __launch_bounds__(256) void rsort_scatter_kernel(int64_t T, int shift, int64_t nchunks,
                                                            const uint32_t* __restrict__ keys_in,
                                                            const int32_t* __restrict__ vals_in,
                                                            const int32_t* __restrict__ base,
                                                            uint32_t* __restrict__ keys_out,
                                                            int32_t* __restrict__ vals_out) {
  __shared__ int wave_cnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) (&wave_cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t p = (int64_t)blockIdx.x * 256 + tid;
  const bool valid = p < T;
  const uint32_t key = valid ? keys_in[p] : 0u;
  const int dg = (int)((key >> shift) & 255u);
  // lanes of this wavefront holding the same digit
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const uint64_t m = __ballot((dg >> b) & 1);
    same &= ((dg >> b) & 1) ? m : ~m;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int r = __popcll(same & below);
  // the last lane of each digit group publishes the group's size
  if (valid && (same >> lane) == 1ull) wave_cnt[wave][dg] = __popcll(same);
  __syncthreads();
  if (!valid) return;
  int pos = base[(int64_t)dg * nchunks + blockIdx.x] + r;
  for (int w = 0; w < wave; ++w) pos += wave_cnt[w][dg];
  keys_out[pos] = key;
  vals_out[pos] = vals_in[p];
}

}  // namespace

int64_t permute_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

size_t priority_sort_bytes(int64_t T) {
  // small T: per-split partial positions; otherwise keys and values, twice
  // (ping-pong), plus the (digit, chunk) histogram
  if (T <= kSmallSort) return (size_t)small_sort_splits(T) * T * 4;
  const int64_t nchunks = permute_chunks(T);
  return (size_t)T * 16 + (size_t)nchunks * 256 * 4;
}

hipError_t launch_priority_order(int64_t T, const float* score, int64_t stride, int32_t* order, void* ws,
                                 hipStream_t s) {
  if (T <= kSmallSort) {
    const int splits = small_sort_splits(T);
    int32_t* partial = reinterpret_cast<int32_t*>(ws);
    const unsigned tiles = (unsigned)((T + 255) / 256);
    hipLaunchKernelGGL(rank_count_kernel, dim3(tiles, (unsigned)splits), dim3(256), 0, s, T, splits, score, stride,
                       partial);
    hipLaunchKernelGGL(rank_scatter_kernel, dim3(tiles), dim3(256), 0, s, T, splits, partial, order);
    return hipGetLastError();
  }
  const int64_t nchunks = permute_chunks(T);
  char* w = reinterpret_cast<char*>(ws);
  uint32_t* ka = reinterpret_cast<uint32_t*>(w);
  uint32_t* kb = ka + T;
  int32_t* vb = reinterpret_cast<int32_t*>(kb + T);
  int32_t* hist = vb + T;
  // the values start in `order`; four passes end there again
  hipLaunchKernelGGL(rsort_prep_kernel, dim3((unsigned)nchunks), dim3(256), 0, s, T, score, stride, ka, order);
  for (int pass = 0; pass < 4; ++pass) {
    const bool even = (pass & 1) == 0;
    const uint32_t* kin = even ? ka : kb;
    uint32_t* kout = even ? kb : ka;
    const int32_t* vin = even ? order : vb;
    int32_t* vout = even ? vb : order;
    hipLaunchKernelGGL(rsort_hist_kernel, dim3((unsigned)nchunks), dim3(256), 0, s, T, 8 * pass, nchunks, kin,
                       hist);
    hipLaunchKernelGGL(rsort_scan_kernel, dim3(1), dim3(1024), 0, s, nchunks * 256, hist);
    hipLaunchKernelGGL(rsort_scatter_kernel, dim3((unsigned)nchunks), dim3(256), 0, s, T, 8 * pass, nchunks, kin,
                       vin, hist, kout, vout);
  }
  return hipGetLastError();
}

hipError_t launch_permute(bool bf16, int64_t T, int d, int E, int k, int64_t cap, const void* x,
                          const int32_t* idx, const int32_t* order, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* slot_row, int32_t* row_slot, void* x_perm,
                          int32_t* chunk_counts, hipStream_t s) {
  if (T <= kLayoutMaxT) {
    const size_t lds = (size_t)(17 * E + 16) * sizeof(int);
    hipLaunchKernelGGL(perm_layout_kernel, dim3(1), dim3(1024), lds, s, (int)T, E, k, cap, idx, order,
                       expert_counts, expert_offsets, slot_row, row_slot);
    if (x_perm == nullptr) return hipGetLastError();   // the layout only: the GEMM gathers the rows
    const size_t row_bytes = (size_t)d * (bf16 ? 2 : 4);
    const int pieces = (int)((row_bytes + 1023) / 1024);
    // few tokens: a wavefront per 1 KB piece, for parallelism
    const int64_t waves = T * pieces;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, T, k, row_bytes,
                       pieces, 1, reinterpret_cast<const char*>(x), slot_row, reinterpret_cast<char*>(x_perm));
    return hipGetLastError();
  }
  const int64_t nchunks = permute_chunks(T);
  hipLaunchKernelGGL(perm_count_kernel, dim3((unsigned)nchunks), dim3(256), (size_t)4 * E * sizeof(int), s, T, E,
                     k, idx, order, chunk_counts, slot_row);
  // token order with few chunks: the scan runs inside the place kernel (every
  // block reads the nchunks x E counts while its rows load); otherwise its own launch
  const int inline_chunks = (order == nullptr && nchunks * E <= kInlineScanCounts) ? (int)nchunks : 0;
  if (inline_chunks == 0)
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, s, (int)nchunks, E, cap, chunk_counts,
                       expert_counts, expert_offsets);
  hipLaunchKernelGGL(perm_place_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, E, k, cap,
                     (size_t)d * (bf16 ? 2 : 4), inline_chunks, idx, chunk_counts, expert_counts, expert_offsets,
                     slot_row, row_slot, reinterpret_cast<const char*>(x), reinterpret_cast<char*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
