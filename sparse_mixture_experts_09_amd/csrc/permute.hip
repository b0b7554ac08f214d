// Permutation with token-order capacity.
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
//   1. hist:    per chunk of 256 tokens, per expert counts (LDS counters;
//               counts do not depend on the order of the increments).
//   2. scan:    one block: per expert, the exclusive prefix of the chunk
//               counts over chunks, the demand, kept = min(demand, cap), and
//               the exclusive prefix of kept over experts (the offsets).
//   3. rank:    per chunk: inside each wavefront, for every expert, a ballot
//               of the lanes (tokens) that chose it and a popcount of the
//               lanes below give the in-wave rank; wave totals in LDS give
//               the in-chunk rank; plus the chunk prefix from step 2. Writes
//               slot_row (row or -1) and row_slot.
//   4. scatter: one wavefront per token reads the x row once with 16-byte
//               loads and writes it to each of its kept rows.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kChunk = 256;   // tokens per chunk = threads per block in hist / rank

__global__ __launch_bounds__(256) void perm_hist_kernel(int64_t T, int E, int k,
                                                        const int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ chunk_counts) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t t = (int64_t)blockIdx.x * kChunk + tid;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) chunk_counts[(int64_t)blockIdx.x * E + tid] = cnt[tid];
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
    for (int b = 0; b < nchunks; ++b) {
      const int c = chunk_counts[(int64_t)b * E + e];
      chunk_counts[(int64_t)b * E + e] = running;   // becomes the chunk base
      running += c;
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

__global__ __launch_bounds__(256) void perm_rank_kernel(int64_t T, int E, int k, int64_t cap,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ chunk_base,
                                                        const int32_t* __restrict__ expert_offsets,
                                                        int32_t* __restrict__ slot_row,
                                                        int32_t* __restrict__ row_slot) {
  __shared__ int wave_cnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t t = (int64_t)blockIdx.x * kChunk + tid;
  const bool valid = t < T;
  int ex[8], rk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = (valid && j < k) ? idx[t * k + j] : -1;
    rk[j] = 0;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < E; ++e) {
    bool has = false;
#pragma unroll
    for (int j = 0; j < 8; ++j) has |= (ex[j] == e);
    const uint64_t m = __ballot(has);
    const int r = __popcll(m & below);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (ex[j] == e) rk[j] = r;
    if (lane == 0) wave_cnt[wave][e] = __popcll(m);
  }
  __syncthreads();
  if (!valid) return;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    const int e = ex[j];
    int row = -1;
    if (e >= 0 && e < E) {
      int rank = chunk_base[(int64_t)blockIdx.x * E + e] + rk[j];
      for (int w = 0; w < wave; ++w) rank += wave_cnt[w][e];
      if (rank < cap) {
        row = expert_offsets[e] + rank;
        row_slot[row] = (int32_t)(t * k + j);
      }
    }
    slot_row[t * k + j] = row;
  }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(int64_t T, int k, size_t row_bytes,
                                                           const char* __restrict__ x,
                                                           const int32_t* __restrict__ slot_row,
                                                           char* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
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
#pragma unroll 2
  for (size_t off = (size_t)lane * 16; off < row_bytes; off += 64 * 16) {
    const u32x4 v = ld16(src + off);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (rows[j] >= 0) st16(x_perm + (size_t)rows[j] * row_bytes + off, v);
  }
}

}  // namespace

int64_t permute_chunks(int64_t T) { return (T + kChunk - 1) / kChunk; }

hipError_t launch_permute(bool bf16, int64_t T, int d, int E, int k, int64_t cap, const void* x,
                          const int32_t* idx, int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* slot_row, int32_t* row_slot, void* x_perm, int32_t* chunk_counts,
                          hipStream_t s) {
  const int64_t nchunks = permute_chunks(T);
  hipLaunchKernelGGL(perm_hist_kernel, dim3((unsigned)nchunks), dim3(256), 0, s, T, E, k, idx,
                     chunk_counts);
  hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(256), 0, s, (int)nchunks, E, cap, chunk_counts,
                     expert_counts, expert_offsets);
  hipLaunchKernelGGL(perm_rank_kernel, dim3((unsigned)nchunks), dim3(256), 0, s, T, E, k, cap, idx,
                     chunk_counts, expert_offsets, slot_row, row_slot);
  const size_t row_bytes = (size_t)d * (bf16 ? 2 : 4);
  hipLaunchKernelGGL(perm_scatter_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, k,
                     row_bytes, reinterpret_cast<const char*>(x), slot_row,
                     reinterpret_cast<char*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
