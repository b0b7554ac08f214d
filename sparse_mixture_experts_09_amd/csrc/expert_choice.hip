// Expert-choice routing: the experts select the tokens.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts": in
// expert choice the selection is reversed -- every expert takes a fixed
// number of tokens, so a token can get no expert, some, or all of them. The
// token-expert score is the dense gate Softmax(x.W_g) of "How do Mixture of
// Expert Models Work?" ("The Math Behind MoEs"); the router kernel writes it
// as a [T, E] fp32 matrix.
//
// Selection, one workgroup per expert e (C tokens each):
//   1. the column score[:, e] becomes 32-bit keys whose ascending order is
//      the descending score order (-0 equal to +0), in a contiguous scratch
//      row (one strided read of the column, coalesced passes afterwards);
//   2. a most-significant-digit radix select finds the C-th smallest key K
//      and how many tokens with key K to take (four 8-bit passes, each an
//      LDS histogram of the keys that match the digits fixed so far);
//   3. in token order, tile by tile, a block scan ranks the tokens with key
//      K (the first ones are taken: ties go to the lower token index) and a
//      second scan gives each chosen token its row e*C + position, so an
//      expert's rows list its tokens in ascending order.
// Every (t, e) of the [T, E] slot map is written (row or -1), so no zeroing
// is needed, and nothing depends on timing.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kSelThreads = 1024;
constexpr int64_t kSelLdsKeys = 32768;   // up to this many tokens the select keys stay in LDS (128 KB)

__device__ __forceinline__ uint32_t desc_score_key(float f) {
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  u ^= (u & 0x80000000u) ? 0xFFFFFFFFu : 0x80000000u;   // ascending image
  return ~u;                                              // larger score -> smaller key
}

// Inclusive scan of one int per thread over the 1024-thread block; returns
// the inclusive value and writes the block total to *total.
__device__ __forceinline__ int scan1024(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / 64; ++w) {
    const int s = sh[w];
    before += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();
  *total = all;
  return v + before;
}

// KL: the keys live in LDS (T <= kSelLdsKeys), else in the global scratch row.
template <bool KL>
__global__ __launch_bounds__(kSelThreads) void ec_select_kernel(int64_t T, int E, int C,
                                                                const float* __restrict__ scores,
                                                                uint32_t* __restrict__ keys_ws,
                                                                int32_t* __restrict__ tokens,
                                                                int32_t* __restrict__ slot,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int hist[256];
  __shared__ int sh[kSelThreads / 64];
  __shared__ int sel_digit, sel_before;
  extern __shared__ uint32_t lkeys[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int e = blockIdx.x;
  uint32_t* keys = KL ? lkeys : keys_ws + (size_t)e * T;
  for (int64_t t = tid; t < T; t += kSelThreads) keys[t] = desc_score_key(scores[t * E + e]);
  __syncthreads();

  // radix select of the C-th smallest key (1-based)
  uint32_t prefix = 0, mask = 0;
  int want = C;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    for (int64_t t = tid; t < T; t += kSelThreads) {
      const uint32_t k = keys[t];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane L holds bins 4L .. 4L+3; find the bin where the running count reaches `want`
      int c[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[4 * lane + i];
        s += c[i];
      }
      int incl = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o);
        if (lane >= o) incl += u;
      }
      int run = incl - s;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (run < want && want <= run + c[i]) {
          sel_digit = 4 * lane + i;
          sel_before = run;
        }
        run += c[i];
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel_digit << shift;
    mask |= 255u << shift;
    want -= sel_before;
    __syncthreads();   // sel_digit / sel_before are rewritten next pass
  }
  const uint32_t K = prefix;   // the C-th smallest key; take the first `want` tokens with key K

  // selection and compaction in token order
  int eq_seen = 0, sel_seen = 0;
  for (int64_t base = 0; base < T; base += kSelThreads) {
    const int64_t t = base + tid;
    const uint32_t k = t < T ? keys[t] : 0xFFFFFFFFu;
    const int eq = (t < T && k == K) ? 1 : 0;
    int eq_total;
    const int eq_rank = eq_seen + scan1024(eq, sh, &eq_total) - eq;
    const int sel = (t < T && (k < K || (eq && eq_rank < want))) ? 1 : 0;
    int sel_total;
    const int pos = sel_seen + scan1024(sel, sh, &sel_total) - sel;
    if (t < T) {
      if (sel) {
        tokens[(int64_t)e * C + pos] = (int32_t)t;
        slot[t * E + e] = e * C + pos;
      } else {
        slot[t * E + e] = -1;
      }
    }
    eq_seen += eq_total;
    sel_seen += sel_total;
  }
  if (tid == 0) {
    offsets[e] = e * C;
    if (e == E - 1) offsets[E] = E * C;
  }
}

// x_perm[r] = x[row_token[r]] for r < R: one wavefront per row, 16-byte
// copies; a token index outside [0, T) gives a zero row.
__global__ __launch_bounds__(256) void gather_rows_kernel(int64_t T, int64_t R, size_t row_bytes,
                                                          const char* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          char* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= R) return;
  const int32_t t = row_token[r];
  char* dst = x_perm + (size_t)r * row_bytes;
  if (t < 0 || t >= T) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (size_t off = (size_t)lane * 16; off < row_bytes; off += 64 * 16) st16(dst + off, z);
    return;
  }
  const char* src = x + (size_t)t * row_bytes;
  for (size_t off = (size_t)lane * 16; off < row_bytes; off += 64 * 16) st16(dst + off, ld16(src + off));
}

// y[t] = store(sum over experts e ascending with 0 <= slot[t, e] < R of
//              score[t, e] * out_perm[slot[t, e]]), fp32 from +0; one wavefront per
// token. Lane l loads slot[t, e0 + l] and score[t, e0 + l] for a group of 64
// experts; a ballot of the chosen ones is walked from the lowest set bit, so
// only chosen experts are visited, in ascending order.
template <typename S>
__global__ __launch_bounds__(256) void ec_combine_kernel(int64_t T, int d, int E, int64_t R,
                                                         const typename S::elem* __restrict__ o,
                                                         const int32_t* __restrict__ slot,
                                                         const float* __restrict__ scores,
                                                         typename S::elem* __restrict__ y) {
  constexpr int V = S::kVec;
  constexpr int MAXC = 8;   // row chunks of 64 lanes x V elements held in registers
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const char* ob = reinterpret_cast<const char*>(o);
  char* yb = reinterpret_cast<char*>(y) + (size_t)t * d * sizeof(typename S::elem);
  const size_t rb = (size_t)d * sizeof(typename S::elem);
  for (int c0 = 0; c0 < d; c0 += 64 * V * MAXC) {
    float acc[MAXC][V];
#pragma unroll
    for (int q = 0; q < MAXC; ++q)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[q][i] = 0.f;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int r_l = e < E ? slot[t * E + e] : -1;
      const float g_l = e < E ? scores[t * E + e] : 0.f;
      uint64_t m = __ballot(r_l >= 0 && r_l < R);
      while (m) {
        // up to 4 chosen experts at a time (ascending), each through its own
        // descriptor (record count 0 and weight 0 for an empty place), so the
        // loads issue together and the sum keeps the one-by-one order and bits
        __amdgpu_buffer_rsrc_t src[4];
        float g[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int sl = m ? __ffsll((unsigned long long)m) - 1 : -1;
          m &= m - 1;
          const int r = __builtin_amdgcn_readfirstlane(sl >= 0 ? __shfl(r_l, sl) : -1);
          g[j] = sl >= 0 ? __shfl(g_l, sl) : 0.f;
          src[j] = make_rsrc(ob + (size_t)(r >= 0 ? r : 0) * rb, r >= 0 ? (uint32_t)rb : 0u);
        }
#pragma unroll
        for (int q = 0; q < MAXC; ++q) {
          const int c = c0 + (q * 64 + lane) * V;
          const uint32_t off = (uint32_t)c * sizeof(typename S::elem);
          u32x4 v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = bload16(src[j], c < d ? off : 0x80000000u);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float f[V];
            unpack16(S(), v[j], f);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[q][i] = fmaf(g[j], f[i], acc[q][i]);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      const int c = c0 + (q * 64 + lane) * V;
      if (c < d) st16(yb + (size_t)c * sizeof(typename S::elem), pack16(S(), acc[q]));
    }
  }
}

}  // namespace

size_t ec_select_bytes(int64_t T, int E) { return (size_t)E * T * 4; }

hipError_t launch_ec_select(int64_t T, int E, int C, const float* scores, void* ws, int32_t* tokens,
                            int32_t* slot, int32_t* offsets, hipStream_t s) {
  if (T <= kSelLdsKeys) {
    const int bytes = (int)(T * 4);
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&ec_select_kernel<true>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)(kSelLdsKeys * 4));
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL(ec_select_kernel<true>, dim3((unsigned)E), dim3(kSelThreads), bytes, s, T, E, C, scores,
                       reinterpret_cast<uint32_t*>(ws), tokens, slot, offsets);
  } else {
    hipLaunchKernelGGL(ec_select_kernel<false>, dim3((unsigned)E), dim3(kSelThreads), 0, s, T, E, C, scores,
                       reinterpret_cast<uint32_t*>(ws), tokens, slot, offsets);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(bool bf16, int64_t T, int64_t R, int d, const void* x, const int32_t* row_token,
                              void* x_perm, hipStream_t s) {
  const size_t row_bytes = (size_t)d * (bf16 ? 2 : 4);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, T, R, row_bytes,
                     reinterpret_cast<const char*>(x), row_token, reinterpret_cast<char*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_ec_combine(bool bf16, int64_t T, int d, int E, int64_t R, const void* out_perm,
                             const int32_t* slot, const float* scores, void* y, hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(ec_combine_kernel<BF16>, grid, dim3(256), 0, s, T, d, E, R,
                       reinterpret_cast<const uint16_t*>(out_perm), slot, scores, reinterpret_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(ec_combine_kernel<F32>, grid, dim3(256), 0, s, T, d, E, R,
                       reinterpret_cast<const float*>(out_perm), slot, scores, reinterpret_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
