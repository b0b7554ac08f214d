// Un-permute and gate-weighted combine, one gather-reduce pass.
//
// "How do Mixture of Expert Models Work?", section "The Math Behind MoEs":
// y = sum_i G(x)_i E_i(x). "[Paper Club] Upcycling Large Language Models into
// Mixture of Experts", the walkthrough: arrange the expert outputs back into
// the token order, then scale by the router probability. A dropped slot
// contributes nothing ("Load Balancing", Expert Capacity: overflow tokens skip
// the layer), so a token with every slot dropped gets y = 0.
//
// One wavefront per token: lane l handles the 16-byte slices l, l+64, ... of
// the row; for each slice it reads the k expert-output rows (in slot order),
// accumulates gate * value in fp32 from +0 and writes the rounded sum once.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

template <typename S>
__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int d, int k,
                                                      const char* __restrict__ out_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate,
                                                      char* __restrict__ y) {
  constexpr int V = S::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[8];
  float g[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? slot_row[t * k + j] : -1;
    g[j] = j < k ? gate[t * k + j] : 0.f;
  }
  const size_t row_bytes = (size_t)d * sizeof(typename S::elem);
  char* dst = y + (size_t)t * row_bytes;
#pragma unroll 2
  for (size_t off = (size_t)lane * 16; off < row_bytes; off += 64 * 16) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] >= 0) {
        float f[V];
        unpack16(S(), ld16(out_perm + (size_t)rows[j] * row_bytes + off), f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(g[j], f[i], acc[i]);
      }
    }
    st16(dst + off, pack16(S(), acc));
  }
}

}  // namespace

hipError_t launch_combine(bool bf16, int64_t T, int d, int k, const void* out_perm,
                          const int32_t* slot_row, const float* gate, void* y, hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<BF16>, grid, block, 0, s, T, d, k,
                       reinterpret_cast<const char*>(out_perm), slot_row, gate,
                       reinterpret_cast<char*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<F32>, grid, block, 0, s, T, d, k,
                       reinterpret_cast<const char*>(out_perm), slot_row, gate,
                       reinterpret_cast<char*>(y));
  return hipGetLastError();
}

}  // namespace moe
