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
// The loads of several slices are issued together before the sums.
// Each slot reads through a buffer descriptor of its own (base at its row,
// record count one row, or 0 for a dropped slot, whose gate is taken as 0),
// so the k loads carry no branch and issue together; a dropped slot adds
// 0 * 0 to a sum that started at +0, which leaves every bit of it unchanged.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

template <typename S, int KM>
__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int d, int k,
                                                      const char* __restrict__ out_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gate,
                                                      char* __restrict__ y) {
  constexpr int V = S::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const uint32_t row_bytes = (uint32_t)d * sizeof(typename S::elem);
  __amdgpu_buffer_rsrc_t src[KM];   // KM: k rounded up to 1, 2, 4 or 8
  float g[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    // the same for every lane (one token per wavefront)
    const int r = __builtin_amdgcn_readfirstlane(j < k ? slot_row[t * k + j] : -1);
    g[j] = r >= 0 ? gate[t * k + j] : 0.f;
    src[j] = make_rsrc(out_perm + (size_t)(r >= 0 ? r : 0) * row_bytes, r >= 0 ? row_bytes : 0u);
  }
  char* dst = y + (size_t)t * row_bytes;
  // U slices (1 KB of the row each) of all k rows are loaded before any is
  // used: 16 loads of 16 bytes in flight a lane (an 8 KB row at k = 2 in one
  // batch). Offsets past the row read zeros (the record count) and are not
  // stored.
  constexpr int U = KM >= 8 ? 2 : 16 / KM;
  for (uint32_t base = (uint32_t)lane * 16; base < row_bytes; base += U * 64 * 16) {
    u32x4 v[U][KM];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < KM; ++j) v[u][j] = bload16<2>(src[j], base + u * 1024);   // read once: nontemporal
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = base + u * 1024;
      if (off >= row_bytes) break;
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        float f[V];
        unpack16(S(), v[u][j], f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(g[j], f[i], acc[i]);
      }
      st16(dst + off, pack16(S(), acc));
    }
  }
}

template <typename S, int KM>
hipError_t launch_combine_k(int64_t T, int d, int k, const void* out_perm, const int32_t* slot_row, const float* gate,
                            void* y, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<S, KM>), dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, k,
                     reinterpret_cast<const char*>(out_perm), slot_row, gate, reinterpret_cast<char*>(y));
  return hipGetLastError();
}

template <typename S>
hipError_t launch_combine_s(int64_t T, int d, int k, const void* out_perm, const int32_t* slot_row,
                            const float* gate, void* y, hipStream_t s) {
  if (k <= 1) return launch_combine_k<S, 1>(T, d, k, out_perm, slot_row, gate, y, s);
  if (k <= 2) return launch_combine_k<S, 2>(T, d, k, out_perm, slot_row, gate, y, s);
  if (k <= 4) return launch_combine_k<S, 4>(T, d, k, out_perm, slot_row, gate, y, s);
  return launch_combine_k<S, 8>(T, d, k, out_perm, slot_row, gate, y, s);
}

}  // namespace

hipError_t launch_combine(bool bf16, int64_t T, int d, int k, const void* out_perm,
                          const int32_t* slot_row, const float* gate, void* y, hipStream_t s) {
  return bf16 ? launch_combine_s<BF16>(T, d, k, out_perm, slot_row, gate, y, s)
              : launch_combine_s<F32>(T, d, k, out_perm, slot_row, gate, y, s);
}

}  // namespace moe
