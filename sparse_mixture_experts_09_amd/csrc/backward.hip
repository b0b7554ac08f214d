// Backward pass of the token-choice layer (bf16), apart from its GEMMs.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts",
// MoE-layer walkthrough: the permutation is recomputed in the backward pass
// instead of being kept. The gradients follow the chain rule of the forward
// definition ("How do Mixture of Expert Models Work?", "The Math Behind
// MoEs": y = sum_j g_j E_j(x), g = Softmax(TopK(x.W_g)); SwiGLU experts).
//
// Kernels here:
//   gate_bwd         per token: dg_j = <dy, o_j>, d_o rows = bf16(g_j dy),
//                    dl = g (dg - sum g dg) (softmax over the chosen logits);
//   router_wgrad     dW_g[e] = sum over (t, j) with S_j = e of dl[t, j] x[t]
//                    (fp32 partial sums over token chunks, added in chunk order);
//   dx_final         dx[t] = bf16(sum_j dl_j W_g[S_j] + sum over kept j of dx_perm[row]).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// One wavefront per token; lane l covers the 8-element pieces l, l + 64, ... of a row.
__global__ __launch_bounds__(256) void gate_bwd_kernel(int64_t T, int d, int k, const uint16_t* __restrict__ dy,
                                                       const uint16_t* __restrict__ o,
                                                       const int32_t* __restrict__ slot_row,
                                                       const float* __restrict__ gate, uint16_t* __restrict__ d_o,
                                                       float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int rows[8];
  float g[8], dot[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    rows[j] = j < k ? slot_row[t * k + j] : -1;
    g[j] = j < k ? gate[t * k + j] : 0.f;
    dot[j] = 0.f;
  }
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float fy[8];
    unpack16(BF16(), ld16(dy + (size_t)t * d + c), fy);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float fo[8], sc[8];
      unpack16(BF16(), ld16(o + (size_t)rows[j] * d + c), fo);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        dot[j] = fmaf(fy[i], fo[i], dot[j]);
        sc[i] = g[j] * fy[i];
      }
      st16(d_o + (size_t)rows[j] * d + c, pack16(BF16(), sc));
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot[j] += __shfl_xor(dot[j], off);
    sum += g[j] * dot[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < k && lane == j) dl[t * k + j] = g[j] * (dot[j] - sum);
}

// grid (token chunks, E); a thread owns 8 consecutive columns (strided over d).
constexpr int kRouterChunk = 128;

__global__ __launch_bounds__(256) void router_wgrad_kernel(int64_t T, int d, int E, int k, const uint16_t* __restrict__ x,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ dl, float* __restrict__ partial) {
  const int e = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kRouterChunk;
  const int64_t t1 = min<int64_t>(T, t0 + kRouterChunk);
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int64_t t = t0; t < t1; ++t) {
      float w = 0.f;
      for (int j = 0; j < k; ++j)
        if (idx[t * k + j] == e) w += dl[t * k + j];
      if (w == 0.f) continue;
      float fx[8];
      unpack16(BF16(), ld16(x + (size_t)t * d + c), fx);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w, fx[i], acc[i]);
    }
    float* p = partial + ((size_t)blockIdx.x * E + e) * d + c;
    *reinterpret_cast<f32x4*>(p) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(int64_t n, int chunks, const float* __restrict__ partial,
                                                                  uint16_t* __restrict__ dwg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += partial[(size_t)c * n + i];
  dwg[i] = (uint16_t)f32_to_bf16(s);
}

__global__ __launch_bounds__(256) void dx_final_kernel(int64_t T, int d, int k, const float* __restrict__ dl,
                                                       const int32_t* __restrict__ idx,
                                                       const uint16_t* __restrict__ wr,
                                                       const uint16_t* __restrict__ dx_perm,
                                                       const int32_t* __restrict__ slot_row,
                                                       uint16_t* __restrict__ dx) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int ex[8], rows[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = j < k ? idx[t * k + j] : -1;
    rows[j] = j < k ? slot_row[t * k + j] : -1;
    w[j] = j < k ? dl[t * k + j] : 0.f;
  }
  for (int c = lane * 8; c < d; c += 64 * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (ex[j] < 0) continue;
      float f[8];
      unpack16(BF16(), ld16(wr + (size_t)ex[j] * d + c), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(w[j], f[i], acc[i]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float f[8];
      unpack16(BF16(), ld16(dx_perm + (size_t)rows[j] * d + c), f);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += f[i];
    }
    st16(dx + (size_t)t * d + c, pack16(BF16(), acc));
  }
}

}  // namespace

size_t router_wgrad_partial_bytes(int64_t T, int d, int E) {
  return (size_t)((T + kRouterChunk - 1) / kRouterChunk) * E * d * 4;
}

hipError_t launch_gate_bwd(int64_t T, int d, int k, const void* dy, const void* o, const int32_t* slot_row,
                           const float* gate, void* d_o, float* dl, hipStream_t s) {
  hipLaunchKernelGGL(gate_bwd_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, k,
                     reinterpret_cast<const uint16_t*>(dy), reinterpret_cast<const uint16_t*>(o), slot_row, gate,
                     reinterpret_cast<uint16_t*>(d_o), dl);
  return hipGetLastError();
}

hipError_t launch_router_wgrad(int64_t T, int d, int E, int k, const void* x, const int32_t* idx, const float* dl,
                               float* partial, void* dwg, hipStream_t s) {
  const int chunks = (int)((T + kRouterChunk - 1) / kRouterChunk);
  hipLaunchKernelGGL(router_wgrad_kernel, dim3((unsigned)chunks, (unsigned)E), dim3(256), 0, s, T, d, E, k,
                     reinterpret_cast<const uint16_t*>(x), idx, dl, partial);
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(router_wgrad_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, chunks,
                     partial, reinterpret_cast<uint16_t*>(dwg));
  return hipGetLastError();
}

hipError_t launch_dx_final(int64_t T, int d, int k, const float* dl, const int32_t* idx, const void* wr,
                           const void* dx_perm, const int32_t* slot_row, void* dx, hipStream_t s) {
  hipLaunchKernelGGL(dx_final_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, k, dl, idx,
                     reinterpret_cast<const uint16_t*>(wr), reinterpret_cast<const uint16_t*>(dx_perm), slot_row,
                     reinterpret_cast<uint16_t*>(dx));
  return hipGetLastError();
}

}  // namespace moe
