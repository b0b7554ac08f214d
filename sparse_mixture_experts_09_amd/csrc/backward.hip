// Backward pass of the token-choice layer (bf16 or fp32 storage), apart from its GEMMs.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts",
// MoE-layer walkthrough: the permutation is recomputed in the backward pass
// instead of being kept. The gradients follow the chain rule of the forward
// definition ("How do Mixture of Expert Models Work?", "The Math Behind
// MoEs": y = sum_j g_j E_j(x), g = Softmax(TopK(x.W_g)); SwiGLU experts).
//
// Kernels here:
//   gate_bwd         per token: dg_j = <dy, o_j>, d_o rows = bf16(g_j dy), and
//                    the logit gradient: for Softmax(TopK) gates
//                    dl_j = g_j (dg_j - sum g dg) on the chosen logits ([T, k]);
//                    for the Switch rules (g_j = s p[S_j], p the softmax over
//                    all E logits; the upcycling talk's Switch order, s = E/k
//                    when rescaled) every logit gets
//                    dl[e] = s p[e] (D[e] - sum_j p[S_j] dg_j) with D[S_j] = dg_j
//                    ([T, E], "dense");
//   router_wgrad     dW_g[e] = sum over tokens of the logit gradient at e
//                    times x[t] (fp32 partial sums over token chunks, added in
//                    chunk order);
//   dx_final         dx[t] = bf16(sum_e dl[t, e] W_g[e] + sum over kept j of dx_perm[row]).
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// One wavefront per token; lane l covers the 8-element pieces l, l + 64, ... of a row.
// logits == nullptr: Softmax(TopK) gates, dl [T, k]; otherwise the Switch
// rules with the router's logits [T, E], dl [T, E] (scale: s).
template <typename S>
__global__ __launch_bounds__(256) void gate_bwd_kernel(int64_t T, int d, int k,
                                                       const typename S::elem* __restrict__ dy,
                                                       const typename S::elem* __restrict__ o,
                                                       const int32_t* __restrict__ slot_row,
                                                       const float* __restrict__ gate,
                                                       typename S::elem* __restrict__ d_o,
                                                       float* __restrict__ dl, int E, const int32_t* __restrict__ idx,
                                                       const float* __restrict__ logits, float scale) {
  constexpr int V = S::kVec;
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
  for (int c = lane * V; c < d; c += 64 * V) {
    float fy[V];
    unpack16(S(), ld16(dy + (size_t)t * d + c), fy);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float fo[V], sc[V];
      unpack16(S(), ld16(o + (size_t)rows[j] * d + c), fo);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        dot[j] = fmaf(fy[i], fo[i], dot[j]);
        sc[i] = g[j] * fy[i];
      }
      st16(d_o + (size_t)rows[j] * d + c, pack16(S(), sc));
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot[j] += __shfl_xor(dot[j], off);
    sum += g[j] * dot[j];
  }
  if (logits == nullptr) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k && lane == j) dl[t * k + j] = g[j] * (dot[j] - sum);
    return;
  }
  // Switch rules: the softmax over all E logits of the token (lane l holds
  // experts l, l + 64, ...), its max and sum by butterflies, then every logit
  int ex[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) ex[j] = j < k ? idx[t * k + j] : -1;
  const float* lt = logits + t * E;
  float lv[4], mx = -INFINITY;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    lv[q] = e < E ? lt[e] : -INFINITY;
    mx = fmaxf(mx, lv[q]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  float z[4], den = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    z[q] = lane + 64 * q < E ? expf(lv[q] - mx) : 0.f;
    den += z[q];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) den += __shfl_xor(den, off);
  float D[4], pd = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    D[q] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (ex[j] == e && rows[j] >= 0) D[q] = dot[j];
    z[q] /= den;   // p[e]
    pd += z[q] * D[q];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pd += __shfl_xor(pd, off);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = lane + 64 * q;
    if (e < E) dl[t * E + e] = scale * z[q] * (D[q] - pd);
  }
}

// grid (token chunks, E); a thread owns 8 consecutive columns (strided over d).
constexpr int kRouterChunk = 128;

// dense: dl is [T, E] (the Switch rules), else [T, k] at the chosen experts.
template <typename S>
__global__ __launch_bounds__(256) void router_wgrad_kernel(int64_t T, int d, int E, int k,
                                                           const typename S::elem* __restrict__ x,
                                                           const int32_t* __restrict__ idx,
                                                           const float* __restrict__ dl, float* __restrict__ partial,
                                                           int dense) {
  constexpr int V = S::kVec;
  const int e = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * kRouterChunk;
  const int64_t t1 = min<int64_t>(T, t0 + kRouterChunk);
  for (int c = threadIdx.x * V; c < d; c += 256 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    for (int64_t t = t0; t < t1; ++t) {
      float w = 0.f;
      if (dense) {
        w = dl[t * E + e];
      } else {
        for (int j = 0; j < k; ++j)
          if (idx[t * k + j] == e) w += dl[t * k + j];
      }
      if (w == 0.f) continue;
      float fx[V];
      unpack16(S(), ld16(x + (size_t)t * d + c), fx);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = fmaf(w, fx[i], acc[i]);
    }
    float* p = partial + ((size_t)blockIdx.x * E + e) * d + c;
#pragma unroll
    for (int i = 0; i < V; i += 4) *reinterpret_cast<f32x4*>(p + i) = f32x4{acc[i], acc[i + 1], acc[i + 2], acc[i + 3]};
  }
}

template <typename S>
__global__ __launch_bounds__(256) void router_wgrad_reduce_kernel(int64_t n, int chunks, const float* __restrict__ partial,
                                                                  typename S::elem* __restrict__ dwg) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += partial[(size_t)c * n + i];
  if constexpr (S::kVec == 8)
    dwg[i] = (uint16_t)f32_to_bf16(s);
  else
    dwg[i] = s;
}

// E > 0: dl is dense [T, E] (the Switch rules); E == 0: [T, k] at idx.
template <typename S>
__global__ __launch_bounds__(256) void dx_final_kernel(int64_t T, int d, int k, const float* __restrict__ dl,
                                                       const int32_t* __restrict__ idx,
                                                       const typename S::elem* __restrict__ wr,
                                                       const typename S::elem* __restrict__ dx_perm,
                                                       const int32_t* __restrict__ slot_row,
                                                       typename S::elem* __restrict__ dx, int E) {
  constexpr int V = S::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  int ex[8], rows[8];
  float w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    ex[j] = j < k ? idx[t * k + j] : -1;
    rows[j] = j < k ? slot_row[t * k + j] : -1;
    w[j] = (j < k && E == 0) ? dl[t * k + j] : 0.f;
  }
  for (int c = lane * V; c < d; c += 64 * V) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    if (E > 0) {   // dense: every expert's router row
      for (int e = 0; e < E; ++e) {
        const float we = dl[t * E + e];
        float f[V];
        unpack16(S(), ld16(wr + (size_t)e * d + c), f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(we, f[i], acc[i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (ex[j] < 0) continue;
        float f[V];
        unpack16(S(), ld16(wr + (size_t)ex[j] * d + c), f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(w[j], f[i], acc[i]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (rows[j] < 0) continue;
      float f[V];
      unpack16(S(), ld16(dx_perm + (size_t)rows[j] * d + c), f);
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] += f[i];
    }
    st16(dx + (size_t)t * d + c, pack16(S(), acc));
  }
}

}  // namespace

size_t router_wgrad_partial_bytes(int64_t T, int d, int E) {
  return (size_t)((T + kRouterChunk - 1) / kRouterChunk) * E * d * 4;
}

template <typename S>
static hipError_t gate_bwd_t(int64_t T, int d, int k, const void* dy, const void* o, const int32_t* slot_row,
                             const float* gate, void* d_o, float* dl, hipStream_t s, int E, const int32_t* idx,
                             const float* logits, float scale) {
  using P = typename S::elem;
  hipLaunchKernelGGL(gate_bwd_kernel<S>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, k,
                     reinterpret_cast<const P*>(dy), reinterpret_cast<const P*>(o), slot_row, gate,
                     reinterpret_cast<P*>(d_o), dl, E, idx, logits, scale);
  return hipGetLastError();
}

hipError_t launch_gate_bwd(int64_t T, int d, int k, const void* dy, const void* o, const int32_t* slot_row,
                           const float* gate, void* d_o, float* dl, hipStream_t s, int E, const int32_t* idx,
                           const float* logits, float scale, bool bf16) {
  return bf16 ? gate_bwd_t<BF16>(T, d, k, dy, o, slot_row, gate, d_o, dl, s, E, idx, logits, scale)
              : gate_bwd_t<F32>(T, d, k, dy, o, slot_row, gate, d_o, dl, s, E, idx, logits, scale);
}

template <typename S>
static hipError_t router_wgrad_t(int64_t T, int d, int E, int k, const void* x, const int32_t* idx, const float* dl,
                                 float* partial, void* dwg, hipStream_t s, bool dense) {
  using P = typename S::elem;
  const int chunks = (int)((T + kRouterChunk - 1) / kRouterChunk);
  hipLaunchKernelGGL(router_wgrad_kernel<S>, dim3((unsigned)chunks, (unsigned)E), dim3(256), 0, s, T, d, E, k,
                     reinterpret_cast<const P*>(x), idx, dl, partial, dense ? 1 : 0);
  const int64_t n = (int64_t)E * d;
  hipLaunchKernelGGL(router_wgrad_reduce_kernel<S>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, n, chunks,
                     partial, reinterpret_cast<P*>(dwg));
  return hipGetLastError();
}

hipError_t launch_router_wgrad(int64_t T, int d, int E, int k, const void* x, const int32_t* idx, const float* dl,
                               float* partial, void* dwg, hipStream_t s, bool dense, bool bf16) {
  return bf16 ? router_wgrad_t<BF16>(T, d, E, k, x, idx, dl, partial, dwg, s, dense)
              : router_wgrad_t<F32>(T, d, E, k, x, idx, dl, partial, dwg, s, dense);
}

template <typename S>
static hipError_t dx_final_t(int64_t T, int d, int k, const float* dl, const int32_t* idx, const void* wr,
                             const void* dx_perm, const int32_t* slot_row, void* dx, hipStream_t s, int dense_E) {
  using P = typename S::elem;
  hipLaunchKernelGGL(dx_final_kernel<S>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, k, dl, idx,
                     reinterpret_cast<const P*>(wr), reinterpret_cast<const P*>(dx_perm), slot_row,
                     reinterpret_cast<P*>(dx), dense_E);
  return hipGetLastError();
}

hipError_t launch_dx_final(int64_t T, int d, int k, const float* dl, const int32_t* idx, const void* wr,
                           const void* dx_perm, const int32_t* slot_row, void* dx, hipStream_t s, int dense_E,
                           bool bf16) {
  return bf16 ? dx_final_t<BF16>(T, d, k, dl, idx, wr, dx_perm, slot_row, dx, s, dense_E)
              : dx_final_t<F32>(T, d, k, dl, idx, wr, dx_perm, slot_row, dx, s, dense_E);
}

}  // namespace moe
