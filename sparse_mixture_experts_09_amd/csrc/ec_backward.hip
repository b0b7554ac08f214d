// Backward pass of the expert-choice layer, apart from its GEMMs.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts", the
// Q&A on expert choice: each expert selects a fixed number of tokens, so a
// token gets anywhere from zero to all experts. The gate of (t, e) is the
// dense score S[t, e] = Softmax(x.W_g)[e] ("How do Mixture of Expert Models
// Work?", "The Math Behind MoEs"); the selection itself is a discrete decision
// and passes no gradient. With y[t] = sum over the experts e that chose t of
// S[t, e] o[slot[t, e]] the chain rule gives, per token:
//   dS[t, e]  = <dy[t], o[row]>          (0 for an expert that did not choose t)
//   d_o[row]  = store(S[t, e] dy[t])
//   dl[t, :]  = S[t, :] (dS[t, :] - sum_e S[t, e] dS[t, e])   (softmax Jacobian)
//   dx[t]     = store(dl[t] W_g + sum over the choosing experts of dx_perm[row])
// The router weight gradient dW_g = dl^T x is the dense path of the
// token-choice router_wgrad kernels.
//
// Kernels here (one wavefront per token; lane l covers the 16-byte slices
// l, l + 64, ... of a row):
//   ec_gate_bwd   dS, d_o and dl. The chosen experts of the token are found by
//                 a ballot over slot[t, e0 + lane] and visited in ascending order;
//                 lane (e mod 64) keeps dS[t, e] and S[t, e] for the softmax step.
//   ec_dx_final   dx from dl, W_g and the dx_perm rows of the choosing experts.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kMaxGroups = 4;   // E <= 256: four groups of 64 experts, one score per lane each

template <typename S>
__global__ __launch_bounds__(256) void ec_gate_bwd_kernel(int64_t T, int d, int E, int64_t R,
                                                          const typename S::elem* __restrict__ dy,
                                                          const typename S::elem* __restrict__ o,
                                                          const int32_t* __restrict__ slot,
                                                          const float* __restrict__ scores,
                                                          typename S::elem* __restrict__ d_o,
                                                          float* __restrict__ dl) {
  constexpr int V = S::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const typename S::elem* dyt = dy + (size_t)t * d;
  float sc[kMaxGroups], D[kMaxGroups];
#pragma unroll
  for (int q = 0; q < kMaxGroups; ++q) {
    const int e = 64 * q + lane;
    sc[q] = e < E ? scores[t * E + e] : 0.f;
    D[q] = 0.f;
    if (64 * q >= E) continue;   // wave-uniform
    const int r_l = e < E ? slot[t * E + e] : -1;
    uint64_t m = __ballot(r_l >= 0 && r_l < R);
    while (m) {
      const int sl = __ffsll((unsigned long long)m) - 1;
      m &= m - 1;
      const int r = __builtin_amdgcn_readfirstlane(__shfl(r_l, sl));
      const float g = __shfl(sc[q], sl);
      const typename S::elem* orow = o + (size_t)r * d;
      typename S::elem* drow = d_o + (size_t)r * d;
      float dot = 0.f;
      for (int c = lane * V; c < d; c += 64 * V) {
        float fy[V], fo[V], v[V];
        unpack16(S(), ld16(dyt + c), fy);
        unpack16(S(), ld16(orow + c), fo);
#pragma unroll
        for (int i = 0; i < V; ++i) {
          dot = fmaf(fy[i], fo[i], dot);
          v[i] = g * fy[i];
        }
        st16(drow + c, pack16(S(), v));
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
      if (lane == sl) D[q] = dot;
    }
  }
  float pd = 0.f;
#pragma unroll
  for (int q = 0; q < kMaxGroups; ++q) pd += sc[q] * D[q];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) pd += __shfl_xor(pd, off);
#pragma unroll
  for (int q = 0; q < kMaxGroups; ++q) {
    const int e = 64 * q + lane;
    if (e < E) dl[t * E + e] = sc[q] * (D[q] - pd);
  }
}

template <typename S>
__global__ __launch_bounds__(256) void ec_dx_final_kernel(int64_t T, int d, int E, int64_t R,
                                                          const float* __restrict__ dl,
                                                          const typename S::elem* __restrict__ wr,
                                                          const typename S::elem* __restrict__ dx_perm,
                                                          const int32_t* __restrict__ slot,
                                                          typename S::elem* __restrict__ dx) {
  constexpr int V = S::kVec;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // The column loop is the same for every lane (a lane past the row's end
  // idles), so the ballots over the token's experts see the whole wavefront.
  for (int c0 = 0; c0 < d; c0 += 64 * V) {
    const int c = c0 + lane * V;
    const bool on = c < d;
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.f;
    if (on) {
      for (int e = 0; e < E; ++e) {
        const float we = dl[t * E + e];
        float f[V];
        unpack16(S(), ld16(wr + (size_t)e * d + c), f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(we, f[i], acc[i]);
      }
    }
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int r_l = e < E ? slot[t * E + e] : -1;
      uint64_t m = __ballot(r_l >= 0 && r_l < R);
      while (m) {
        const int sl = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const int r = __builtin_amdgcn_readfirstlane(__shfl(r_l, sl));
        if (on) {
          float f[V];
          unpack16(S(), ld16(dx_perm + (size_t)r * d + c), f);
#pragma unroll
          for (int i = 0; i < V; ++i) acc[i] += f[i];
        }
      }
    }
    if (on) st16(dx + (size_t)t * d + c, pack16(S(), acc));
  }
}

template <typename S>
hipError_t ec_gate_bwd_t(int64_t T, int d, int E, int64_t R, const void* dy, const void* o, const int32_t* slot,
                         const float* scores, void* d_o, float* dl, hipStream_t s) {
  using P = typename S::elem;
  hipLaunchKernelGGL(ec_gate_bwd_kernel<S>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, E, R,
                     reinterpret_cast<const P*>(dy), reinterpret_cast<const P*>(o), slot, scores,
                     reinterpret_cast<P*>(d_o), dl);
  return hipGetLastError();
}

template <typename S>
hipError_t ec_dx_final_t(int64_t T, int d, int E, int64_t R, const float* dl, const void* wr, const void* dx_perm,
                         const int32_t* slot, void* dx, hipStream_t s) {
  using P = typename S::elem;
  hipLaunchKernelGGL(ec_dx_final_kernel<S>, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, T, d, E, R, dl,
                     reinterpret_cast<const P*>(wr), reinterpret_cast<const P*>(dx_perm), slot,
                     reinterpret_cast<P*>(dx));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ec_gate_bwd(bool bf16, int64_t T, int d, int E, int64_t R, const void* dy, const void* o,
                              const int32_t* slot, const float* scores, void* d_o, float* dl, hipStream_t s) {
  return bf16 ? ec_gate_bwd_t<BF16>(T, d, E, R, dy, o, slot, scores, d_o, dl, s)
              : ec_gate_bwd_t<F32>(T, d, E, R, dy, o, slot, scores, d_o, dl, s);
}

hipError_t launch_ec_dx_final(bool bf16, int64_t T, int d, int E, int64_t R, const float* dl, const void* wr,
                              const void* dx_perm, const int32_t* slot, void* dx, hipStream_t s) {
  return bf16 ? ec_dx_final_t<BF16>(T, d, E, R, dl, wr, dx_perm, slot, dx, s)
              : ec_dx_final_t<F32>(T, d, E, R, dl, wr, dx_perm, slot, dx, s);
}

}  // namespace moe
