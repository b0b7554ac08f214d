// Router: logits = x . W_g^T, arg-top-k and softmax over the chosen logits.
//
// "How do Mixture of Expert Models Work?", section "The Math Behind MoEs":
// G(x) = Softmax(TopK(x.W_g)), the softmax of only the k largest logits with
// every other gate 0. "[Paper Club] Upcycling Large Language Models into
// Mixture of Experts": the router is a plain learnable matrix multiply.
//
// Layout of the work: a block is 4 wavefronts; each wavefront owns TW
// consecutive tokens. Lane l covers the 16-byte slices l, l+64, l+128, ... of
// a token row, so every x row is read once with coalesced 16-byte loads. The
// experts are processed in passes of 8: a lane accumulates TW x 8 partial dot
// products (bf16 widened exactly to fp32, then fma), then one transposed
// wave reduction leaves every (token, expert) total in some lane. The logits
// go to LDS and the arg-top-k runs per token over one wavefront: each lane
// holds up to four experts (E <= 256), and k rounds of a 64-lane butterfly
// argmax on (value desc, index asc) pick the experts in slot order.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kRouterWaves = 4;
constexpr int kEPass = 8;

// bf16 values widen exactly to fp32; products and sums are plain fp32 fma.
__device__ __forceinline__ float dot16(BF16, const u32x4& xv, const u32x4& wv, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(bf16_lo(xv[i]), bf16_lo(wv[i]), acc);
    acc = fmaf(bf16_hi(xv[i]), bf16_hi(wv[i]), acc);
  }
  return acc;
}
__device__ __forceinline__ float dot16(F32, const u32x4& xv, const u32x4& wv, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(xv[i]), __uint_as_float(wv[i]), acc);
  return acc;
}

// (v1, i1) beats (v2, i2): larger value, ties to the lower index.
__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <typename S, int TW>
__global__ __launch_bounds__(256) void router_kernel(int64_t T, int d, int E, int k,
                                                     const typename S::elem* __restrict__ x,
                                                     const typename S::elem* __restrict__ wr,
                                                     int32_t* __restrict__ topk_idx,
                                                     float* __restrict__ topk_gate,
                                                     float* __restrict__ logits_out) {
  constexpr int V = TW * kEPass;
  constexpr int kShift = 6 - Log2<V>::value;
  __shared__ float lg[kRouterWaves][TW][256];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t t0 = ((int64_t)blockIdx.x * kRouterWaves + wave) * TW;
  const int nt = t0 < T ? (int)min<int64_t>(TW, T - t0) : 0;
  const int vec = S::kVec;
  const size_t row_bytes = (size_t)d * sizeof(typename S::elem);
  const char* xb = reinterpret_cast<const char*>(x);
  const char* wb = reinterpret_cast<const char*>(wr);

  if (nt > 0) {
    for (int e0 = 0; e0 < E; e0 += kEPass) {
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      for (int c = lane * vec; c < d; c += kWave * vec) {
        const size_t off = (size_t)c * sizeof(typename S::elem);
        u32x4 xv[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
          const int ti = i < nt ? i : 0;   // rows past T reuse row t0; results unused
          xv[i] = ld16(xb + (size_t)(t0 + ti) * row_bytes + off);
        }
#pragma unroll
        for (int ee = 0; ee < kEPass; ++ee) {
          const int e = e0 + ee < E ? e0 + ee : E - 1;
          const u32x4 wv = ld16(wb + (size_t)e * row_bytes + off);
#pragma unroll
          for (int i = 0; i < TW; ++i) acc[i * kEPass + ee] = dot16(S(), xv[i], wv, acc[i * kEPass + ee]);
        }
      }
      wave_transpose_sum<V>(acc, lane);
      const int q = lane >> kShift;            // value index this lane now holds
      const int ti = q / kEPass, e = e0 + q % kEPass;
      if ((lane & ((1 << kShift) - 1)) == 0 && e < E) lg[wave][ti][e] = acc[0];
    }
  }
  __syncthreads();
  if (nt == 0) return;

  for (int i = 0; i < nt; ++i) {
    const int64_t t = t0 + i;
    float v[4];
    bool taken[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = e < E ? lg[wave][i][e] : 0.f;
      taken[q] = e >= E;
      if (logits_out != nullptr && e < E) logits_out[t * E + e] = v[q];
    }
    float sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= k) break;
      // local best among this lane's untaken experts
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (!taken[q] && beats(v[q], e, bv, bi)) {
          bv = v[q];
          bi = e;
        }
      }
      // butterfly argmax over the wave; every lane ends with the winner
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (beats(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel_v[j] = bv;
      sel_i[j] = bi;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q == bi) taken[q] = true;
    }
    // softmax over the k chosen logits, largest first
    float s = 0.f;
    float ex[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ex[j] = expf(sel_v[j] - sel_v[0]);
        s += ex[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k && lane == j) {
        topk_idx[t * k + j] = sel_i[j];
        topk_gate[t * k + j] = ex[j] / s;
      }
    }
  }
}

template <typename S, int TW>
hipError_t launch_router_tw(int64_t T, int d, int E, int k, const void* x, const void* wr,
                            int32_t* idx, float* gate, float* logits, hipStream_t s) {
  const int64_t per_block = (int64_t)kRouterWaves * TW;
  const int64_t blocks = (T + per_block - 1) / per_block;
  hipLaunchKernelGGL((router_kernel<S, TW>), dim3((unsigned)blocks), dim3(256), 0, s, T, d, E, k,
                     reinterpret_cast<const typename S::elem*>(x),
                     reinterpret_cast<const typename S::elem*>(wr), idx, gate, logits);
  return hipGetLastError();
}

template <typename S>
hipError_t launch_router_s(int64_t T, int d, int E, int k, const void* x, const void* wr,
                           int32_t* idx, float* gate, float* logits, hipStream_t s) {
  // Tokens per wavefront: enough waves to fill the chip first, then reuse of
  // each W_g load across tokens.
  const int64_t waves_wanted = 4096;
  if (T >= waves_wanted * 8) return launch_router_tw<S, 8>(T, d, E, k, x, wr, idx, gate, logits, s);
  if (T >= waves_wanted * 4) return launch_router_tw<S, 4>(T, d, E, k, x, wr, idx, gate, logits, s);
  if (T >= waves_wanted * 2) return launch_router_tw<S, 2>(T, d, E, k, x, wr, idx, gate, logits, s);
  return launch_router_tw<S, 1>(T, d, E, k, x, wr, idx, gate, logits, s);
}

}  // namespace

hipError_t launch_router(bool bf16, int64_t T, int d, int E, int k, const void* x, const void* wr,
                         int32_t* idx, float* gate, float* logits, hipStream_t s) {
  if (bf16) return launch_router_s<BF16>(T, d, E, k, x, wr, idx, gate, logits, s);
  return launch_router_s<F32>(T, d, E, k, x, wr, idx, gate, logits, s);
}

}  // namespace moe
