// Router: logits = x . W_g^T, arg-top-k and softmax over the chosen logits.
//
// "How do Mixture of Expert Models Work?", section "The Math Behind MoEs":
// G(x) = Softmax(TopK(x.W_g)), the softmax of only the k largest logits with
// every other gate 0. "[Paper Club] Upcycling Large Language Models into
// Mixture of Experts": the router is a plain learnable matrix multiply; its
// upcycling part also gives the Switch-Transformer order (softmax over all E
// experts first, then the top k, whose probabilities no longer sum to one)
// and the E/k rescale of the expert outputs, applied here to the kept gates.
//
// gating: 0 = Softmax(TopK(l)); 1 = TopK(Softmax(l)); 2 = the same times E/k.
// The chosen experts are the same in every mode (softmax is monotone).
// gating 3 (expert choice): no top-k; logits_out receives the dense gate
// Softmax(l) over all E experts ("How do Mixture of Expert Models Work?",
// "The Math Behind MoEs"), the score each expert ranks the tokens by.
//
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

// (v1, i1) beats (v2, i2): larger value, ties to the lower index.
__device__ __forceinline__ bool beats(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// Softmax denominator over all E logits of one token held by a group of L
// lanes (lane bits below L), each lane adding exp(v - vmax) over its own
// experts (part). The group's first lane's total is broadcast, so every gate
// of the token uses one value.
template <int L>
__device__ __forceinline__ float group_sum(float part, int lane) {
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1) part += __shfl_xor(part, o);
  return __shfl(part, lane & ~(L - 1));
}


// ---------------------------------------------------------------------------
// fp32 router: a wavefront owns TW consecutive tokens and
// lane l covers the 16-byte slices l, l+64, ... of each token row, so x is read
// once with coalesced loads; experts go in passes of 8, each lane accumulating
// TW x 8 partial dot products that one transposed wave reduction completes.
// The W_g slices come from L2/L1; TW tokens share every W_g load. bf16 data
// goes to the matrix-core kernel below.
// ---------------------------------------------------------------------------

constexpr int kRouterWaves = 4;
constexpr int kEPass = 8;

__device__ __forceinline__ float dot16(F32, const u32x4& xv, const u32x4& wv, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(xv[i]), __uint_as_float(wv[i]), acc);
  return acc;
}

template <typename S, int TW>
__global__ __launch_bounds__(256) void router_kernel(int64_t T, int d, int E, int k, int gating,
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
      if (gating != 3 && logits_out != nullptr && e < E) logits_out[t * E + e] = v[q];
    }
    if (gating == 3) {
      float mx = -INFINITY;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) mx = fmaxf(mx, v[q]);
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) part += expf(v[q] - mx);
      const float den = group_sum<64>(part, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) logits_out[t * E + lane + 64 * q] = expf(v[q] - mx) / den;
      continue;
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
    // softmax over the k chosen logits (largest first), or over all E
    float s = 0.f;
    float ex[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k) {
        ex[j] = expf(sel_v[j] - sel_v[0]);
        s += ex[j];
      }
    }
    float scale = 1.f;
    if (gating != 0) {
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (lane + 64 * q < E) part += expf(v[q] - sel_v[0]);
      s = group_sum<64>(part, lane);
      if (gating == 2) scale = (float)E / (float)k;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j < k && lane == j) {
        topk_idx[t * k + j] = sel_i[j];
        topk_gate[t * k + j] = ex[j] / s * scale;
      }
    }
  }
}

template <typename S, int TW>
hipError_t launch_router_tw(int64_t T, int d, int E, int k, int gating, const void* x, const void* wr,
                            int32_t* idx, float* gate, float* logits, hipStream_t s) {
  const int64_t per_block = (int64_t)kRouterWaves * TW;
  const int64_t blocks = (T + per_block - 1) / per_block;
  hipLaunchKernelGGL((router_kernel<S, TW>), dim3((unsigned)blocks), dim3(256), 0, s, T, d, E, k, gating,
                     reinterpret_cast<const typename S::elem*>(x),
                     reinterpret_cast<const typename S::elem*>(wr), idx, gate, logits);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// bf16 router on the matrix cores. The logits are a [T, d] x [d, E] product
// with E small, so the work is bound by reading x from HBM once. A block owns
// BT = 16 * MT tokens; its NW wavefronts split d: the 128-column steps of d go
// round-robin to the wavefronts, which issue the W_g loads of D steps and then
// the x loads of those steps at once before computing on them (W_g comes from
// L2 and lands first, so a step's MFMAs start as soon as its x pieces arrive). In a step, lane l of a wavefront holds row l % 16
// of each 16-token tile and of each 16-expert tile of W_g, with the 16-byte
// pieces at columns 32 j + 8 (l / 16) (j = 0..3), which is the operand layout
// of v_mfma_f32_16x16x32_bf16 for the 32 columns of piece j. W_g is the first
// operand, so lane l ends up holding experts 4 (l / 16) .. + 3 of token l % 16.
// bf16 products are exact in fp32 and the sums are fp32, as in the plain dot
// product. The NW partial logit tiles meet in LDS and are added in wavefront
// order (a fixed order: the logits do not depend on timing). Arg-top-k then
// runs per token on LPT lanes that hold EPL experts each.
// ---------------------------------------------------------------------------

constexpr int kRStep = 128;   // d columns per step

template <int NT>
struct RouterSel {   // lanes per token and experts per lane for the arg-top-k
  static constexpr int LPT = NT <= 4 ? 16 : (NT == 8 ? 32 : 64);
  static constexpr int EPL = 16 * NT / LPT;
};

template <int NT, int MT, int NW>
constexpr size_t router_mfma_lds() {
  return (size_t)NW * 16 * MT * (16 * NT + 4) * sizeof(float);
}

template <int NT, int MT, int NW, int D>
__global__ __launch_bounds__(NW * 64) void router_mfma_kernel(int64_t T, int d, int E, int k, int gating,
                                                              const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wr,
                                                              int32_t* __restrict__ topk_idx,
                                                              float* __restrict__ topk_gate,
                                                              float* __restrict__ logits_out) {
  constexpr int BT = 16 * MT;
  constexpr int EP = 16 * NT;
  constexpr int RS = EP + 4;   // floats per LDS row of partial logits
  constexpr int LPT = RouterSel<NT>::LPT, EPL = RouterSel<NT>::EPL;
  extern __shared__ __align__(16) float red[];   // [NW][BT][RS]

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const size_t rb = (size_t)d * 2;
  const char* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t t = min<int64_t>(t0 + mt * 16 + r16, T - 1);   // rows past T: results unused
    xr[mt] = reinterpret_cast<const char*>(x) + (size_t)t * rb;
  }
  const char* wrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int e = min(nt * 16 + r16, E - 1);   // experts past E: results unused
    wrow[nt] = reinterpret_cast<const char*>(wr) + (size_t)e * rb;
  }

  f32x4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const u32x4 zero = {0u, 0u, 0u, 0u};
  const int S = (d + kRStep - 1) / kRStep;
  // W_g pieces of all D steps up front while they fit in registers (up to 32
  // pieces a lane); beyond that, per step and expert tile after the x loads
  constexpr bool kPre = D * NT <= 8;
  for (int s0 = wave; s0 < S; s0 += NW * D) {
    bf16x8 bw[kPre ? D : 1][kPre ? NT : 1][4];
#pragma unroll
    for (int i = 0; i < (kPre ? D : 0); ++i) {
      const int c = (s0 + i * NW) * kRStep + 8 * g;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bw[i][nt][j] = __builtin_bit_cast(
              bf16x8, (s0 + i * NW < S && c + 32 * j < d) ? ld16(wrow[nt] + (size_t)(c + 32 * j) * 2) : zero);
    }
    bf16x8 a[D][MT][4];
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const int c = (s0 + i * NW) * kRStep + 8 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = s0 + i * NW < S && c + 32 * j < d;   // d is a multiple of 8: whole pieces
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          a[i][mt][j] = __builtin_bit_cast(bf16x8, in ? ld16(xr[mt] + (size_t)(c + 32 * j) * 2) : zero);
      }
    }
#pragma unroll
    for (int i = 0; i < D; ++i) {
      if (s0 + i * NW >= S) break;
      const int c = (s0 + i * NW) * kRStep + 8 * g;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bf16x8 bl[4];
        if constexpr (!kPre) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            bl[j] = __builtin_bit_cast(bf16x8, c + 32 * j < d ? ld16(wrow[nt] + (size_t)(c + 32 * j) * 2) : zero);
        }
        const bf16x8* b = kPre ? bw[kPre ? i : 0][kPre ? nt : 0] : bl;   // (indices 0 when unused)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[j], a[i][mt][j], acc[mt][nt], 0, 0, 0);
      }
    }
  }

  // partial tiles to LDS, then the sum over wavefronts in wavefront order
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(&red[(wave * BT + mt * 16 + r16) * RS + nt * 16 + 4 * g]) = acc[mt][nt];
  __syncthreads();
  for (int q = threadIdx.x; q < BT * EP; q += NW * 64) {
    const int row = q / EP, col = q % EP;
    float v = red[row * RS + col];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[(w * BT + row) * RS + col];
    red[row * RS + col] = v;   // only this thread touches (row, col) of any wavefront
  }
  __syncthreads();

  // arg-top-k and softmax, one token per LPT lanes
  constexpr int TS = 64 / LPT;
  const int slot = lane / LPT, el = lane % LPT;
  for (int tb = wave * TS; tb < BT; tb += NW * TS) {
    const int tl = tb + slot;
    const int64_t t = t0 + tl;
    const bool live = tl < BT && t < T;
    float v[EPL];
    bool taken[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = el + LPT * j;
      taken[j] = e >= E;
      v[j] = (tl < BT && e < E) ? red[tl * RS + e] : 0.f;
      if (gating != 3 && logits_out != nullptr && live && e < E) logits_out[t * E + e] = v[j];
    }
    if (gating == 3) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (el + LPT * j < E) mx = fmaxf(mx, v[j]);
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (el + LPT * j < E) part += expf(v[j] - mx);
      const float den = group_sum<LPT>(part, lane);
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = el + LPT * j;
        if (live && e < E) logits_out[t * E + e] = expf(v[j] - mx) / den;
      }
      continue;
    }
    float sel_v[8];
    int sel_i[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r >= k) break;
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int e = el + LPT * j;
        if (!taken[j] && beats(v[j], e, bv, bi)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int o = LPT / 2; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (beats(ov, oi, bv, bi)) {
          bv = ov;
          bi = oi;
        }
      }
      sel_v[r] = bv;
      sel_i[r] = bi;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (el + LPT * j == bi) taken[j] = true;
    }
    float ssum = 0.f;
    float ex[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if (r < k) {
        ex[r] = expf(sel_v[r] - sel_v[0]);
        ssum += ex[r];
      }
    }
    float scale = 1.f;
    if (gating != 0) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (el + LPT * j < E) part += expf(v[j] - sel_v[0]);
      ssum = group_sum<LPT>(part, lane);
      if (gating == 2) scale = (float)E / (float)k;
    }
    if (live) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        if (r < k && el == r) {
          topk_idx[t * k + r] = sel_i[r];
          topk_gate[t * k + r] = ex[r] / ssum * scale;
        }
      }
    }
  }
}

template <int NT, int MT, int NW, int D>
hipError_t launch_router_mfma(int64_t T, int d, int E, int k, int gating, const void* x, const void* wr,
                              int32_t* idx, float* gate, float* logits, hipStream_t s) {
  constexpr size_t kLds = router_mfma_lds<NT, MT, NW>();
  auto kern = &router_mfma_kernel<NT, MT, NW, D>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = (T + 16 * MT - 1) / (16 * MT);
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(NW * 64), kLds, s, T, d, E, k, gating,
                     reinterpret_cast<const uint16_t*>(x), reinterpret_cast<const uint16_t*>(wr), idx, gate,
                     logits);
  return hipGetLastError();
}

template <int NT>
hipError_t launch_router_nt(int64_t T, int d, int E, int k, int gating, const void* x, const void* wr,
                            int32_t* idx, float* gate, float* logits, hipStream_t s) {
  // 32-token blocks once they still give every compute unit a block: each
  // block reads all of W_g, so larger blocks halve that traffic
  constexpr int NW = NT <= 4 ? 8 : 4;
  if (T >= 32 * (int64_t)compute_units())
    return launch_router_mfma<NT, 2, NW, 2>(T, d, E, k, gating, x, wr, idx, gate, logits, s);
  return launch_router_mfma<NT, 1, NW, 4>(T, d, E, k, gating, x, wr, idx, gate, logits, s);
}

hipError_t launch_router_f32(int64_t T, int d, int E, int k, int g, const void* x, const void* wr, int32_t* idx,
                             float* gate, float* logits, hipStream_t s) {
  // tokens per wavefront: enough waves to fill the chip first, then reuse of
  // each W_g load across tokens
  const int64_t waves_wanted = 4096;
  if (T >= waves_wanted * 8) return launch_router_tw<F32, 8>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  if (T >= waves_wanted * 4) return launch_router_tw<F32, 4>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  if (T >= waves_wanted * 2) return launch_router_tw<F32, 2>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  return launch_router_tw<F32, 1>(T, d, E, k, g, x, wr, idx, gate, logits, s);
}

hipError_t launch_router_bf16(int64_t T, int d, int E, int k, int g, const void* x, const void* wr,
                              int32_t* idx, float* gate, float* logits, hipStream_t s) {
  if (E <= 16) return launch_router_nt<1>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  if (E <= 32) return launch_router_nt<2>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  if (E <= 64) return launch_router_nt<4>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  if (E <= 128) return launch_router_nt<8>(T, d, E, k, g, x, wr, idx, gate, logits, s);
  return launch_router_nt<16>(T, d, E, k, g, x, wr, idx, gate, logits, s);
}

}  // namespace

hipError_t launch_router(bool bf16, int64_t T, int d, int E, int k, int gating, const void* x, const void* wr,
                         int32_t* idx, float* gate, float* logits, hipStream_t s) {
  if (bf16) return launch_router_bf16(T, d, E, k, gating, x, wr, idx, gate, logits, s);
  return launch_router_f32(T, d, E, k, gating, x, wr, idx, gate, logits, s);
}

}  // namespace moe
