// Grouped SwiGLU expert FFN, fp32 storage and true fp32 multiply-add.
//
// Same products as the bf16 path ("The Math Behind MoEs": Mixtral's SwiGLU
// experts; the talk's grouped GEMM over all experts in one launch per
// projection), for layers stored in fp32:
//   GEMM1: h[r, f] = silu(x_perm[r] . W_gate[e][f]) * (x_perm[r] . W_up[e][f])
//   GEMM2: o[r, n] = h[r] . W_down[e][n]
// on the vector ALUs with fma. A block computes a 64 x 64 output tile with a
// 16-deep K step staged in LDS (K-major, so a thread's 4 rows and 4 columns
// are contiguous reads); each of the 256 threads owns a 4 x 4 sub-tile.
#include "ffn_sched.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kBM = 64, kBN = 64, kBKf = 16;

template <bool SWIGLU>
__global__ __launch_bounds__(256) void ffn_f32_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                      int K, const float* __restrict__ A,
                                                      const float* __restrict__ B0,
                                                      const float* __restrict__ B1,
                                                      float* __restrict__ C, int NT) {
  __shared__ float As[kBKf][kBM + 4];
  __shared__ float Bs[kBKf][kBN + 4];
  __shared__ float Us[SWIGLU ? kBKf : 1][kBN + 4];
  TileCoord tc;
  if (!find_tile(offsets, E, kBM, NT, blockIdx.x, tc)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int n0 = tc.n_tile * kBN;
  const int lrow = tid >> 2, lk = (tid & 3) * 4;
  const int ar = min(tc.m0 + lrow, tc.seg_rows - 1);
  const float* a_src = A + (size_t)(tc.seg_start + ar) * K;
  const int bn = min(n0 + lrow, N - 1);
  const size_t wofs = (size_t)tc.e * (size_t)N * K;
  const float* b_src = B0 + wofs + (size_t)bn * K;
  const float* u_src = SWIGLU ? B1 + wofs + (size_t)bn * K : nullptr;

  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kBKf) {
    const int kk = k0 + lk;
    f32x4 av = {0.f, 0.f, 0.f, 0.f}, bv = av, uv = av;
    if (kk < K) {   // K is a multiple of 4, so a 4-wide load is all in or all out
      av = *reinterpret_cast<const f32x4*>(a_src + kk);
      bv = *reinterpret_cast<const f32x4*>(b_src + kk);
      if (SWIGLU) uv = *reinterpret_cast<const f32x4*>(u_src + kk);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lrow] = av[i];
      Bs[lk + i][lrow] = bv[i];
      if (SWIGLU) Us[lk + i][lrow] = uv[i];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kBKf; ++q) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[q][ty * 4 + i];
        b[i] = Bs[q][tx * 4 + i];
        if (SWIGLU) u[i] = Us[q][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (SWIGLU) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tc.m0 + ty * 4 + i;
    if (r >= tc.seg_rows) continue;
    float* crow = C + (size_t)(tc.seg_start + r) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      const float g = acc[i][j];
      crow[col] = SWIGLU ? (g / (1.0f + expf(-g))) * accu[i][j] : g;
    }
  }
}

template <bool SWIGLU>
hipError_t launch_gemm_f32_t(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A,
                           const void* B0, const void* B1, void* C, hipStream_t s) {
  const int NT = (N + kBN - 1) / kBN;
  const int64_t blocks = ((R_max + kBM - 1) / kBM + E) * NT;
  hipLaunchKernelGGL((ffn_f32_kernel<SWIGLU>), dim3((unsigned)blocks), dim3(256), 0, s, E, offsets, N,
                     K, reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(B0),
                     reinterpret_cast<const float*>(B1), reinterpret_cast<float*>(C), NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_f32(int which, int64_t R_max, int d, int E, int F, const void* in,
                           const int32_t* offsets, const void* w0, const void* w1, void* out,
                           hipStream_t s) {
  if (which == 1) return launch_gemm_f32_t<true>(R_max, E, offsets, F, d, in, w0, w1, out, s);
  return launch_gemm_f32_t<false>(R_max, E, offsets, d, F, in, w0, nullptr, out, s);
}

hipError_t launch_ffn_f32(int64_t R_max, int d, int E, int F, const void* x_perm,
                          const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                          void* h, void* out, hipStream_t s) {
  hipError_t err = launch_gemm_f32(1, R_max, d, E, F, x_perm, offsets, wg, wu, h, s);
  if (err != hipSuccess) return err;
  return launch_gemm_f32(2, R_max, d, E, F, h, offsets, wd, nullptr, out, s);
}

}  // namespace moe
