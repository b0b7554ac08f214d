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
// The same kernel, with other operand layouts and epilogues, and a grouped-K
// kernel make the backward pass's products for fp32 layers.
#include "ffn_sched.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kBM = 64, kBN = 64, kBKf = 16;

// Epilogues: the forward's plain and SwiGLU tiles; the backward's recompute
// (h, and the a and b it came from) and SwiGLU backward (dh -> da, db).
enum { F32_PLAIN = 0, F32_SWIGLU = 1, F32_SWIGLU_AB = 2, F32_SWIGLU_BWD = 3 };

__device__ __forceinline__ float sigmoid_f32(float a) { return 1.0f / (1.0f + expf(-a)); }

// C[r, n] = sum_k A[r, k] B_e(k, n) over each expert's rows of A [R, K].
// BT false: B_e(k, n) = B0[e][n][k] (weights [E, N, K], the forward's layout).
// BT true:  B_e(k, n) = B0[e][k][n] for k < ksplit, else B1[e][k - ksplit][n]
//           (weights read as stored with their output dimension contiguous:
//           W_down [E, d, F] for dh, [W_gate; W_up] [E, F, d] each for dx_perm).
// SWIGLU / SWIGLU_AB: a second product with B1 (the up projection) and
// h = silu(a) b; SWIGLU_AB also stores a to aux0 and b to aux1 ([R, N]).
// SWIGLU_BWD: acc is dh; a = aux0, b = aux1 ([R, N]); da = dh b silu'(a) to
// C[r][n] and db = dh silu(a) to C[r][N + n] (C is [R, 2N]).
template <int EPI, bool BT>
__global__ __launch_bounds__(256) void ffn_f32_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                      int K, const float* __restrict__ A,
                                                      const float* __restrict__ B0,
                                                      const float* __restrict__ B1,
                                                      float* __restrict__ C, int NT, int ksplit,
                                                      float* __restrict__ aux0, float* __restrict__ aux1) {
  constexpr bool DUAL = EPI == F32_SWIGLU || EPI == F32_SWIGLU_AB;
  __shared__ float As[kBKf][kBM + 4];
  __shared__ float Bs[kBKf][kBN + 4];
  __shared__ float Us[DUAL ? kBKf : 1][kBN + 4];
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
  const float* u_src = DUAL ? B1 + wofs + (size_t)bn * K : nullptr;
  // BT: thread loads 4 consecutive n of k-row k0 + (tid >> 4)
  const int tk = tid >> 4, tn = (tid & 15) * 4;
  const size_t bt_lo = (size_t)tc.e * (size_t)ksplit * N, bt_hi = (size_t)tc.e * (size_t)(K - ksplit) * N;

  float acc[4][4] = {}, accu[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kBKf) {
    const int kk = k0 + lk;
    f32x4 av = {0.f, 0.f, 0.f, 0.f}, bv = av, uv = av;
    if (kk < K) {   // K is a multiple of 4, so a 4-wide load is all in or all out
      av = *reinterpret_cast<const f32x4*>(a_src + kk);
      if (!BT) bv = *reinterpret_cast<const f32x4*>(b_src + kk);
      if (DUAL) uv = *reinterpret_cast<const f32x4*>(u_src + kk);
    }
    if (BT) {
      const int k = k0 + tk;
      if (k < K && n0 + tn < N)   // N is a multiple of 4
        bv = k < ksplit ? *reinterpret_cast<const f32x4*>(B0 + bt_lo + (size_t)k * N + n0 + tn)
                        : *reinterpret_cast<const f32x4*>(B1 + bt_hi + (size_t)(k - ksplit) * N + n0 + tn);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lrow] = av[i];
      if (BT)
        Bs[tk][tn + i] = bv[i];
      else
        Bs[lk + i][lrow] = bv[i];
      if (DUAL) Us[lk + i][lrow] = uv[i];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kBKf; ++q) {
      float a[4], b[4], u[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[q][ty * 4 + i];
        b[i] = Bs[q][tx * 4 + i];
        if (DUAL) u[i] = Us[q][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
          if (DUAL) accu[i][j] = fmaf(a[i], u[j], accu[i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tc.m0 + ty * 4 + i;
    if (r >= tc.seg_rows) continue;
    const size_t row = (size_t)(tc.seg_start + r);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col >= N) continue;
      const float g = acc[i][j];
      if constexpr (EPI == F32_PLAIN) {
        C[row * N + col] = g;
      } else if constexpr (EPI == F32_SWIGLU || EPI == F32_SWIGLU_AB) {
        C[row * N + col] = (g / (1.0f + expf(-g))) * accu[i][j];
        if (EPI == F32_SWIGLU_AB) {
          aux0[row * N + col] = g;
          aux1[row * N + col] = accu[i][j];
        }
      } else {   // SwiGLU backward: g is dh
        const float av = aux0[row * N + col], bv = aux1[row * N + col];
        const float sg = sigmoid_f32(av);
        C[row * 2 * N + col] = g * bv * (sg * (1.0f + av * (1.0f - sg)));
        C[row * 2 * N + N + col] = g * (av * sg);
      }
    }
  }
}

template <int EPI, bool BT>
hipError_t launch_gemm_f32_t(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A,
                             const void* B0, const void* B1, void* C, hipStream_t s, int ksplit = 0,
                             void* aux0 = nullptr, void* aux1 = nullptr) {
  const int NT = (N + kBN - 1) / kBN;
  const int64_t blocks = ((R_max + kBM - 1) / kBM + E) * NT;
  hipLaunchKernelGGL((ffn_f32_kernel<EPI, BT>), dim3((unsigned)blocks), dim3(256), 0, s, E, offsets, N,
                     K, reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(B0),
                     reinterpret_cast<const float*>(B1), reinterpret_cast<float*>(C), NT, ksplit,
                     reinterpret_cast<float*>(aux0), reinterpret_cast<float*>(aux1));
  return hipGetLastError();
}

// Weight gradients over each expert's rows (a grouped-K product): block
// (tile of C, expert) accumulates A^T B over the expert's rows in steps of
// 16 rows staged in LDS (each thread loads 4 consecutive columns of a row);
// an expert without rows writes zeros.
__global__ __launch_bounds__(256) void wgrad_f32_kernel(const int32_t* __restrict__ offsets, int M, int M1, int N,
                                                        int lda, int ldb, const float* __restrict__ A,
                                                        const float* __restrict__ B, float* __restrict__ C0,
                                                        float* __restrict__ C1, int MT) {
  __shared__ float As[kBKf][kBM + 4];
  __shared__ float Bs[kBKf][kBN + 4];
  const int e = blockIdx.y;
  const int m0 = (blockIdx.x % MT) * kBM, n0 = (blockIdx.x / MT) * kBN;
  const int lo = offsets[e], hi = offsets[e + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int lr = tid >> 4, lc = (tid & 15) * 4;
  float acc[4][4] = {};
  for (int r0 = lo; r0 < hi; r0 += kBKf) {
    const int r = r0 + lr;
    f32x4 av = {0.f, 0.f, 0.f, 0.f}, bv = av;
    if (r < hi) {   // M and N are multiples of 4: a 4-wide load is all in or all out
      if (m0 + lc < M) av = *reinterpret_cast<const f32x4*>(A + (size_t)r * lda + m0 + lc);
      if (n0 + lc < N) bv = *reinterpret_cast<const f32x4*>(B + (size_t)r * ldb + n0 + lc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lr][lc + i] = av[i];
      Bs[lr][lc + i] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kBKf; ++q) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[q][ty * 4 + i];
        b[i] = Bs[q][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    float* crow = m < M1 ? C0 + ((size_t)e * M1 + m) * N : C1 + ((size_t)e * (M - M1) + (m - M1)) * N;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n < N) crow[n] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(int which, int64_t R_max, int d, int E, int F, const void* in,
                           const int32_t* offsets, const void* w0, const void* w1, void* out,
                           hipStream_t s) {
  if (which == 1) return launch_gemm_f32_t<F32_SWIGLU, false>(R_max, E, offsets, F, d, in, w0, w1, out, s);
  return launch_gemm_f32_t<F32_PLAIN, false>(R_max, E, offsets, d, F, in, w0, nullptr, out, s);
}

hipError_t launch_bwd_f32_recompute(int64_t R_max, int d, int E, int F, const void* x_perm, const int32_t* offsets,
                                    const void* wg, const void* wu, void* h, void* a, void* b, hipStream_t s) {
  return launch_gemm_f32_t<F32_SWIGLU_AB, false>(R_max, E, offsets, F, d, x_perm, wg, wu, h, s, 0, a, b);
}

hipError_t launch_bwd_f32_dh(int64_t R_max, int d, int E, int F, const void* d_o, const int32_t* offsets,
                             const void* w_down, const void* a, const void* b, void* dab, hipStream_t s) {
  // dh[r, f] = sum_n d_o[r, n] W_down[e][n][f]: K = d, N = F, B as stored [d][F]
  return launch_gemm_f32_t<F32_SWIGLU_BWD, true>(R_max, E, offsets, F, d, d_o, w_down, w_down, dab, s, d,
                                                 const_cast<void*>(a), const_cast<void*>(b));
}

hipError_t launch_bwd_f32_dx_perm(int64_t R_max, int d, int E, int F, const void* dab, const int32_t* offsets,
                                  const void* w_gate, const void* w_up, void* dx_perm, hipStream_t s) {
  // dx_perm[r, j] = sum_{k < 2F} dab[r, k] [W_gate[e]; W_up[e]][k][j]: K = 2F, N = d
  return launch_gemm_f32_t<F32_PLAIN, true>(R_max, E, offsets, d, 2 * F, dab, w_gate, w_up, dx_perm, s, F);
}

hipError_t launch_wgrad_f32(int E, const int32_t* offsets, int M, int M1, int N, int lda, int ldb, const void* A,
                            const void* B, void* C0, void* C1, hipStream_t s) {
  const int MT = (M + kBM - 1) / kBM, NT = (N + kBN - 1) / kBN;
  hipLaunchKernelGGL(wgrad_f32_kernel, dim3((unsigned)(MT * NT), (unsigned)E), dim3(256), 0, s, offsets, M, M1, N,
                     lda, ldb, reinterpret_cast<const float*>(A), reinterpret_cast<const float*>(B),
                     reinterpret_cast<float*>(C0), reinterpret_cast<float*>(C1), MT);
  return hipGetLastError();
}

hipError_t launch_ffn_f32(int64_t R_max, int d, int E, int F, const void* x_perm,
                          const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                          void* h, void* out, hipStream_t s) {
  hipError_t err = launch_gemm_f32(1, R_max, d, E, F, x_perm, offsets, wg, wu, h, s);
  if (err != hipSuccess) return err;
  return launch_gemm_f32(2, R_max, d, E, F, h, offsets, wd, nullptr, out, s);
}

}  // namespace moe
