// Grouped SwiGLU expert FFN in bf16 on the CDNA4 matrix cores.
//
// "[Paper Club] Upcycling Large Language Models into Mixture of Experts",
// Megatron-Core part: looping over experts with one GEMM each is slow; a
// grouped GEMM takes any number of experts and tokens in one operation.
// "How do Mixture of Expert Models Work?", section "The Math Behind MoEs":
// Mixtral's experts are SwiGLU. Here:
//   GEMM1 (fused SwiGLU): h[r, f] = bf16(silu(x_perm[r] . W_gate[e][f]) * (x_perm[r] . W_up[e][f]))
//   GEMM2:                o[r, n] = bf16(h[r] . W_down[e][n])
// both accumulating in fp32 with v_mfma_f32_32x32x16_bf16.
//
// Both GEMMs are "NT": activations [rows, K] and weights [N, K] are K-contiguous,
// so every MFMA operand fragment is 8 consecutive bf16 of one row (one 16-byte
// LDS read per lane). The weights feed the MFMA's first operand and the
// activations its second, so each lane's accumulator holds 4 consecutive output
// features of one row, stored as one 8-byte write.
//
// Block tile BM rows x BN output features, K step 64, 4 wavefronts in 2 x 2;
// a wavefront owns (BM/2) x (BN/2) outputs (and, in GEMM1, the gate and the up
// accumulator of each). The weight tile of GEMM1 holds BN gate rows followed by
// BN up rows, so the two products for one h element sit in the same lane and
// register, and the SwiGLU epilogue needs no data exchange.
//
// LDS: double-buffered A and B tiles, rows of 128 bytes split into eight
// 16-byte chunks; chunk c of row r lives at chunk position c ^ (r & 7), so the
// 8 lanes that read one chunk column of 8 consecutive rows hit 8 different
// 16-byte bank groups.
#include "ffn_sched.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;            // bf16 elements per K step (128 bytes per row)
constexpr int kRowBytes = kBK * 2;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float silu(float a) { return a / (1.0f + __expf(-a)); }

template <int BM, int BN, bool SWIGLU>
__global__ __launch_bounds__(256) void ffn_bf16_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                       int K, const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B0,
                                                       const uint16_t* __restrict__ B1,
                                                       uint16_t* __restrict__ C, int NT) {
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;    // weight rows staged per K step
  constexpr int WM = BM / 2, WN = BN / 2;        // wave tile (output rows x output features)
  constexpr int MB = WM / 32, NB = WN / 32;      // 32x32 MFMA blocks per wave
  constexpr int NACC = (SWIGLU ? 2 : 1) * MB * NB;
  constexpr int A_LD = BM * 8 / 256;             // 16-byte chunks per thread per K step
  constexpr int B_LD = BROWS * 8 / 256;
  constexpr int STAGE = (BM + BROWS) * kRowBytes;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  extern __shared__ __align__(16) char smem[];

  TileCoord tc;
  if (!find_tile(offsets, E, BM, NT, blockIdx.x, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = tc.n_tile * BN;
  const size_t ldk = (size_t)K;   // elements per row for both operands

  // global source rows for this thread's loads (clamped: rows past the
  // expert's segment or past N repeat a valid row; their results are not stored)
  const uint16_t* a_src[A_LD];
  int a_lds[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + 256 * i, row = q >> 3, c = q & 7;
    const int r = min(tc.m0 + row, tc.seg_rows - 1);
    a_src[i] = A + (size_t)(tc.seg_start + r) * ldk + c * 8;
    a_lds[i] = swz(row, c);
  }
  const uint16_t* b_src[B_LD];
  int b_lds[B_LD];
  const size_t wofs = (size_t)tc.e * (size_t)N * ldk;
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + 256 * i, row = q >> 3, c = q & 7;
    const uint16_t* base = B0;
    int n = row;
    if (SWIGLU && row >= BN) {
      base = B1;
      n = row - BN;
    }
    n = min(n0 + n, N - 1);
    b_src[i] = base + wofs + (size_t)n * ldk + c * 8;
    b_lds[i] = BM * kRowBytes + swz(row, c);
  }

  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = ld16(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = ld16(b_src[i] + k0);
  };
  auto lstore = [&](char* st) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) st16(st + a_lds[i], ra[i]);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) st16(st + b_lds[i], rb[i]);
  };

  const int KT = K / kBK;
  gload(0);
  lstore(smem);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    if (kt + 1 < KT) gload((kt + 1) * kBK);
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 xa[MB];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int row = wm * WM + mb * 32 + (lane & 31);
        xa[mb] = __builtin_bit_cast(bf16x8, ld16(cur + swz(row, chunk)));
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int row = wn * WN + nb * 32 + (lane & 31);
        const bf16x8 wg = __builtin_bit_cast(bf16x8, ld16(cur + BM * kRowBytes + swz(row, chunk)));
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          acc[mb * NB + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wg, xa[mb], acc[mb * NB + nb], 0, 0, 0);
        if (SWIGLU) {
          const bf16x8 wu =
              __builtin_bit_cast(bf16x8, ld16(cur + BM * kRowBytes + swz(BN + row, chunk)));
#pragma unroll
          for (int mb = 0; mb < MB; ++mb)
            acc[MB * NB + mb * NB + nb] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(wu, xa[mb], acc[MB * NB + mb * NB + nb], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < KT) lstore(smem + ((kt + 1) & 1) * STAGE);
    __syncthreads();
  }

  // epilogue: lane holds, for its row (lane & 31), features 8*g + 4*(lane>>5) + 0..3
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int rloc = tc.m0 + wm * WM + mb * 32 + (lane & 31);
    if (rloc >= tc.seg_rows) continue;
    uint16_t* crow = C + (size_t)(tc.seg_start + rloc) * (size_t)N;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * WN + nb * 32 + 8 * g + 4 * (lane >> 5);
        if (col >= N) continue;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float a = acc[mb * NB + nb][4 * g + i];
          v[i] = SWIGLU ? silu(a) * acc[MB * NB + mb * NB + nb][4 * g + i] : a;
        }
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(crow + col) = w;
      }
    }
  }
}

template <int BM, int BN, bool SWIGLU>
hipError_t launch_gemm(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A,
                       const void* B0, const void* B1, void* C, hipStream_t s) {
  const int NT = (N + BN - 1) / BN;
  const int64_t mt_max = (R_max + BM - 1) / BM + E;
  const int64_t blocks = mt_max * NT;
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;
  const size_t lds = 2 * (size_t)(BM + BROWS) * kRowBytes;
  hipLaunchKernelGGL((ffn_bf16_kernel<BM, BN, SWIGLU>), dim3((unsigned)blocks), dim3(256), lds, s, E,
                     offsets, N, K, reinterpret_cast<const uint16_t*>(A),
                     reinterpret_cast<const uint16_t*>(B0), reinterpret_cast<const uint16_t*>(B1),
                     reinterpret_cast<uint16_t*>(C), NT);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16(int which, int64_t R_max, int d, int E, int F, const void* in,
                            const int32_t* offsets, const void* w0, const void* w1, void* out,
                            hipStream_t s) {
  if (which == 1) return launch_gemm<128, 64, true>(R_max, E, offsets, F, d, in, w0, w1, out, s);
  return launch_gemm<128, 128, false>(R_max, E, offsets, d, F, in, w0, nullptr, out, s);
}

hipError_t launch_ffn_bf16(int64_t R_max, int d, int E, int F, const void* x_perm,
                           const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                           void* h, void* out, hipStream_t s) {
  hipError_t err = launch_gemm_bf16(1, R_max, d, E, F, x_perm, offsets, wg, wu, h, s);
  if (err != hipSuccess) return err;
  return launch_gemm_bf16(2, R_max, d, E, F, h, offsets, wd, nullptr, out, s);
}

}  // namespace moe
