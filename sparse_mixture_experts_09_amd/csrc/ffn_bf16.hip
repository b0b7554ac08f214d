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
// Kernels (one fragment layout):
//   ffn_bf16_w4_kernel      256-row tiles, 4 wavefronts (1 per SIMD) of 128 x 128,
//                           K step 64, register-staged loads into two LDS
//                           stages, fragments read a substep ahead (the forward
//                           main path, and the backward pass's dx_perm GEMM over
//                           K-major weights);
//   ffn_bf16_reg_kernel     the same tiles with 8 wavefronts (2 per SIMD) of
//                           128 x 64 (the backward pass's recomputation and dh
//                           GEMMs, whose epilogues move three or four tiles);
//   ffn_bf16_kernel         128-row tiles, 4 wavefronts (experts average fewer
//                           than 128 rows: big tiles would waste work on the
//                           ragged last tile of each expert);
//   ffn_bf16_skinny_kernel  at most 64 rows per expert (decode): streams the
//                           weights through per-wavefront LDS stages;
//   wgrad_kernel            weight gradients (grouped K over each expert's rows;
//                           both operands K-major, transposing LDS reads).
// In GEMM1 the weight tile holds BN gate rows followed by BN up rows, so the
// two products for one h element sit in the same lane and register and the
// SwiGLU epilogue needs no data exchange.
#include "ffn_sched.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kBK = 64;            // bf16 elements per K step (128 bytes per row)
constexpr int kRowBytes = kBK * 2;

// 16-byte chunk c of row r sits at position c ^ (r & 7) ^ ((r >> 3) & 1): the lanes of one ds_read_b128
// phase (rows r..r+15, one chunk column) then hit distinct 16-byte bank groups whether the LDS
// serves 8 lanes over 32 banks or 16 lanes over 64 banks per cycle, and so do the row-major writes.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

// sigmoid with the hardware reciprocal (1 ulp in fp32; every consumer rounds
// to bf16): a large negative a gives exp(-a) = inf and sigmoid 0, so silu
// is -0 there as with a true division
__device__ __forceinline__ float sigmoid(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }
__device__ __forceinline__ float silu(float a) { return a * sigmoid(a); }

template <int BM, int BN, bool SWIGLU, int NWM, int NWN>
__global__ __launch_bounds__(64 * NWM * NWN) void ffn_bf16_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                       int K, const uint16_t* __restrict__ A,
                                                       const uint16_t* __restrict__ B0,
                                                       const uint16_t* __restrict__ B1,
                                                       uint16_t* __restrict__ C, int NT) {
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;    // weight rows staged per K step
  constexpr int NT_ = 64 * NWM * NWN;            // threads per block
  constexpr int WM = BM / NWM, WN = BN / NWN;    // wave tile (output rows x output features)
  constexpr int MB = WM / 32, NB = WN / 32;      // 32x32 MFMA blocks per wave
  constexpr int NACC = (SWIGLU ? 2 : 1) * MB * NB;
  constexpr int A_LD = BM * 8 / NT_;             // 16-byte chunks per thread per K step
  constexpr int B_LD = BROWS * 8 / NT_;
  constexpr int STAGE = (BM + BROWS) * kRowBytes;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && (BM * 8) % NT_ == 0 && (BROWS * 8) % NT_ == 0, "tile");
  extern __shared__ __align__(16) char smem[];

  TileCoord tc;
  if (!find_tile(offsets, E, BM, NT, blockIdx.x, tc)) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int n0 = tc.n_tile * BN;
  const size_t ldk = (size_t)K;   // elements per row for both operands

  // global source rows for this thread's loads (clamped: rows past the
  // expert's segment or past N repeat a valid row; their results are not stored)
  const uint16_t* a_src[A_LD];
  int a_lds[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int q = tid + NT_ * i, row = q >> 3, c = q & 7;
    const int r = min(tc.m0 + row, tc.seg_rows - 1);
    a_src[i] = A + (size_t)(tc.seg_start + r) * ldk + c * 8;
    a_lds[i] = swz(row, c);
  }
  const uint16_t* b_src[B_LD];
  int b_lds[B_LD];
  const size_t wofs = (size_t)tc.e * (size_t)N * ldk;
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int q = tid + NT_ * i, row = q >> 3, c = q & 7;
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

  // Fragments for one 16-deep substep: MB activation blocks and NBF weight
  // blocks (gate blocks, then up blocks in GEMM1). Two register sets: the
  // reads for substep s+1 are issued before the MFMAs of substep s, so the LDS
  // latency hides behind MB*NBF matrix instructions.
  constexpr int NBF = (SWIGLU ? 2 : 1) * NB;
  bf16x8 fa[2][MB], fb[2][NBF];
  auto read_frags = [&](const char* buf, int s, bf16x8(&A_)[MB], bf16x8(&B_)[NBF]) {
    const int chunk = 2 * s + (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      A_[mb] = __builtin_bit_cast(bf16x8, ld16(buf + swz(wm * WM + mb * 32 + (lane & 31), chunk)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = wn * WN + nb * 32 + (lane & 31);
      B_[nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowBytes + swz(row, chunk)));
      if (SWIGLU) B_[NB + nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowBytes + swz(BN + row, chunk)));
    }
  };
  auto mma = [&](const bf16x8(&A_)[MB], const bf16x8(&B_)[NBF]) {
#pragma unroll
    for (int nb = 0; nb < NBF; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        // accumulator order: [gate|plain][mb][nb], then [up][mb][nb]
        const int a = (nb / NB) * MB * NB + mb * NB + (nb % NB);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B_[nb], A_[mb], acc[a], 0, 0, 0);
      }
  };
  static_assert(kBK / 16 == 4, "the substep schedule below assumes four 16-deep substeps");

  const int KT = K / kBK;
  gload(0);
  lstore(smem);
  __syncthreads();
  read_frags(smem, 0, fa[0], fb[0]);

  for (int kt = 0; kt < KT; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < KT;
    if (more) gload((kt + 1) * kBK);
    read_frags(cur, 1, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    read_frags(cur, 2, fa[0], fb[0]);
    mma(fa[1], fb[1]);
    read_frags(cur, 3, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    // the next buffer was last read before the previous barrier
    if (more) lstore(nxt);
    mma(fa[1], fb[1]);
    __syncthreads();
    if (more) read_frags(nxt, 0, fa[0], fb[0]);
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

// ---------------------------------------------------------------------------
// Tiles of the grouped GEMMs: K step 64, so a K-contiguous operand row is one
// 128-byte LDS row; 16-byte chunk c of row r sits at position c ^ f(r),
// f(r) = (r & 7) ^ ((r >> 3) & 1), which keeps both the row-wise 16-byte
// writes and the fragment reads (rows r..r+15 of one chunk column) free of
// bank conflicts, whether the LDS serves 8 lanes over 32 banks or 16 lanes
// over 64 banks per cycle.
// ---------------------------------------------------------------------------

constexpr int kRowB = kBK * 2;                  // 128 bytes per LDS row
constexpr int kMaxSplit = 8;                    // most K-slices per split tail tile
__device__ __forceinline__ int dswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int daddr(int r, int chunk) { return r * kRowB + ((chunk ^ dswz(r)) << 4); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N & 0x30) << 10) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0), other counters untouched
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Epilogues: EPI_PLAIN C = bf16(acc); EPI_SWIGLU C = bf16(silu(gate) * up);
// EPI_SWIGLU_AB the same plus C2 = bf16(gate), C3 = bf16(up) (the backward
// pass's recomputation); EPI_SWIGLU_BWD (plain tile, acc = dh): with a = X0,
// b = X1 at the same element, C = bf16(dh * b * silu'(a)), C2 = bf16(dh * silu(a)).
// ldc / ldx: row strides (elements) of the outputs / of X0 and X1.
constexpr int EPI_PLAIN = 0, EPI_SWIGLU = 1, EPI_SWIGLU_AB = 2, EPI_SWIGLU_BWD = 3;

// Epilogues of the 256-row tiles (wavefront (wm, wn) owns rows wm*WM.. and
// columns wn*WN.. of the tile; acc[mb*NB + nb] is the 32x32 block mb, nb, and
// in SwiGLU tiles acc[MB*NB + ...] holds the matching up products). A lane
// holds, for its row (lane & 31), columns 8*g + 4*(lane>>5) + 0..3.
template <int BN, int MB, int NB, int WM, int WN>
__device__ __forceinline__ void store_partials(const f32x16* acc, float* pt, int wm, int wn, int lane) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int row = wm * WM + mb * 32 + (lane & 31);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * WN + nb * 32 + 8 * g + 4 * (lane >> 5);
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = acc[mb * NB + nb][4 * g + i];
        *reinterpret_cast<f32x4*>(pt + (size_t)row * BN + col) = v;
      }
  }
}

// Output tiles through LDS (the stage buffers, free once the K loop is done):
// the wavefronts write their bf16 values into a [BM][W] tile (row r at r * 2W
// bytes, 16-byte chunk c at position c ^ (r mod W/8)), then every thread
// stores whole 16-byte pieces, W/8 lanes per output row, so each store
// instruction covers whole 128-byte lines. Stored straight from the MFMA
// layout, one 8-byte store spans 32 rows (32 partial lines); draining those
// cost ~9 us per 256 x 256 tile round. Callers pass a barrier after their
// last LDS read before lds_put_tile.

// byte offset of the 4 bf16 at (row, col), col a multiple of 4, in the tile
template <int W>
__device__ __forceinline__ int lds_tile_pos(int row, int col) {
  return row * (W * 2) + (((col >> 3) ^ (row & (W / 8 - 1))) << 4) + ((col >> 2) & 1) * 8;
}
// SERIAL: one row block at a time (a scheduling fence after each), for
// callers whose accumulators fill the register file: hoisting every
// conversion ahead of the LDS writes would spill.
template <int MB, int NB, int WM, int WN, int W, class Val, bool SERIAL = false>
__device__ __forceinline__ void lds_put_tile(char* lds, int wm, int wn, int lane, Val val) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (SERIAL) __builtin_amdgcn_sched_barrier(0);
    const int row = wm * WM + mb * 32 + (lane & 31);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * WN + nb * 32 + 8 * g + 4 * (lane >> 5);
        uint2 o;
        o.x = pack_bf16x2(val(mb, nb, g, 0), val(mb, nb, g, 1));
        o.y = pack_bf16x2(val(mb, nb, g, 2), val(mb, nb, g, 3));
        *reinterpret_cast<uint2*>(lds + lds_tile_pos<W>(row, col)) = o;
      }
  }
}
// The reverse of lds_store_rows: tile row r from src + r * ld (a buffer whose
// record count ends at the last valid row, so rows past it read zeros), its
// 16-byte piece c only if c < chunks (else zeros).
// Tile row j comes from source row row_of(j).
template <int BM, int W, class RowOf>
__device__ __forceinline__ void lds_load_rows(char* lds, int tid, int chunks, __amdgpu_buffer_rsrc_t src, int ld,
                                              RowOf row_of) {
  constexpr int CH = W / 8, RB = W * 2;
  constexpr int PER = BM * CH / 512;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int cidx = tid + i * 512, row = cidx / CH, ch = cidx % CH;
    const u32x4 v = bload16(src, ch < chunks ? (uint32_t)(row_of(row) * ld + ch * 8) * 2u : 0x80000000u);
    st16(lds + row * RB + ((ch ^ (row & (CH - 1))) << 4), v);
  }
}
// Then, after a barrier: tile row r goes to row_ptr(r) (nullptr: not stored),
// its 16-byte piece c only if c < chunks.
template <int BM, int W, class RowPtr, int NTHR = 512>
__device__ __forceinline__ void lds_store_rows(const char* lds, int tid, int chunks, RowPtr row_ptr) {
  constexpr int CH = W / 8, RB = W * 2;
  constexpr int PER = BM * CH / NTHR;          // pieces per thread (NTHR threads)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int cidx = tid + i * NTHR, row = cidx / CH, ch = cidx % CH;
    const u32x4 v = ld16(lds + row * RB + ((ch ^ (row & (CH - 1))) << 4));
    uint16_t* dst = row_ptr(row);
    if (dst != nullptr && ch < chunks) st16(dst + ch * 8, v);
  }
}

// Plain and SwiGLU epilogues of the grouped GEMM tiles, through LDS: rows at
// or past the segment's end and columns at or past N (a multiple of 8) are
// not stored.
template <int EPI, int BM, int MB, int NB, int WM, int WN, int W, int NTHR = 512>
__device__ __forceinline__ void store_tile_lds(const f32x16* acc, const TileCoord& tc, int wm, int wn, int n0, int N,
                                               int ldc, uint16_t* __restrict__ C, char* lds, int tid) {
  static_assert(EPI == EPI_PLAIN || EPI == EPI_SWIGLU, "plain or SwiGLU tile");
  auto val = [&](int mb, int nb, int g, int i) {
    const float a = acc[mb * NB + nb][4 * g + i];
    return EPI == EPI_SWIGLU ? silu(a) * acc[MB * NB + mb * NB + nb][4 * g + i] : a;
  };
  lds_put_tile<MB, NB, WM, WN, W, decltype(val), NTHR == 256>(lds, wm, wn, tid & 63, val);
  __syncthreads();
  const int rows = min(BM, tc.seg_rows - tc.m0);
  uint16_t* c0 = C + (size_t)(tc.seg_start + tc.m0) * ldc + n0;
  auto row_ptr = [&](int row) { return row < rows ? c0 + (size_t)row * ldc : static_cast<uint16_t*>(nullptr); };
  lds_store_rows<BM, W, decltype(row_ptr), NTHR>(lds, tid, (N - n0) / 8, row_ptr);
}

// Plain tiles of MT rows x BN through LDS as fp32, [128][BN] floats at a time
// (16-byte chunk c of row r at position c ^ (r mod BN/4)). With MT = 256 the
// wavefronts are 2 x 2 and own 128 rows each (wavefront row wm); pass h takes
// row blocks 2h and 2h+1 of every wavefront (tile rows wm*128 + 64h + 0..63),
// so all four wavefronts write in both passes, and LDS row j holds tile row
// (j / 64) * 128 + 64h + j % 64. With MT <= 128 the wavefronts are 1 x 4 and
// one pass holds the tile (LDS row j = tile row j). After a pass the threads
// store whole 16-byte pieces: fp32 rows of the partial tile pt of a split
// tail slice ([256][BN], row-major), or, with pt null, the bf16 tile (8
// floats per piece; rows at or past the segment's end and columns at or past
// N are not stored). Both cases share the writes of the accumulators, so no
// accumulator is live across a branch (with 256 of them a lane, a branch
// there made the register allocator spill).
template <int MT, int BN, int MB, int NB, int WN, int NTHR>
__device__ __forceinline__ void store_plain_lds(const f32x16* acc, int wm, int wn, int lane, int tid, char* lds,
                                                float* pt, const TileCoord& tc, int n0, int N, int ldc,
                                                uint16_t* __restrict__ C) {
  constexpr int CH = BN / 4, RB = BN * 4;
  constexpr int PASSES = MT == 256 ? 2 : 1, PR = MT == 256 ? 128 : MT;   // passes, rows per pass
  static_assert(128 * RB <= 2 * 65536, "128 fp32 rows of the tile fit in LDS");
  static_assert(MT == 256 ? MB == 4 : MB * 32 == MT, "2 x 2 wavefronts of 128 rows or 1 x 4 of the whole tile");
  const int rows = min(MT, tc.seg_rows - tc.m0);
  const int ncols = N - n0;
  uint16_t* c0 = C + (size_t)(tc.seg_start + tc.m0) * ldc + n0;
  auto at = [&](int row, int c) { return lds + row * RB + ((c ^ (row & (CH - 1))) << 4); };
#pragma unroll
  for (int h = 0; h < PASSES; ++h) {
    __syncthreads();
#pragma unroll
    for (int m = 0; m < (MT == 256 ? 2 : MB); ++m) {
      __builtin_amdgcn_sched_barrier(0);
      const int mb = MT == 256 ? 2 * h + m : m;
      const int row = (MT == 256 ? wm * 64 : 0) + m * 32 + (lane & 31);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = acc[mb * NB + nb][4 * g + i];
          *reinterpret_cast<f32x4*>(at(row, (wn * WN + nb * 32 + 8 * g + 4 * (lane >> 5)) >> 2)) = v;
        }
    }
    __syncthreads();
    auto trow = [&](int j) { return MT == 256 ? (j >> 6) * 128 + 64 * h + (j & 63) : j; };
    if (pt != nullptr) {
#pragma unroll 4
      for (int i = 0; i < PR * CH / NTHR; ++i) {
        const int cidx = tid + i * NTHR, row = cidx / CH, c = cidx % CH;
        st16(pt + (size_t)trow(row) * BN + 4 * c, ld16(at(row, c)));
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < PR * (CH / 2) / NTHR; ++i) {
        const int cidx = tid + i * NTHR, row = cidx / (CH / 2), c8 = cidx % (CH / 2);
        const f32x4 lo = __builtin_bit_cast(f32x4, ld16(at(row, 2 * c8)));
        const f32x4 hi = __builtin_bit_cast(f32x4, ld16(at(row, 2 * c8 + 1)));
        const u32x4 o = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                         pack_bf16x2(hi[2], hi[3])};
        const int tr = trow(row);
        if (tr < rows && 8 * c8 < ncols) st16(c0 + (size_t)tr * ldc + 8 * c8, o);
      }
    }
  }
}

// Sum the K-slice partials of each split tail tile in slice order and store
// the bf16 result (rows inside the expert's segment, columns below N).
// One block per (split tile, 16-row group); each wavefront sums four rows,
// a lane four columns: every load instruction reads one whole 1 KB partial
// row, and all S x 4 loads of a wavefront are in flight before the sums.
template <int S>
__device__ __forceinline__ void split_reduce_rows(const float* __restrict__ part, size_t slice_stride, int row0,
                                                  int rows_left, int col, bool col_ok, uint16_t* __restrict__ crow0,
                                                  size_t ldc) {
  constexpr int BN = 256, RW = 4;
  f32x4 v[RW][S];
#pragma unroll
  for (int i = 0; i < RW; ++i)
#pragma unroll
    for (int j = 0; j < S; ++j)
      v[i][j] = (col_ok && i < rows_left)
                    ? *reinterpret_cast<const f32x4*>(part + j * slice_stride + (size_t)(row0 + i) * BN + col)
                    : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    f32x4 sum = v[i][0];
#pragma unroll
    for (int j = 1; j < S; ++j) sum += v[i][j];
    if (col_ok && i < rows_left) {
      uint2 w;
      w.x = pack_bf16x2(sum[0], sum[1]);
      w.y = pack_bf16x2(sum[2], sum[3]);
      *reinterpret_cast<uint2*>(crow0 + (size_t)i * ldc + col) = w;
    }
  }
}

__global__ __launch_bounds__(256) void split_reduce_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                           int K, int NT, int P, int max_split,
                                                           const float* __restrict__ partials,
                                                           uint16_t* __restrict__ C) {
  constexpr int BM = 256, BN = 256;
  const WorkPlan p = make_plan(offsets, E, BM, NT, P, max_split, K / kBK);
  const int t = blockIdx.x / (BM / 16);
  if (t >= p.r) return;
  TileCoord tc;
  if (!locate_tile(offsets, E, BM, NT, p.full + t, tc)) return;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x % (BM / 16)) * 16 + (threadIdx.x >> 6) * 4;
  const int rows_left = tc.seg_rows - (tc.m0 + row0);
  if (rows_left <= 0) return;
  const int col = lane * 4;
  const bool col_ok = tc.n_tile * BN + col < N;
  const float* part = partials + (size_t)(t * p.s) * BM * BN;
  const size_t ss = (size_t)BM * BN;
  uint16_t* crow0 = C + (size_t)(tc.seg_start + tc.m0 + row0) * (size_t)N + (size_t)tc.n_tile * BN;
  switch (p.s) {
    case 2: split_reduce_rows<2>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 3: split_reduce_rows<3>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 4: split_reduce_rows<4>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 5: split_reduce_rows<5>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 6: split_reduce_rows<6>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 7: split_reduce_rows<7>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    default: split_reduce_rows<kMaxSplit>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
  }
}

// The same for the per-XCD plan: one block per (XCD tail tile, 16-row group);
// XCD x's tail tile t has its partials at slots x Px + t s .. + s - 1.
__global__ __launch_bounds__(256) void split_reduce_xcd_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                               int K, int NT, int P, int max_split,
                                                               const float* __restrict__ partials,
                                                               uint16_t* __restrict__ C) {
  constexpr int BM = 256, BN = 256;
  __shared__ int ws[24];
  const int Px = P / kXcds;
  const int tg = blockIdx.x / (BM / 16), xcd = tg / Px, t = tg % Px;
  int tiles;
  const ExpertScan es = expert_scan(offsets, E, NT, ws, tiles);
  const XcdRun q = xcd_run(tiles, Px, max_split, K / kBK, xcd);
  if (t >= q.r) return;
  const TileCoord tc = locate_tile_scan(es, E, NT, q.first + q.full + t, ws + 16);
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x % (BM / 16)) * 16 + (threadIdx.x >> 6) * 4;
  const int rows_left = tc.seg_rows - (tc.m0 + row0);
  if (rows_left <= 0) return;
  const int col = lane * 4;
  const bool col_ok = tc.n_tile * BN + col < N;
  const float* part = partials + (size_t)(xcd * Px + t * q.s) * BM * BN;
  const size_t ss = (size_t)BM * BN;
  uint16_t* crow0 = C + (size_t)(tc.seg_start + tc.m0 + row0) * (size_t)N + (size_t)tc.n_tile * BN;
  switch (q.s) {
    case 2: split_reduce_rows<2>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 3: split_reduce_rows<3>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 4: split_reduce_rows<4>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 5: split_reduce_rows<5>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 6: split_reduce_rows<6>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    case 7: split_reduce_rows<7>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
    default: split_reduce_rows<kMaxSplit>(part, ss, row0, rows_left, col, col_ok, crow0, N); break;
  }
}

// ---------------------------------------------------------------------------
// 8-wavefront tiles (the backward pass's recomputation and dh GEMMs, whose
// epilogues move three or four tiles; the plain and SwiGLU epilogues and the
// split tail serve the same tiles in the forward layout): 256 x BN tiles
// (256 weight rows: BN gate + BN up rows in GEMM1), wavefronts split 2 x 4,
// the LDS layout and bank swizzle above and the LDS-staged epilogues, with
// register-staged loads:
// each thread fetches four 16-byte pieces of each operand per K step with
// buffer loads (whole 128-byte rows across 8 lanes; the descriptors' record
// counts end at the expert's last row and at the weight's last row, so
// loads past them return zeros), and writes them to the other LDS stage
// with the bank swizzle applied on the LDS side. Two schedules of a K step,
// both pinned with sched_group_barrier, one barrier per step:
//   spread (plain tiles): the eight pieces one by one: in each of the four
//     16-deep substeps two pieces of tile kt+1 are written to the other LDS
//     stage and their registers at once reloaded with tile kt+2, so every
//     load has one K step to land and the LDS writes (served at about a third
//     of the LDS read rate) are spread over the step. A substep: the next
//     substep's fragment reads, 2 MFMAs, a write, a load, 2 MFMAs, a write,
//     a load, 4 MFMAs.
//   bunched (SwiGLU tiles): fragments of substeps 0 and 1; substep 0 MFMAs
//     with all writes of tile kt+1, substep 1 MFMAs with all loads of tile
//     kt+2, substeps 2 and 3 with their fragment reads (loads get 3/4 of a
//     step). Measured on one box, spread is ~1.5% faster on plain tiles and
//     ~2% slower on SwiGLU tiles.
// The last K step is peeled and the body has no branches (the load past the
// last tile reloads the last one).
// ---------------------------------------------------------------------------

template <int BN, bool SWIGLU, int EPI = (SWIGLU ? EPI_SWIGLU : EPI_PLAIN), bool BT = false>
__global__ __launch_bounds__(512) void ffn_bf16_reg_kernel(
    int E, const int32_t* __restrict__ offsets, int N, int K, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, int NT,
    int P, int max_split, float* __restrict__ partials, int ldc, uint16_t* __restrict__ C2,
    uint16_t* __restrict__ C3, const uint16_t* __restrict__ X0, const uint16_t* __restrict__ X1, int ldx,
    const int32_t* __restrict__ a_slot, int a_k, uint32_t a_records, int ldb, int ksplit) {
  static_assert(SWIGLU == (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_AB), "tile layout and epilogue");
  static_assert(!BT || !SWIGLU, "K-major weights: plain tiles only");
  constexpr int BM = 256, NWM = 2, NWN = 4, NT_ = 512;
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;
  static_assert(BROWS == 256, "both operands are 256-row tiles");
  constexpr int WM = BM / NWM, WN = BN / NWN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int NBF = (SWIGLU ? 2 : 1) * NB;
  constexpr int NACC = MB * NBF;
  constexpr int PT = 2048 / NT_;                 // 16-byte pieces per thread per operand per K step
  constexpr int RSTEP = NT_ / 8;                 // rows between a thread's pieces
  constexpr int STAGE = (BM + BROWS) * kRowB;
  // MFMAs and fragment reads per substep (a K-major weight fragment takes two transposing reads)
  constexpr int NM = MB * NBF, NR = MB + (BT ? 2 : 1) * NBF;
  extern __shared__ __align__(16) char smem[];

  const int KTall = K / kBK;
  WorkItem w;
  if (!find_item(offsets, E, BM, NT, P, max_split, KTall, blockIdx.x, w)) return;
  const TileCoord tc = w.tc;
  int kb = 0, KT = KTall;
  if (w.split >= 0) {
    const int ns = make_plan(offsets, E, BM, NT, P, max_split, KTall).s;
    kb = w.slice * KTall / ns;
    KT = (w.slice + 1) * KTall / ns - kb;
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int n0 = tc.n_tile * BN;

  const size_t rowb = (size_t)K * 2;
  const int a_rows = min(BM, tc.seg_rows - tc.m0);
  const int b_rows = min(BN, N - n0);
  const size_t wrow0 = (size_t)tc.e * N + n0;
  // K-major weights (BT): expert e's rows k < ksplit are B0[e] [ksplit][ldb],
  // rows k >= ksplit are B1[e] [K - ksplit][ldb]; the descriptors start at
  // column n0 (columns past N read the next row and are never stored)
  const auto rb0 = BT ? make_rsrc(B0 + (size_t)tc.e * ksplit * ldb + n0, (uint32_t)(((size_t)ksplit * ldb - n0) * 2))
                      : make_rsrc(B0 + wrow0 * K, (uint32_t)(b_rows * rowb));
  const auto rb1 = BT ? make_rsrc((K > ksplit ? B1 : B0) + (size_t)tc.e * (K - ksplit) * ldb + n0,
                                  (uint32_t)(((size_t)(K - ksplit) * ldb - n0) * 2))
                      : make_rsrc((SWIGLU ? B1 : B0) + wrow0 * K, (uint32_t)(b_rows * rowb));
  // BT staging: piece i of a thread is k-row (tid >> 5) + 16 i, 16-byte chunk tid & 31 of the
  // 256 columns; in LDS the [64][256] tile has 512-byte rows with chunk c of row r at
  // position c ^ ((r & 3) << 2), which keeps the transposing fragment reads conflict-free
  const int bk0 = tid >> 5, bch = tid & 31;
  const uint32_t bt_off = (uint32_t)(bk0 * ldb + bch * 8) * 2u;
  const int bt_wofs = BM * kRowB + bk0 * 512 + ((bch ^ ((bk0 & 3) << 2)) << 4);
  const int row0 = tid >> 3, ch = tid & 7;
  const uint32_t voff = (uint32_t)(row0 * rowb) + ch * 16 + (uint32_t)kb * kRowB;
  const uint32_t rstep = (uint32_t)(RSTEP * rowb);
  // Token rows: the expert's segment of A, or (a_slot given) rows gathered
  // from the unpermuted activations A [a_records / rowb rows]: permuted row r
  // is token a_slot[r] / a_k; a tile row past the segment gets an offset at
  // the record count, so it reads zeros.
  __amdgpu_buffer_rsrc_t ra;
  uint32_t aoff[PT];
  if (a_slot != nullptr) {
    ra = make_rsrc(A, a_records);
#pragma unroll
    for (int p = 0; p < PT; ++p) {
      const int r = row0 + p * RSTEP;
      aoff[p] = r < a_rows ? ((uint32_t)a_slot[tc.seg_start + tc.m0 + r] / (uint32_t)a_k) * (uint32_t)rowb + ch * 16 +
                                 (uint32_t)kb * kRowB
                           : a_records;
    }
  } else {
    ra = make_rsrc(A + (size_t)(tc.seg_start + tc.m0) * K, (uint32_t)(a_rows * rowb));
#pragma unroll
    for (int p = 0; p < PT; ++p) aoff[p] = voff + p * rstep;
  }
  const int wofs = row0 * kRowB + ((ch ^ dswz(row0)) << 4);   // RSTEP is a multiple of 16: same swizzle

  // A thread's pieces: p < PT are token rows row0 + p*RSTEP, p >= PT weight
  // rows row0 + (p-PT)*RSTEP (plain tiles read B0; SwiGLU tiles read BN gate
  // rows, then BN up rows).
  constexpr int NP = 2 * PT;
  u32x4 stg[NP];
  auto gl = [&](int p, int kt) {
    const uint32_t ko = (uint32_t)(kt < KT ? kt : KT - 1) * kRowB;
    if (p < PT) {
      stg[p] = bload16(ra, aoff[p] + ko);
    } else if constexpr (BT) {
      const int k = ((kt < KT ? kt : KT - 1) + kb) * kBK;   // first k-row of the step (whole in B0 or in B1)
      const int i = p - PT;
      stg[p] = k < ksplit ? bload16(rb0, bt_off + (uint32_t)((k + 16 * i) * ldb) * 2u)
                          : bload16(rb1, bt_off + (uint32_t)((k - ksplit + 16 * i) * ldb) * 2u);
    } else {
      const int i = p - PT;
      const bool up = SWIGLU && i * RSTEP >= BN;
      stg[p] = bload16(up ? rb1 : rb0, voff + (up ? i * rstep - BN * (uint32_t)rowb : i * rstep) + ko);
    }
  };
  auto sw = [&](int p, int stage) {
    char* b = smem + stage * STAGE;
    if (BT && p >= PT)   // k-row bk0 + 16 i: (r & 3) is the same for every i
      st16(b + bt_wofs + (p - PT) * 16 * 512, stg[p]);
    else
      st16(p < PT ? b + wofs + p * RSTEP * kRowB : b + wofs + BM * kRowB + (p - PT) * RSTEP * kRowB, stg[p]);
  };

  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  bf16x8 fa[2][MB], fb[2][NBF];
  // BT fragment reads: ds_read_b64_tr_b16 gives lane i of a 16-lane group
  // element i & 3 of the 4-element vectors read by lanes (i >> 2) + 4 j,
  // j = 0..3. Lane s of group q reads k-row k0 + (s >> 2), columns
  // n0 + 4 (s & 3) .. +3 (k0 = 16 sub + 8 (q >> 1), n0 = the block's first
  // column + 16 (q & 1)), so lane i receives rows k0..k0+3 of column n0 + i;
  // a second read at k0 + 4 completes the 8 k of the MFMA operand.
  const int tq = lane >> 4, ts = lane & 15;
  auto read_frags = [&](int stage, int sub, bf16x8(&A_)[MB], bf16x8(&B_)[NBF]) {
    const char* buf = smem + stage * STAGE;
    const int chunk = 2 * sub + (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      A_[mb] = __builtin_bit_cast(bf16x8, ld16(buf + daddr(wm * WM + mb * 32 + (lane & 31), chunk)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (BT) {
        const int k = 16 * sub + 8 * (tq >> 1) + (ts >> 2);
        const int n = wn * WN + nb * 32 + 16 * (tq & 1) + 4 * (ts & 3);
        const char* at = buf + BM * kRowB + k * 512 + (((n >> 3) ^ ((k & 3) << 2)) << 4) + (n & 4) * 2;
        const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)at));
        const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(at + 4 * 512)));
        const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
        B_[nb] = __builtin_bit_cast(bf16x8, v);
      } else {
        const int row = wn * WN + nb * 32 + (lane & 31);
        B_[nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowB + daddr(row, chunk)));
        if (SWIGLU) B_[NB + nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowB + daddr(BN + row, chunk)));
      }
    }
  };
  auto mma = [&](const bf16x8(&A_)[MB], const bf16x8(&B_)[NBF]) {
#pragma unroll
    for (int nb = 0; nb < NBF; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int a = (nb / NB) * MB * NB + mb * NB + (nb % NB);
        acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B_[nb], A_[mb], acc[a], 0, 0, 0);
      }
  };

#pragma unroll
  for (int p = 0; p < NP; ++p) gl(p, 0);
  wait_vmcnt<0>();
#pragma unroll
  for (int p = 0; p < NP; ++p) sw(p, 0);
#pragma unroll
  for (int p = 0; p < NP; ++p) gl(p, 1);
  wait_lgkm0();
  __syncthreads();
  static_assert(NP == 8 && NM == 8, "two pieces and eight MFMAs per substep");
  for (int kt = 0; kt < KT - 1; ++kt) {
    const int cur = kt & 1;
    if constexpr (SWIGLU) {
      // bunched: all writes of tile kt+1 in substep 0, all loads of tile kt+2 in substep 1
      read_frags(cur, 0, fa[0], fb[0]);
      read_frags(cur, 1, fa[1], fb[1]);
      mma(fa[0], fb[0]);
      wait_vmcnt<0>();             // tile kt+1 is in the staging registers
#pragma unroll
      for (int p = 0; p < NP; ++p) sw(p, cur ^ 1);
#pragma unroll
      for (int p = 0; p < NP; ++p) gl(p, kt + 2);
      read_frags(cur, 2, fa[0], fb[0]);
      mma(fa[1], fb[1]);
      read_frags(cur, 3, fa[1], fb[1]);
      mma(fa[0], fb[0]);
      mma(fa[1], fb[1]);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * NR, 0);   // fragments of substeps 0 and 1
#pragma unroll
      for (int i = 0; i < NP; ++i) {                             // substep 0 MFMAs with the LDS writes
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < NP; ++i) {                             // substep 1 MFMAs with the buffer loads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 2 * NR; ++i) {                         // substeps 2, 3 fragments among MFMAs
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 64, 0);
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      continue;
    }
    // spread: two write/reload pairs per substep
    read_frags(cur, 0, fa[0], fb[0]);
#pragma unroll
    for (int sub = 0; sub < 4; ++sub) {
      if (sub < 3) read_frags(cur, sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
      mma(fa[sub & 1], fb[sub & 1]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = 2 * sub + j;
        wait_vmcnt<NP - 1>();      // piece p of tile kt+1 has landed (loaded one step ago)
        sw(p, cur ^ 1);
        gl(p, kt + 2);             // its register now takes tile kt+2
      }
      if (sub < 3) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);   // next substep's fragments
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
  }
  {
    const int cur = (KT - 1) & 1;
    read_frags(cur, 0, fa[0], fb[0]);
    read_frags(cur, 1, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    read_frags(cur, 2, fa[0], fb[0]);
    mma(fa[1], fb[1]);
    read_frags(cur, 3, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    mma(fa[1], fb[1]);
  }
  wait_vmcnt<0>();   // the reload past the last tile

  if (!SWIGLU && w.split >= 0) {
    const int ns = make_plan(offsets, E, BM, NT, P, max_split, KTall).s;
    store_partials<BN, MB, NB, WM, WN>(acc, partials + (size_t)(w.split * ns + w.slice) * BM * BN, wm, wn, lane);
    return;
  }
  if constexpr (EPI == EPI_PLAIN || EPI == EPI_SWIGLU) {
    __syncthreads();   // every wavefront is done reading the stages
    store_tile_lds<EPI, BM, MB, NB, WM, WN, BN>(acc, tc, wm, wn, n0, N, ldc, C, smem, tid);
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // a and b come in and da, db go out as whole-row 16-byte pieces through
    // LDS, in two passes over half of every wavefront's row blocks (128 tile
    // rows: wm * 128 + 64 h + 0..63 for pass h). A pass loads those rows of a
    // and b into the two LDS halves (lds rows j = 64 wm + 0..63), turns b into
    // da and a into db in place, and stores both. Stored straight from the
    // MFMA layout each 8-byte access spanned 32 rows (32 partial lines).
    static_assert(2 * (BM / 2) * BN * 2 <= 2 * STAGE && MB % 2 == 0, "two [BM/2][BN] bf16 tiles in LDS");
    constexpr int HR = BM / 2, HALF = HR * BN * 2;
    const int rows = min(BM, tc.seg_rows - tc.m0);
    const int chunks = (N - n0) / 8;
    const size_t xr0 = (size_t)(tc.seg_start + tc.m0) * ldx + n0;
    const size_t cr0 = (size_t)(tc.seg_start + tc.m0) * ldc + n0;
    const uint32_t xbytes = (uint32_t)((size_t)rows * ldx * 2);
    const auto ra = make_rsrc(X0 + xr0, xbytes), rbv = make_rsrc(X1 + xr0, xbytes);
    char* la = smem;
    char* lb = smem + HALF;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      auto row_of = [&](int jr) { return (jr >> 6) * 128 + 64 * h + (jr & 63); };   // lds row -> tile row
      __syncthreads();
      lds_load_rows<HR, BN>(la, tid, chunks, ra, ldx, row_of);
      lds_load_rows<HR, BN>(lb, tid, chunks, rbv, ldx, row_of);
      __syncthreads();
#pragma unroll
      for (int m = 0; m < MB / 2; ++m)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int jr = wm * 64 + m * 32 + (lane & 31);
            const int pos = lds_tile_pos<BN>(jr, wn * WN + nb * 32 + 8 * g + 4 * (lane >> 5));
            uint2* pa = reinterpret_cast<uint2*>(la + pos);
            uint2* pb = reinterpret_cast<uint2*>(lb + pos);
            const uint2 a2 = *pa, b2 = *pb;
            const float av[4] = {bf16_lo(a2.x), bf16_hi(a2.x), bf16_lo(a2.y), bf16_hi(a2.y)};
            const float bv[4] = {bf16_lo(b2.x), bf16_hi(b2.x), bf16_lo(b2.y), bf16_hi(b2.y)};
            float da[4], db[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // silu(a) = a sg and silu'(a) = sg (1 + a (1 - sg)), sg = sigmoid(a)
              const float dh = acc[(MB / 2 * h + m) * NB + nb][4 * g + i], sg = sigmoid(av[i]);
              da[i] = dh * bv[i] * (sg * (1.0f + av[i] * (1.0f - sg)));
              db[i] = dh * (av[i] * sg);
            }
            uint2 wa, wb;
            wa.x = pack_bf16x2(da[0], da[1]);
            wa.y = pack_bf16x2(da[2], da[3]);
            wb.x = pack_bf16x2(db[0], db[1]);
            wb.y = pack_bf16x2(db[2], db[3]);
            *pb = wa;
            *pa = wb;
          }
      __syncthreads();
      lds_store_rows<HR, BN>(lb, tid, chunks, [&](int jr) {
        const int r = row_of(jr);
        return r < rows ? C + cr0 + (size_t)r * ldc : static_cast<uint16_t*>(nullptr);
      });
      lds_store_rows<HR, BN>(la, tid, chunks, [&](int jr) {
        const int r = row_of(jr);
        return r < rows ? C2 + cr0 + (size_t)r * ldc : static_cast<uint16_t*>(nullptr);
      });
    }
  } else if constexpr (EPI == EPI_SWIGLU_AB) {
    // h and a (gate) through the two halves of LDS, then b (up)
    static_assert(BN * BM * 2 * 2 <= 2 * STAGE, "two [BM][BN] bf16 tiles in LDS");
    constexpr int HALF = BM * BN * 2;
    const int rows = min(BM, tc.seg_rows - tc.m0);
    const size_t r0 = (size_t)(tc.seg_start + tc.m0) * ldc + n0;
    auto rows_of = [&](uint16_t* base) {
      return [=](int row) { return row < rows ? base + r0 + (size_t)row * ldc : static_cast<uint16_t*>(nullptr); };
    };
    __syncthreads();
    lds_put_tile<MB, NB, WM, WN, BN>(smem, wm, wn, lane, [&](int mb, int nb, int g, int i) {
      return silu(acc[mb * NB + nb][4 * g + i]) * acc[MB * NB + mb * NB + nb][4 * g + i];
    });
    lds_put_tile<MB, NB, WM, WN, BN>(smem + HALF, wm, wn, lane,
                                     [&](int mb, int nb, int g, int i) { return acc[mb * NB + nb][4 * g + i]; });
    __syncthreads();
    lds_store_rows<BM, BN>(smem, tid, (N - n0) / 8, rows_of(C));
    lds_store_rows<BM, BN>(smem + HALF, tid, (N - n0) / 8, rows_of(C2));
    __syncthreads();
    lds_put_tile<MB, NB, WM, WN, BN>(smem, wm, wn, lane, [&](int mb, int nb, int g, int i) {
      return acc[MB * NB + mb * NB + nb][4 * g + i];
    });
    __syncthreads();
    lds_store_rows<BM, BN>(smem, tid, (N - n0) / 8, rows_of(C3));
  }
}

// ---------------------------------------------------------------------------
// Forward tiles with 4 wavefronts (one per SIMD). A 256-row tile gives each
// wavefront 128 token rows x 128 weight rows (2 x 2; 256 fp32 accumulators
// a lane, held in the accumulation registers), so a K step reads a third
// less from LDS than with 8 wavefronts of 128 x 64. With one wavefront per
// SIMD nothing hides a fragment read that an MFMA waits for, so the reads
// run one 16-deep substep ahead of the MFMAs, across the K steps too: the
// pieces a thread stages per K step (token rows, then 8 weight rows) are
// written to the other LDS stage a quarter per substep, each reloaded at
// once with the step after (one K step to land); the last quarter is
// written early in substep 3, then the step's one barrier, and the first
// fragments of the next step are read while the rest of substep 3's MFMAs
// run. Stage reuse: a stage is rewritten only after the barrier that follows
// every wavefront's last read of it.
// An expert's last row tile is ragged. A tile of at most 128 (64) rows runs
// with the wavefronts side by side (1 x 4, each 128 (64) rows x a quarter of
// the weight rows) and stages only its token rows, so it costs half (a
// quarter) of the MFMAs of a full tile (MT: the rows a tile body handles).
// Tile plan, gather, split tail and LDS-staged epilogues as in
// ffn_bf16_reg_kernel. Measured against that kernel on a dense 1024 x 65536
// GEMM: +3% at K = 4096, +5% at K = 14336.
// ---------------------------------------------------------------------------
template <int BN, bool SWIGLU, int MT, bool BT>
__device__ __forceinline__ void w4_tile(const XcdItem& w, int KTall, int E, const int32_t* __restrict__ offsets,
                                        int N, int K, const uint16_t* __restrict__ A,
                                        const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1,
                                        uint16_t* __restrict__ C, int NT, int P, int max_split,
                                        float* __restrict__ partials, int ldc, const int32_t* __restrict__ a_slot,
                                        int a_k, uint32_t a_records, int ldb, int ksplit, char* smem) {
  constexpr int BM = 256, NT_ = 256;
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;
  static_assert(BROWS == 256, "the weight tile has 256 rows");
  static_assert(!BT || !SWIGLU, "K-major weights: plain tiles only");
  constexpr int NWM = MT == 256 ? 2 : 1, NWN = 4 / NWM;
  constexpr int WM = MT / NWM, WN = BN / NWN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int NBF = (SWIGLU ? 2 : 1) * NB;
  constexpr int NACC = MB * NBF, NM = NACC, NR = MB + (BT ? 2 : 1) * NBF;   // MFMAs, LDS reads a substep
  constexpr int RSTEP = NT_ / 8;                 // rows between a thread's pieces
  constexpr int PA = MT / RSTEP, PB = BROWS / RSTEP, NP = PA + PB;   // 16-byte pieces per thread per K step
  constexpr int STAGE = (BM + BROWS) * kRowB;
  static_assert(MB >= 1 && NB >= 1 && NM % 2 == 0, "whole 32 x 32 blocks");

  const TileCoord tc = w.tc;
  const int kb = w.slice * KTall / w.nslices;
  const int KT = (w.slice + 1) * KTall / w.nslices - kb;
  // the thread index through an opaque step: the per-thread address arithmetic
  // then stays inside the loop over a block's tiles instead of being hoisted
  // out of it (for three tile shapes), where it would hold registers throughout
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int n0 = tc.n_tile * BN;

  const size_t rowb = (size_t)K * 2;
  const int a_rows = min(MT, tc.seg_rows - tc.m0);
  const int b_rows = min(BN, N - n0);
  const size_t wrow0 = (size_t)tc.e * N + n0;
  // K-major weights (BT) as in ffn_bf16_reg_kernel: expert e's k-rows below
  // ksplit from B0[e] [ksplit][ldb], the rest from B1[e]; staged as a
  // [64 k][256 n] tile of 512-byte rows (chunk c of row r at c ^ ((r & 3) << 2)),
  // piece i of a thread k-row (tid >> 5) + 8 i, chunk tid & 31
  const auto rb0 = BT ? make_rsrc(B0 + (size_t)tc.e * ksplit * ldb + n0, (uint32_t)(((size_t)ksplit * ldb - n0) * 2))
                      : make_rsrc(B0 + wrow0 * K, (uint32_t)(b_rows * rowb));
  const auto rb1 = BT ? make_rsrc((K > ksplit ? B1 : B0) + (size_t)tc.e * (K - ksplit) * ldb + n0,
                                  (uint32_t)(((size_t)(K - ksplit) * ldb - n0) * 2))
                      : make_rsrc((SWIGLU ? B1 : B0) + wrow0 * K, (uint32_t)(b_rows * rowb));
  const int row0 = tid >> 3, ch = tid & 7;
  const uint32_t voff = (uint32_t)(row0 * rowb) + ch * 16 + (uint32_t)kb * kRowB;
  const uint32_t rstep = (uint32_t)(RSTEP * rowb);
  __amdgpu_buffer_rsrc_t ra;
  uint32_t aoff[PA];
  if (a_slot != nullptr) {   // gathered token rows, as in ffn_bf16_reg_kernel
    ra = make_rsrc(A, a_records);
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int r = row0 + p * RSTEP;
      aoff[p] = r < a_rows ? ((uint32_t)a_slot[tc.seg_start + tc.m0 + r] / (uint32_t)a_k) * (uint32_t)rowb + ch * 16 +
                                 (uint32_t)kb * kRowB
                           : a_records;
    }
  } else {
    ra = make_rsrc(A + (size_t)(tc.seg_start + tc.m0) * K, (uint32_t)(a_rows * rowb));
#pragma unroll
    for (int p = 0; p < PA; ++p) aoff[p] = voff + p * rstep;
  }
  const int wofs = row0 * kRowB + ((ch ^ dswz(row0)) << 4);   // RSTEP is a multiple of 16: same swizzle

  // piece p < PA: token row row0 + p*RSTEP; p >= PA: weight row row0 + (p-PA)*RSTEP
  // (SwiGLU tiles: BN gate rows, then BN up rows)
  const int bk0 = tid >> 5, bch = tid & 31;
  const uint32_t bt_off = (uint32_t)(bk0 * ldb + bch * 8) * 2u;
  const int bt_wofs = BM * kRowB + bk0 * 512 + ((bch ^ ((bk0 & 3) << 2)) << 4);   // rows bk0 + 8 i: same swizzle
  u32x4 stg[NP];
  auto gl = [&](int p, int kt) {
    const uint32_t ko = (uint32_t)(kt < KT ? kt : KT - 1) * kRowB;
    if (p < PA) {
      stg[p] = bload16(ra, aoff[p] + ko);
    } else if constexpr (BT) {
      const int k = ((kt < KT ? kt : KT - 1) + kb) * kBK;   // first k-row of the step (whole in B0 or in B1)
      const int i = p - PA;
      stg[p] = k < ksplit ? bload16(rb0, bt_off + (uint32_t)((k + 8 * i) * ldb) * 2u)
                          : bload16(rb1, bt_off + (uint32_t)((k - ksplit + 8 * i) * ldb) * 2u);
    } else {
      const int i = p - PA;
      const bool up = SWIGLU && i * RSTEP >= BN;
      stg[p] = bload16(up ? rb1 : rb0, voff + (up ? i * rstep - BN * (uint32_t)rowb : i * rstep) + ko);
    }
  };
  auto sw = [&](int p, int stage) {
    char* b = smem + stage * STAGE;
    if (BT && p >= PA)
      st16(b + bt_wofs + (p - PA) * 8 * 512, stg[p]);
    else
      st16(p < PA ? b + wofs + p * RSTEP * kRowB : b + wofs + BM * kRowB + (p - PA) * RSTEP * kRowB, stg[p]);
  };

  f32x16 acc[NACC];
#pragma unroll
  for (int i = 0; i < NACC; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  bf16x8 fa[2][MB], fb[2][NBF];
  auto read_frags = [&](int stage, int sub, bf16x8(&A_)[MB], bf16x8(&B_)[NBF]) {
    const char* buf = smem + stage * STAGE;
    const int chunk = 2 * sub + (lane >> 5);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      A_[mb] = __builtin_bit_cast(bf16x8, ld16(buf + daddr(wm * WM + mb * 32 + (lane & 31), chunk)));
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (BT) {   // transposing reads, as in ffn_bf16_reg_kernel
        const int tq = lane >> 4, ts = lane & 15;
        const int k = 16 * sub + 8 * (tq >> 1) + (ts >> 2);
        const int n = wn * WN + nb * 32 + 16 * (tq & 1) + 4 * (ts & 3);
        const char* at = buf + BM * kRowB + k * 512 + (((n >> 3) ^ ((k & 3) << 2)) << 4) + (n & 4) * 2;
        const uint2 lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)at));
        const uint2 hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(at + 4 * 512)));
        const u32x4 v = {lo.x, lo.y, hi.x, hi.y};
        B_[nb] = __builtin_bit_cast(bf16x8, v);
      } else {
        const int row = wn * WN + nb * 32 + (lane & 31);
        B_[nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowB + daddr(row, chunk)));
        if (SWIGLU) B_[NB + nb] = __builtin_bit_cast(bf16x8, ld16(buf + BM * kRowB + daddr(BN + row, chunk)));
      }
    }
  };
  // MFMAs [i0, i1) of a substep
  auto mma = [&](const bf16x8(&A_)[MB], const bf16x8(&B_)[NBF], int i0, int i1) {
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      if (i < i0 || i >= i1) continue;
      const int nb = i / MB, mb = i % MB;
      const int a = (nb / NB) * MB * NB + mb * NB + (nb % NB);
      acc[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B_[nb], A_[mb], acc[a], 0, 0, 0);
    }
  };
  // substep sub writes (and reloads) pieces [q0(sub), q0(sub+1))
  auto q0 = [](int sub) { return NP * sub / 4; };
  auto pieces = [&](int sub, int stage, int kt) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p < q0(sub) || p >= q0(sub + 1)) continue;
      wait_vmcnt<NP - 1>();   // piece p of tile kt-1 has landed (loaded one step ago)
      sw(p, stage);
      gl(p, kt);              // its register now takes tile kt
    }
  };

#pragma unroll
  for (int p = 0; p < NP; ++p) gl(p, 0);
  wait_vmcnt<0>();
#pragma unroll
  for (int p = 0; p < NP; ++p) sw(p, 0);
#pragma unroll
  for (int p = 0; p < NP; ++p) gl(p, 1);
  wait_lgkm0();
  __syncthreads();
  read_frags(0, 0, fa[0], fb[0]);
  for (int kt = 0; kt < KT - 1; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int sub = 0; sub < 3; ++sub) {
      read_frags(cur, sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
      mma(fa[sub & 1], fb[sub & 1], 0, NM);
      pieces(sub, cur ^ 1, kt + 2);
      // the next fragments among the first MFMAs, then the write / reload pairs, each with an
      // MFMA while any is left
      const int nq = q0(sub + 1) - q0(sub);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        if (j < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int j = 0; j < nq; ++j) {
        if (NR + j < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
#pragma unroll
      for (int j = NR + nq; j < NM; ++j) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    // substep 3: the last pieces among its first MFMAs, the barrier, then the next tile's
    // first fragments among the rest
    mma(fa[1], fb[1], 0, NM / 2);
    pieces(3, cur ^ 1, kt + 2);
#pragma unroll
    for (int j = 0; j < NP - q0(3); ++j) {
      if (2 * j < NM / 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (2 * j + 1 < NM / 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    read_frags(cur ^ 1, 0, fa[0], fb[0]);
    mma(fa[1], fb[1], NM / 2, NM);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if (j < NM / 2) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  }
  {
    const int cur = (KT - 1) & 1;
    read_frags(cur, 1, fa[1], fb[1]);
    mma(fa[0], fb[0], 0, NM);
    read_frags(cur, 2, fa[0], fb[0]);
    mma(fa[1], fb[1], 0, NM);
    read_frags(cur, 3, fa[1], fb[1]);
    mma(fa[0], fb[0], 0, NM);
    mma(fa[1], fb[1], 0, NM);
  }
  wait_vmcnt<0>();   // the reload past the last tile

  if constexpr (SWIGLU) {
    __syncthreads();   // every wavefront is done reading the stages
    store_tile_lds<EPI_SWIGLU, MT, MB, NB, WM, WN, BN, NT_>(acc, tc, wm, wn, n0, N, ldc, C, smem, tid);
  } else {
    float* pt = w.slot >= 0 ? partials + (size_t)w.slot * BM * BN : nullptr;
    store_plain_lds<MT, BN, MB, NB, WN, NT_>(acc, wm, wn, lane, tid, smem, pt, tc, n0, N, ldc, C);
  }
}

template <int BN, bool SWIGLU, bool BT>
__global__ __launch_bounds__(256) void ffn_bf16_w4_kernel(
    int E, const int32_t* __restrict__ offsets, int N, int K, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ B0, const uint16_t* __restrict__ B1, uint16_t* __restrict__ C, int NT, int P,
    int max_split, float* __restrict__ partials, int ldc, const int32_t* __restrict__ a_slot, int a_k,
    uint32_t a_records, int ldb, int ksplit) {
  extern __shared__ __align__(16) char smem[];
  int* ws = reinterpret_cast<int*>(smem);   // plan words; the stages are free between tiles
  const int KTall = K / kBK, xcd = blockIdx.x % kXcds, Px = P / kXcds;
  int tiles;
  const ExpertScan es = expert_scan(offsets, E, NT, ws, tiles);
  const XcdRun q = xcd_run(tiles, Px, max_split, KTall, xcd);
  const int stride = gridDim.x / kXcds;
  for (int l = blockIdx.x / kXcds;; l += stride) {
    XcdItem w;
    int tile;
    if (!xcd_item(q, xcd, Px, l, tile, w)) break;
    w.tc = locate_tile_scan(es, E, NT, tile, ws + 16);
    __syncthreads();   // every thread has its tile before the stages are written
    const int rows = w.tc.seg_rows - w.tc.m0;   // the tile's token rows (at most 256 are used)
    if (rows <= 64)
      w4_tile<BN, SWIGLU, 64, BT>(w, KTall, E, offsets, N, K, A, B0, B1, C, NT, P, max_split, partials, ldc, a_slot,
                              a_k, a_records, ldb, ksplit, smem);
    else if (rows <= 128)
      w4_tile<BN, SWIGLU, 128, BT>(w, KTall, E, offsets, N, K, A, B0, B1, C, NT, P, max_split, partials, ldc, a_slot,
                               a_k, a_records, ldb, ksplit, smem);
    else
      w4_tile<BN, SWIGLU, 256, BT>(w, KTall, E, offsets, N, K, A, B0, B1, C, NT, P, max_split, partials, ldc, a_slot,
                               a_k, a_records, ldb, ksplit, smem);
  }
}

// ---------------------------------------------------------------------------
// Few rows per expert (decode): the grouped GEMMs read every weight once and
// the token rows are few, so the time is the weight stream from HBM.
//
// A block computes one 32-row weight tile (GEMM1: 16 gate rows then the 16
// up rows of the same features; GEMM2: 32 rows of W_down) against all rows
// of one expert (MT tiles of 32; rows past the expert's last read as zeros).
// Its NW wavefronts split the 64-deep K steps round-robin and never wait for
// each other inside the K loop: each wavefront streams its steps through D
// stages of its own LDS with buffer -> LDS DMA (8 lanes fetch one whole
// 128-byte row piece, so every load instruction covers 8 full lines) and
// reads the MFMA fragments back with the bank swizzle of the tiled kernels.
// At the end the partial tiles are added in wavefront order through LDS.
// The DMA past the last K step uses offsets above every record count, so it
// fetches nothing and the wait counts stay the same on every step.
// ---------------------------------------------------------------------------
// AUX: the cache policy bits of the load (2: nontemporal, for data read once)
template <int AUX = 0>
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voff, 0, 0, AUX);
#endif
}

template <bool SWIGLU, int MT, int D, int NW>
__global__ __launch_bounds__(64 * NW) void ffn_bf16_skinny_kernel(int E, const int32_t* __restrict__ offsets, int N,
                                                                  int K, const uint16_t* __restrict__ A,
                                                                  const uint16_t* __restrict__ B0,
                                                                  const uint16_t* __restrict__ B1,
                                                                  uint16_t* __restrict__ C) {
  constexpr int TF = SWIGLU ? 16 : 32;          // output features per block
  constexpr int ROWS = 32 * (1 + MT);           // LDS rows per stage: weight tile, then token rows
  constexpr int L = ROWS / 8;                   // DMA instructions per stage
  constexpr int STAGE = ROWS * kRowB;
  extern __shared__ __align__(16) char lds[];   // NW * D * STAGE
  const int NTb = N / TF;
  const int e = blockIdx.x / NTb, f0 = (blockIdx.x % NTb) * TF;
  const int lo = offsets[e], cnt = offsets[e + 1] - lo;
  if (cnt <= 0) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, g = lane >> 5;
  const uint32_t rowb = (uint32_t)K * 2;
  char* my = lds + wave * D * STAGE;
  const auto rw0 = make_rsrc(B0 + (size_t)e * N * K, (uint32_t)N * rowb);
  const auto rw1 = make_rsrc((SWIGLU ? B1 : B0) + (size_t)e * N * K, (uint32_t)N * rowb);
  const auto rx = make_rsrc(A + (size_t)lo * K, (uint32_t)min(cnt, 32 * MT) * rowb);
  // DMA instruction i fills LDS rows 8i..8i+7 of a stage; lane l brings the
  // 16-byte piece that belongs at slot l % 8 of row 8i + l / 8.
  const int lr = lane >> 3, lc = lane & 7;
  uint32_t src[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const int row = 8 * i + lr;
    const uint32_t c = (uint32_t)(lc ^ dswz(row));
    const int srow = i < 4 ? (SWIGLU ? f0 + 8 * (i & 1) + lr : f0 + row) : row - 32;
    src[i] = (uint32_t)srow * rowb + c * 16;
  }
  const int KT = K / kBK;
  auto issue = [&](int stage, int kt) {
    char* st = my + stage * STAGE;
    const uint32_t ko = kt < KT ? (uint32_t)kt * kRowB : 0x80000000u;
    // the weights stream through once: nontemporal; the token rows are read by every block
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < 4)
        bdma16<2>((SWIGLU && i >= 2) ? rw1 : rw0, src[i] + ko, st + i * 1024);
      else
        bdma16(rx, src[i] + ko, st + i * 1024);
    }
  };
  f32x16 acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[m][q] = 0.f;
  const int S = wave < KT ? (KT - wave + NW - 1) / NW : 0;   // K steps of this wavefront
#pragma unroll
  for (int j = 0; j < D - 1; ++j) issue(j, wave + NW * j);
  int rs = 0, ws = D - 1;
  for (int j = 0; j < S; ++j) {
    issue(ws, wave + NW * (j + D - 1));   // into the stage read one step ago
    wait_vmcnt<(D - 1) * L>();            // stage rs has landed
    const char* st = my + rs * STAGE;
    bf16x8 wf[4], xf[4][MT];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 2 * s + g;
      wf[s] = __builtin_bit_cast(bf16x8, ld16(st + daddr(r, c)));
#pragma unroll
      for (int m = 0; m < MT; ++m) xf[s][m] = __builtin_bit_cast(bf16x8, ld16(st + daddr(32 * (1 + m) + r, c)));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[s], xf[s][m], acc[m], 0, 0, 0);
    wait_lgkm0();                         // reads of stage rs done before it is refilled
    rs = rs + 1 == D ? 0 : rs + 1;
    ws = ws + 1 == D ? 0 : ws + 1;
  }
  wait_vmcnt<0>();   // the empty DMAs past the end, before the stage memory is reused
  float* red = reinterpret_cast<float*>(my);
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) red[(m * 16 + q) * 64 + lane] = acc[m][q];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w2 = 1; w2 < NW; ++w2) {
    const float* rw = reinterpret_cast<const float*>(lds + w2 * D * STAGE);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[m][q] += rw[(m * 16 + q) * 64 + lane];
  }
  // lane: row m*32 + r; GEMM1 features f0 + 8 q4 + 4 g + i from gate acc[4 q4 + i]
  // and up acc[8 + 4 q4 + i] (tile rows 16.. are the up rows); GEMM2 features
  // f0 + 8 q4 + 4 g + i from acc[4 q4 + i]
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int row = m * 32 + r;
    if (row >= cnt) continue;
    uint16_t* crow = C + (size_t)(lo + row) * N;
#pragma unroll
    for (int q4 = 0; q4 < (SWIGLU ? 2 : 4); ++q4) {
      const int col = f0 + 8 * q4 + 4 * g;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        v[i] = SWIGLU ? silu(acc[m][4 * q4 + i]) * acc[m][8 + 4 * q4 + i] : acc[m][4 * q4 + i];
      uint2 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(crow + col) = o;
    }
  }
}

template <bool SWIGLU, int MT, int D, int NW>
hipError_t launch_skinny_cfg(int E, const int32_t* offsets, int N, int K, const void* A, const void* B0,
                             const void* B1, void* C, hipStream_t s) {
  constexpr int kLds = NW * D * 32 * (1 + MT) * kRowB;
  static_assert(kLds <= 160 * 1024, "LDS per block");
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_bf16_skinny_kernel<SWIGLU, MT, D, NW>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = (int64_t)E * (N / (SWIGLU ? 16 : 32));
  hipLaunchKernelGGL((ffn_bf16_skinny_kernel<SWIGLU, MT, D, NW>), dim3((unsigned)blocks), dim3(64 * NW), kLds, s, E,
                     offsets, N, K, reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(B0),
                     reinterpret_cast<const uint16_t*>(B1), reinterpret_cast<uint16_t*>(C));
  return hipGetLastError();
}

// seg_max rows per expert at most (<= 64); N a multiple of 32, N * K * 2 < 2^31.
template <bool SWIGLU>
hipError_t launch_skinny(int64_t seg_max, int E, const int32_t* offsets, int N, int K, const void* A,
                         const void* B0, const void* B1, void* C, hipStream_t s) {
  if (SWIGLU)
    return seg_max <= 32 ? launch_skinny_cfg<true, 1, 3, 2>(E, offsets, N, K, A, B0, B1, C, s)
                         : launch_skinny_cfg<true, 2, 3, 2>(E, offsets, N, K, A, B0, B1, C, s);
  return seg_max <= 32 ? launch_skinny_cfg<false, 1, 2, 8>(E, offsets, N, K, A, B0, B1, C, s)
                       : launch_skinny_cfg<false, 2, 2, 4>(E, offsets, N, K, A, B0, B1, C, s);
}

// ---------------------------------------------------------------------------
// Weight gradients: per expert e, C_e[m][n] = sum over the expert's rows r in
// [offsets[e], offsets[e+1]) of A[r][m] * B[r][n], with A [R, lda] and
// B [R, ldb] the activations as stored (the token dimension is the
// contraction, so both operands are K-major). Rows m < M1 go to C0[e][m][n],
// rows m >= M1 to C1[e][m - M1][n] (gate and up gradients from one launch).
// 256 x 256 tiles, 8 wavefronts, K step 64: both operands are staged as
// [64 r][256 cols] tiles (32 lanes per 512-byte row) with the register-staged
// spread schedule of the main path, and both MFMA fragments come from
// transposing LDS reads (see ffn_bf16_reg_kernel with BT). The descriptors'
// record counts end at the expert's last row, so the rows of the last step
// past it read zeros. Tiles run expert by expert with m-tiles fastest, each
// XCD a contiguous run of them; an expert with no rows gets a zero gradient.
// The K extent is an expert's rows (about a thousand), so a tile is only ~16
// K steps: the blocks stay resident (one per compute unit, stepping through
// their XCD's run with the grid's stride) and load the next tile's first K
// step before the current tile's epilogue, so that load's latency and the
// block launch no longer sit between the tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void wgrad_kernel(int E, const int32_t* __restrict__ offsets, int M, int M1, int N,
                                                    int lda, int ldb, const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ B, uint16_t* __restrict__ C0,
                                                    uint16_t* __restrict__ C1) {
  constexpr int BM = 256, BN = 256, NWM = 2, NWN = 4;
  constexpr int WM = BM / NWM, WN = BN / NWN;
  constexpr int MB = WM / 32, NB = WN / 32, NACC = MB * NB;
  constexpr int PT = 4, NP = 2 * PT;               // 16-byte pieces per thread per operand per K step (512 threads)
  constexpr int TILE = 64 * 512;                   // one operand's [64][256] bf16 tile
  constexpr int STAGE = 2 * TILE;
  constexpr int NM = MB * NB, NR = 2 * (MB + NB);  // MFMAs and transposing reads per substep
  static_assert(NP == 8 && NM == 8, "two pieces and eight MFMAs per substep");
  extern __shared__ __align__(16) char smem[];

  const int MT = (M + BM - 1) / BM, NTn = (N + BN - 1) / BN;
  const int tiles = E * MT * NTn;
  const int x = blockIdx.x % kXcds, stride = gridDim.x / kXcds;
  const int q = tiles / kXcds, rr = tiles % kXcds;
  const int first = x * q + min(x, rr), run = q + (x < rr ? 1 : 0);
  int l = blockIdx.x / kXcds;
  if (l >= run) return;
  // Consecutive tiles (the blocks of one XCD at a time) share one operand's
  // column slab and each read a different slab of the other, which is so
  // read again for every tile of the shared one: that re-read operand is the
  // narrower one (A when M <= N), whose rows of an expert stay cached. (Over
  // [da | db], 2F = 28672 columns, it would be 58 MB an expert, 8 experts at
  // once: more than the 256 MB Infinity Cache.)
  const bool m_fast = M <= N;
  int e, m0, n0, lo, cnt, KT;
  auto coords = [&](int tile) {
    e = tile / (MT * NTn);
    const int rem = tile % (MT * NTn);
    m0 = (m_fast ? rem % MT : rem / NTn) * BM;
    n0 = (m_fast ? rem / MT : rem % NTn) * BN;
    lo = offsets[e];
    cnt = offsets[e + 1] - lo;
    KT = (cnt + kBK - 1) / kBK;
  };
  // The per-thread offsets are worked out again for every tile from the
  // thread index passed through an opaque step: left to itself the compiler
  // would hoist them out of the loop over tiles, where they would hold
  // registers through the epilogue and spill.
  int tid, lane, wave, wm, wn, k0, c, tq, ts, wofs;
  uint32_t a_off, b_off;
  auto thread_setup = [&]() {
    tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    lane = tid & 63;
    wave = tid >> 6;
    wm = wave / NWN;
    wn = wave % NWN;
    k0 = tid >> 5;
    c = tid & 31;
    a_off = (uint32_t)(k0 * lda + c * 8) * 2u;
    b_off = (uint32_t)(k0 * ldb + c * 8) * 2u;
    wofs = k0 * 512 + ((c ^ ((k0 & 3) << 2)) << 4);   // rows k0 + 16 i share (row & 3)
    // lane i of 16-lane group tq gets rows k..k+3 of column (block base + 16 (tq & 1) + i)
    tq = lane >> 4;
    ts = lane & 15;
  };

  // columns past M (N) read the next row and are never stored; an expert
  // without rows has no records, so its loads read zeros
  __amdgpu_buffer_rsrc_t ra, rb;
  auto descriptors = [&]() {
    ra = make_rsrc(A + (size_t)lo * lda + m0, cnt > 0 ? (uint32_t)(((size_t)cnt * lda - m0) * 2) : 0u);
    rb = make_rsrc(B + (size_t)lo * ldb + n0, cnt > 0 ? (uint32_t)(((size_t)cnt * ldb - n0) * 2) : 0u);
  };
  u32x4 stg[NP];
  // a step past the last one fetches nothing
  auto gl = [&](int p, int kt) {
    const uint32_t k = (uint32_t)(kt * kBK + 16 * (p % PT));
    stg[p] = p < PT ? bload16(ra, kt < KT ? a_off + k * (uint32_t)lda * 2u : 0x80000000u)
                    : bload16(rb, kt < KT ? b_off + k * (uint32_t)ldb * 2u : 0x80000000u);
  };
  auto sw = [&](int p, int stage) {
    st16(smem + stage * STAGE + (p < PT ? 0 : TILE) + wofs + (p % PT) * 16 * 512, stg[p]);
  };
  auto frag = [&](const char* t, int sub, int col0) {
    const int k = 16 * sub + 8 * (tq >> 1) + (ts >> 2);
    const int n = col0 + 16 * (tq & 1) + 4 * (ts & 3);
    const char* at = t + k * 512 + (((n >> 3) ^ ((k & 3) << 2)) << 4) + (n & 4) * 2;
    const uint2 lo2 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)at));
    const uint2 hi2 = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(at + 4 * 512)));
    const u32x4 v = {lo2.x, lo2.y, hi2.x, hi2.y};
    return __builtin_bit_cast(bf16x8, v);
  };
  f32x16 acc[NACC];
  bf16x8 fa[2][MB], fb[2][NB];
  auto read_frags = [&](int stage, int sub, bf16x8(&A_)[MB], bf16x8(&B_)[NB]) {
    const char* buf = smem + stage * STAGE;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) A_[mb] = frag(buf, sub, wm * WM + mb * 32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) B_[nb] = frag(buf + TILE, sub, wn * WN + nb * 32);
  };
  auto mma = [&](const bf16x8(&A_)[MB], const bf16x8(&B_)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb * NB + nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(B_[nb], A_[mb], acc[mb * NB + nb], 0, 0, 0);
  };

  // stage 0 <- step 0 (in registers), registers <- step 1
  auto start_tile = [&]() {
#pragma unroll
    for (int p = 0; p < NP; ++p) sw(p, 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) gl(p, 1);
    wait_lgkm0();
    __syncthreads();
  };
  thread_setup();
  coords(first + l);
  descriptors();
#pragma unroll
  for (int p = 0; p < NP; ++p) gl(p, 0);
  start_tile();
  for (;;) {
    thread_setup();
#pragma unroll
    for (int i = 0; i < NACC; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    if (KT > 0) {
      for (int kt = 0; kt < KT - 1; ++kt) {
        const int cur = kt & 1;
        read_frags(cur, 0, fa[0], fb[0]);
#pragma unroll
        for (int sub = 0; sub < 4; ++sub) {
          if (sub < 3) read_frags(cur, sub + 1, fa[(sub + 1) & 1], fb[(sub + 1) & 1]);
          mma(fa[sub & 1], fb[sub & 1]);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int p = 2 * sub + jj;
            wait_vmcnt<NP - 1>();    // piece p of step kt+1 has landed (loaded one step ago)
            sw(p, cur ^ 1);
            gl(p, kt + 2);
          }
          if (sub < 3) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
      const int cur = (KT - 1) & 1;
      read_frags(cur, 0, fa[0], fb[0]);
      read_frags(cur, 1, fa[1], fb[1]);
      mma(fa[0], fb[0]);
      read_frags(cur, 2, fa[0], fb[0]);
      mma(fa[1], fb[1]);
      read_frags(cur, 3, fa[1], fb[1]);
      mma(fa[0], fb[0]);
      mma(fa[1], fb[1]);
    }
    wait_vmcnt<0>();   // the empty loads past the last step
    thread_setup();    // (nothing derived from the thread index stays live through the K loop)
    // the tile through LDS: row m < M1 of expert e goes to C0[e][m], m >= M1 to C1[e][m - M1]
    __syncthreads();
    lds_put_tile<MB, NB, WM, WN, BN>(smem, wm, wn, lane,
                                     [&](int mb, int nb, int g, int i) { return acc[mb * NB + nb][4 * g + i]; });
    // the next tile's first step is loaded while this tile is stored
    const int e_c = e, m0_c = m0, n0_c = n0;
    l += stride;
    const bool more = l < run;
    if (more) {
      coords(first + l);
      descriptors();
#pragma unroll
      for (int p = 0; p < NP; ++p) gl(p, 0);
    }
    __syncthreads();
    // Every thread issues the same stores whatever the tile's shape (a piece
    // of C0 and one of C1, each past its expert's record count where it does
    // not belong), so the waits for the loads above do not have to cover them.
    {
      const auto rc0 = make_rsrc(C0 + (size_t)e_c * M1 * N, (uint32_t)((size_t)M1 * N * 2));
      const auto rc1 = make_rsrc(M1 < M ? C1 + (size_t)e_c * (M - M1) * N : C0,
                                 M1 < M ? (uint32_t)((size_t)(M - M1) * N * 2) : 0u);
#pragma unroll
      for (int i = 0; i < BM * BN / 8 / 512; ++i) {
        const int cidx = tid + i * 512, row = cidx >> 5, ch = cidx & 31;
        const u32x4 v = ld16(smem + row * 512 + ((ch ^ (row & 31)) << 4));
        const int m = m0_c + row, col = n0_c + ch * 8;
        const bool in = col < N;
        bstore16(rc0, in && m < M1 ? (uint32_t)(m * N + col) * 2u : 0x80000000u, v);
        bstore16(rc1, in && m >= M1 && m < M ? (uint32_t)((m - M1) * N + col) * 2u : 0x80000000u, v);
      }
    }
    if (!more) break;
    wait_lgkm0();
    __syncthreads();   // every wavefront is done reading the tile out of LDS
    start_tile();
  }
}

template <int BN, bool SWIGLU, int EPI = (SWIGLU ? EPI_SWIGLU : EPI_PLAIN), bool BT = false>
hipError_t launch_reg(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A, const void* B0,
                      const void* B1, void* C, float* partials, int P, hipStream_t s, int ldc = 0,
                      void* C2 = nullptr, void* C3 = nullptr, const void* X0 = nullptr, const void* X1 = nullptr,
                      int ldx = 0, const int32_t* a_slot = nullptr, int a_k = 1, uint32_t a_records = 0,
                      int ldb = 0, int ksplit = 0) {
  constexpr int BM = 256;
  constexpr size_t kLds = 2 * (size_t)(BM + 256) * kRowB;
  auto kern = &ffn_bf16_reg_kernel<BN, SWIGLU, EPI, BT>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int NT = (N + BN - 1) / BN;
  const int64_t tiles_ub = ((R_max + BM - 1) / BM + E) * NT;
  const bool split = EPI == EPI_PLAIN && partials != nullptr && P > 0 && (ldc == 0 || ldc == N);
  const int max_split = split ? kMaxSplit : 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid_blocks(tiles_ub, P, split)), dim3(512), kLds, s, E, offsets, N, K,
                     reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(B0),
                     reinterpret_cast<const uint16_t*>(B1), reinterpret_cast<uint16_t*>(C), NT, P, max_split,
                     partials, ldc ? ldc : N, reinterpret_cast<uint16_t*>(C2), reinterpret_cast<uint16_t*>(C3),
                     reinterpret_cast<const uint16_t*>(X0), reinterpret_cast<const uint16_t*>(X1), ldx, a_slot, a_k,
                     a_records, ldb, ksplit);
  if (split)
    hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)(P * (BM / 16))), dim3(256), 0, s, E, offsets, N, K, NT,
                       P, max_split, partials, reinterpret_cast<uint16_t*>(C));
  return hipGetLastError();
}

template <int BN, bool SWIGLU, bool BT = false>
hipError_t launch_w4(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A, const void* B0,
                     const void* B1, void* C, float* partials, int P, hipStream_t s,
                     const int32_t* a_slot = nullptr, int a_k = 1, uint32_t a_records = 0, int ldb = 0,
                     int ksplit = 0) {
  constexpr int BM = 256;
  constexpr size_t kLds = 2 * (size_t)(BM + 256) * kRowB;
  auto kern = &ffn_bf16_w4_kernel<BN, SWIGLU, BT>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int NT = (N + BN - 1) / BN;
  const int64_t tiles_ub = ((R_max + BM - 1) / BM + E) * NT;
  const bool split = !SWIGLU && partials != nullptr && P >= kXcds;
  const int max_split = split ? kMaxSplit : 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)xcd_grid_blocks(tiles_ub, P, split)), dim3(256), kLds, s, E,
                     offsets, N, K, reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(B0),
                     reinterpret_cast<const uint16_t*>(B1), reinterpret_cast<uint16_t*>(C), NT, P, max_split,
                     partials, N, a_slot, a_k, a_records, ldb, ksplit);
  if (split)
    hipLaunchKernelGGL(split_reduce_xcd_kernel, dim3((unsigned)(P / kXcds * kXcds * (BM / 16))), dim3(256), 0, s, E,
                       offsets, N, K, NT, P, max_split, partials, reinterpret_cast<uint16_t*>(C));
  return hipGetLastError();
}

template <int BM, int BN, bool SWIGLU, int NWM = 2, int NWN = 2>
hipError_t launch_gemm(int64_t R_max, int E, const int32_t* offsets, int N, int K, const void* A,
                       const void* B0, const void* B1, void* C, hipStream_t s) {
  constexpr int BROWS = SWIGLU ? 2 * BN : BN;
  constexpr size_t kLds = 2 * (size_t)(BM + BROWS) * kRowBytes;
  auto kern = &ffn_bf16_kernel<BM, BN, SWIGLU, NWM, NWN>;
  // opt in to more than 64 KiB of dynamic LDS once per instantiation
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  const int NT = (N + BN - 1) / BN;
  const int64_t mt_max = (R_max + BM - 1) / BM + E;
  const int64_t blocks = mt_max * NT;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * NWM * NWN), kLds, s, E, offsets, N, K,
                     reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(B0),
                     reinterpret_cast<const uint16_t*>(B1), reinterpret_cast<uint16_t*>(C), NT);
  return hipGetLastError();
}

}  // namespace

int compute_units() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

bool ffn_bf16_big_tiles(int64_t R_max, int E) { return R_max >= 128 * (int64_t)E; }

size_t ffn_bf16_workspace_bytes(int64_t R_max, int E) {
  // partial tiles of the down projection's split tail: at most one per compute unit
  if (!ffn_bf16_big_tiles(R_max, E)) return 0;
  return (size_t)compute_units() * 256 * 256 * sizeof(float);
}

bool ffn_bf16_skinny(int64_t seg_max, int d, int F) {
  return seg_max <= 64 && (int64_t)d * F * 2 < ((int64_t)1 << 31);
}

bool ffn_bf16_can_gather(int64_t R_max, int64_t seg_max, int d, int E, int F, int64_t T) {
  return !ffn_bf16_skinny(seg_max, d, F) && ffn_bf16_big_tiles(R_max, E) &&
         (T + 1) * (int64_t)d * 2 < ((int64_t)1 << 31);
}

// Gathering saves the scatter of R rows (up to k T) but puts one more memory
// round trip (the row -> slot map) in front of every tile's first loads. On
// MI355X that was a loss at k = 2 (Mixtral-shaped layer +40 us, scatter 17 us)
// and a gain at k = 8 (fine-grained layer -50 us, scatter 53 us).
bool ffn_bf16_gathers(int64_t R_max, int64_t seg_max, int d, int E, int F, int64_t T, int k) {
  return k >= 4 && ffn_bf16_can_gather(R_max, seg_max, d, E, F, T);
}

hipError_t launch_gemm_bf16(int which, int64_t R_max, int64_t seg_max, int d, int E, int F, const void* in,
                            const int32_t* offsets, const void* w0, const void* w1, void* out,
                            void* ws, hipStream_t s, const int32_t* gather_slot, int gather_k, int64_t gather_T) {
  if (gather_slot != nullptr) {
    // GEMM1 reading token rows straight from the unpermuted activations
    if (which != 1 || !ffn_bf16_can_gather(R_max, seg_max, d, E, F, gather_T) || gather_k < 1)
      return hipErrorInvalidValue;
    return launch_w4<128, true>(R_max, E, offsets, F, d, in, w0, w1, out, nullptr, 0, s, gather_slot, gather_k,
                                (uint32_t)(gather_T * d * 2));
  }
  // At most 64 rows per expert: stream the weights, no row tiles.
  if (ffn_bf16_skinny(seg_max, d, F)) {
    if (which == 1) return launch_skinny<true>(seg_max, E, offsets, F, d, in, w0, w1, out, s);
    return launch_skinny<false>(seg_max, E, offsets, d, F, in, w0, nullptr, out, s);
  }
  // 256-row tiles once experts average at least 128 rows; below that the
  // 128-row tiles waste less work on the ragged last tile of each expert.
  if (ffn_bf16_big_tiles(R_max, E)) {
    if (which == 1) return launch_w4<128, true>(R_max, E, offsets, F, d, in, w0, w1, out, nullptr, 0, s);
    return launch_w4<256, false>(R_max, E, offsets, d, F, in, w0, nullptr, out, reinterpret_cast<float*>(ws),
                                 ws ? compute_units() : 0, s);
  }
  if (which == 1) return launch_gemm<128, 64, true>(R_max, E, offsets, F, d, in, w0, w1, out, s);
  return launch_gemm<128, 128, false>(R_max, E, offsets, d, F, in, w0, nullptr, out, s);
}

hipError_t launch_ffn_bf16(int64_t R_max, int64_t seg_max, int d, int E, int F, const void* x_perm,
                           const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                           void* h, void* out, void* ws, hipStream_t s, const int32_t* gather_slot, int gather_k,
                           int64_t gather_T) {
  hipError_t err = launch_gemm_bf16(1, R_max, seg_max, d, E, F, x_perm, offsets, wg, wu, h, nullptr, s, gather_slot,
                                    gather_k, gather_T);
  if (err != hipSuccess) return err;
  return launch_gemm_bf16(2, R_max, seg_max, d, E, F, h, offsets, wd, nullptr, out, ws, s);
}

// ---------------------------------------------------------------------------
// backward GEMMs (bf16)
// ---------------------------------------------------------------------------

hipError_t launch_bwd_recompute_gate_up(int64_t R_max, int d, int E, int F, const void* x_perm,
                                        const int32_t* offsets, const void* wg, const void* wu, void* h,
                                        void* a_st, void* b_st, hipStream_t s) {
  return launch_reg<128, true, EPI_SWIGLU_AB>(R_max, E, offsets, F, d, x_perm, wg, wu, h, nullptr, 0, s, F, a_st,
                                              b_st);
}

hipError_t launch_bwd_dh(int64_t R_max, int d, int E, int F, const void* d_o, const int32_t* offsets,
                         const void* w_down, const void* a_st, const void* b_st, void* dab, hipStream_t s) {
  // dab [R, 2F]: da in columns 0..F-1, db in F..2F-1; the epilogue's buffer
  // offsets within a 256-row tile of dab, and those within one expert's
  // W_down [d][F], must stay below 2^31
  if ((int64_t)256 * 2 * F * 2 >= ((int64_t)1 << 31) || (int64_t)d * F * 2 >= ((int64_t)1 << 31))
    return hipErrorInvalidValue;
  // dh = d_o . W_down[e] (contraction over d): W_down[e] [d][F] is the K-major weight
  return launch_reg<256, false, EPI_SWIGLU_BWD, true>(R_max, E, offsets, F, d, d_o, w_down, nullptr, dab, nullptr, 0,
                                                      s, 2 * F, reinterpret_cast<uint16_t*>(dab) + F, nullptr, a_st,
                                                      b_st, F, nullptr, 1, 0, F, d);
}

hipError_t launch_bwd_dx_perm(int64_t R_max, int d, int E, int F, const void* dab, const int32_t* offsets,
                              const void* w_gate, const void* w_up, void* dx_perm, void* ws, hipStream_t s) {
  if ((int64_t)d * F * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  // dx_perm = [da, db] . [W_gate[e]; W_up[e]] (contraction over 2F): K-major
  // weight rows 0..F-1 from W_gate[e] [F][d], F..2F-1 from W_up[e]
  return launch_w4<256, false, true>(R_max, E, offsets, d, 2 * F, dab, w_gate, w_up, dx_perm,
                                     reinterpret_cast<float*>(ws), ws ? compute_units() : 0, s, nullptr, 1, 0, d, F);
}

hipError_t launch_wgrad(int E, const int32_t* offsets, int M, int M1, int N, int lda, int ldb, int64_t R,
                        const void* A, const void* B, void* C0, void* C1, hipStream_t s) {
  // buffer offsets within one expert's rows, and within one expert's C0 or
  // C1 gradient, must stay below 2^31
  if (R * (int64_t)(lda > ldb ? lda : ldb) * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  if ((int64_t)(M1 > M - M1 ? M1 : M - M1) * N * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  constexpr size_t kLds = 2 * (size_t)(2 * 64 * 512);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&wgrad_kernel),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLds);
  if (attr != hipSuccess) return attr;
  // one resident block per compute unit of each XCD (at most one per tile)
  const int64_t tiles = (int64_t)E * ((M + 255) / 256) * ((N + 255) / 256);
  const int P = compute_units();
  if (P < kXcds) return hipErrorInvalidValue;
  const int64_t per_xcd = (tiles + kXcds - 1) / kXcds;
  const int64_t grid = (per_xcd < P / kXcds ? per_xcd : P / kXcds) * kXcds;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(512), kLds, s, E, offsets, M, M1, N, lda, ldb,
                     reinterpret_cast<const uint16_t*>(A), reinterpret_cast<const uint16_t*>(B),
                     reinterpret_cast<uint16_t*>(C0), reinterpret_cast<uint16_t*>(C1));
  return hipGetLastError();
}

}  // namespace moe
