// libmoe C interface: argument checks, capacity and workspace arithmetic,
// and the launch sequence of the layer. No device memory is allocated here and
// no call synchronises; see include/moe.h for the contract of each entry point.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int kMaxDim = 1 << 24;           // d and F
constexpr int64_t kMaxTokens = (int64_t)1 << 31;   // T (T * k < 2^31 for the layer entry points)

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_bytes(int dt) { return dt == MOE_BF16 ? 2 : 4; }

struct Range {
  const void* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

// The first nout ranges are outputs; each must be disjoint from every other
// listed range (inputs and the other outputs).
bool any_overlap(const Range* all, int nout, int nall) {
  for (int i = 0; i < nout; ++i)
    for (int j = 0; j < nall; ++j)
      if (j != i && overlap(all[i], all[j])) return true;
  return false;
}

int64_t capacity_of(int64_t T, int E, int k, float cf) {
  if (cf == 0.0f) return T;
  const double c = ceil((double)cf * (double)T * (double)k / (double)E);
  return c >= (double)T ? T : (int64_t)c;
}

int64_t rows_max_of(int64_t T, int E, int k, int64_t cap) {
  const int64_t a = T * k, b = (int64_t)E * cap;
  return a < b ? a : b;
}

// Rows of any one expert: a token takes an expert at most once, and no expert
// keeps more than its capacity (cap <= T).
int64_t seg_max_of(int64_t cap, int64_t R_max) { return cap < R_max ? cap : R_max; }

// Scalar checks shared by every entry point. F < 0 means "not used".
int check_scalars(int64_t T, int d, int E, int k, float cf, int F, int dt, bool ffn) {
  if (T < 0 || d < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (F != -1 && F < 1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(cf) || cf < 0.0f) return MOE_ERR_INVALID_ARG;
  if (dt != MOE_F32 && dt != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (T > ((((int64_t)1 << 31) - 1) / k)) return MOE_ERR_UNSUPPORTED;   // T * k < 2^31, without overflow
  if (d > kMaxDim || F > kMaxDim) return MOE_ERR_UNSUPPORTED;           // buffer sizes fit 64 bits
  const int vec = dt == MOE_BF16 ? 8 : 4;
  if (d % vec != 0) return MOE_ERR_UNSUPPORTED;
  if (F > 0 && F % vec != 0) return MOE_ERR_UNSUPPORTED;
  if (ffn && dt == MOE_BF16 && (d % 64 != 0 || F % 64 != 0)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

bool valid_gating(int g) {
  return g == MOE_GATING_TOPK_SOFTMAX || g == MOE_GATING_SOFTMAX_TOPK || g == MOE_GATING_SOFTMAX_TOPK_SCALED;
}
bool valid_fill(int f) { return f == MOE_FILL_TOKEN_ORDER || f == MOE_FILL_PRIORITY; }

// Permutation workspace: chunk histograms, then (priority fill only) the
// order and the sort's buffers, each 256-byte aligned.
size_t permute_ws_bytes(int64_t T, int E, bool priority) {
  size_t b = round_up((size_t)moe::permute_chunks(T) * E * 4);
  if (priority) b += round_up((size_t)T * 4) + round_up(moe::priority_sort_bytes(T));
  return b;
}

struct ForwardLayout {
  size_t topk_idx, topk_gate, slot_row, row_slot, counts, offsets, chunks, order, sort, x_perm, h, out_perm,
      ffn, total;
};

size_t ffn_ws_bytes(int64_t R_max, int E, int dt) {
  return dt == MOE_BF16 ? moe::ffn_bf16_workspace_bytes(R_max, E) : 0;
}

ForwardLayout forward_layout(int64_t T, int d, int E, int k, int64_t R_max, int F, int dt) {
  ForwardLayout L;
  const size_t s = elem_bytes(dt);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.topk_idx = take((size_t)T * k * 4);
  L.topk_gate = take((size_t)T * k * 4);
  L.slot_row = take((size_t)T * k * 4);
  L.row_slot = take((size_t)R_max * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.chunks = take((size_t)moe::permute_chunks(T) * E * 4);
  L.order = take((size_t)T * 4);
  L.sort = take(moe::priority_sort_bytes(T));
  L.x_perm = take((size_t)R_max * d * s);
  L.h = take((size_t)R_max * F * s);
  L.out_perm = take((size_t)R_max * d * s);
  L.ffn = take(ffn_ws_bytes(R_max, E, dt));
  L.total = o;
  return L;
}

// Scratch of moe_permute_noalloc: the permutation's per-chunk expert
// histograms live in this file-scope device array instead of a caller
// workspace. Every GPU the library runs on holds its own copy until the
// process ends. On the host the name is only a stand-in: kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kPermuteScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) char permute_scratch[kPermuteScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of permute_scratch on the current device, looked up once
// per device (with that device current) and kept.
int permute_scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(permute_scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// One wavefront: the shader-clock counter (s_memtime, counts core clock
// cycles) and the constant-rate wall clock (s_memrealtime) at the start, a
// wait of `ticks` wall-clock ticks (s_sleep between reads, so the wave takes
// almost no issue slots from kernels sharing its compute unit), and both
// counters again; out = {core cycles, wall ticks} over the wait. The wall
// clock only moves forward, so the wait always ends.
__global__ __launch_bounds__(64) void clock_probe_kernel(uint64_t* __restrict__ out, uint64_t ticks) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  uint64_t r1 = r0;
  while (r1 - r0 < ticks) {
    __builtin_amdgcn_s_sleep(8);
    r1 = __builtin_amdgcn_s_memrealtime();
  }
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[0] = c1 - c0;
    out[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

int moe_clock_probe(uint64_t* out, int64_t wall_ticks, hipStream_t stream) {
  if (out == nullptr || wall_ticks < 1 || wall_ticks > 100000000) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out)) return MOE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(clock_probe_kernel, dim3(1), dim3(64), 0, stream, out, (uint64_t)wall_ticks);
  return hip_status(hipGetLastError());
}

int moe_wall_clock_khz(int32_t* khz) {
  if (khz == nullptr) return MOE_ERR_INVALID_ARG;
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return MOE_ERR_HIP;
  *khz = v;
  return MOE_OK;
}

int64_t moe_capacity(int64_t T, int32_t E, int32_t k, float cf) {
  if (T < 0 || E < 1 || k < 1 || k > E || !isfinite(cf) || cf < 0.0f) return -1;
  return capacity_of(T, E, k, cf);
}

int moe_rows_max(int64_t T, int32_t E, int32_t k, float cf, int64_t* rows) {
  if (rows == nullptr) return MOE_ERR_INVALID_ARG;
  const int64_t cap = moe_capacity(T, E, k, cf);
  if (cap < 0) return MOE_ERR_INVALID_ARG;
  if (T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  *rows = rows_max_of(T, E, k, cap);
  return MOE_OK;
}

int moe_permute_workspace_bytes(int64_t T, int32_t E, size_t* bytes) {
  if (bytes == nullptr || T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  *bytes = permute_ws_bytes(T, E, false);
  return MOE_OK;
}

int moe_permute_priority_workspace_bytes(int64_t T, int32_t E, size_t* bytes) {
  if (bytes == nullptr || T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  *bytes = permute_ws_bytes(T, E, true);
  return MOE_OK;
}

int moe_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                        size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  const int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  const int64_t R_max = rows_max_of(T, E, k, capacity_of(T, E, k, cf));
  *bytes = forward_layout(T, d, E, k, R_max, F, dt).total;
  return MOE_OK;
}

int moe_ffn_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                            size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  const int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  *bytes = ffn_ws_bytes(rows_max_of(T, E, k, capacity_of(T, E, k, cf)), E, dt);
  return MOE_OK;
}

int moe_route_gating(int64_t T, int32_t d, int32_t E, int32_t k, int32_t dt, int32_t gating,
                     const void* x, const void* w_router, int32_t* topk_idx, float* topk_gate,
                     float* logits_opt, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, 0.0f, -1, dt, false);
  if (st != MOE_OK) return st;
  if (!valid_gating(gating)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_idx) || !aligned16(topk_gate) ||
      !aligned16(logits_opt))
    return MOE_ERR_UNSUPPORTED;
  const size_t s = elem_bytes(dt);
  const Range all[] = {{topk_idx, (size_t)T * k * 4}, {topk_gate, (size_t)T * k * 4},
                       {logits_opt, (size_t)T * E * 4}, {x, (size_t)T * d * s},
                       {w_router, (size_t)E * d * s}};
  if (any_overlap(all, 3, 5)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_router(dt == MOE_BF16, T, d, E, k, gating, x, w_router, topk_idx, topk_gate,
                                       logits_opt, stream));
}

int moe_route(int64_t T, int32_t d, int32_t E, int32_t k, int32_t dt, const void* x,
              const void* w_router, int32_t* topk_idx, float* topk_gate, float* logits_opt,
              hipStream_t stream) {
  return moe_route_gating(T, d, E, k, dt, MOE_GATING_TOPK_SOFTMAX, x, w_router, topk_idx, topk_gate,
                          logits_opt, stream);
}

// static_scratch: take the workspace from permute_scratch (ws / ws_bytes are
// ignored) instead of the caller's buffer.
static int permute_impl(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt, const void* x,
                        const int32_t* topk_idx, const float* score, int64_t score_stride,
                        int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_row,
                        int32_t* row_slot, void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream,
                        bool static_scratch = false) {
  int st = check_scalars(T, d, E, k, cf, -1, dt, false);
  if (st != MOE_OK) return st;
  const bool priority = score != nullptr;
  if (priority && score_stride < 1) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !expert_counts || !expert_offsets || !slot_row || !row_slot || !x_perm ||
      (!ws && !static_scratch))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(topk_idx) || !aligned16(expert_counts) || !aligned16(expert_offsets) ||
      !aligned16(slot_row) || !aligned16(row_slot) || !aligned16(x_perm) || !aligned16(ws) ||
      (reinterpret_cast<uintptr_t>(score) & 3u) != 0)
    return MOE_ERR_UNSUPPORTED;
  const size_t need = permute_ws_bytes(T, E, priority);
  if (static_scratch) {
    ws = nullptr;                       // looked up after every argument check
    ws_bytes = kPermuteScratchBytes;
  }
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int64_t cap = capacity_of(T, E, k, cf);
  const int64_t R_max = rows_max_of(T, E, k, cap);
  const size_t s = elem_bytes(dt);
  const Range all[] = {{expert_counts, (size_t)E * 4}, {expert_offsets, (size_t)(E + 1) * 4},
                       {slot_row, (size_t)T * k * 4},  {row_slot, (size_t)R_max * 4},
                       {x_perm, (size_t)R_max * d * s}, {ws, need},
                       {x, (size_t)T * d * s},          {topk_idx, (size_t)T * k * 4},
                       {score, priority ? (size_t)((T - 1) * score_stride + 1) * 4 : 0}};
  if (any_overlap(all, 6, 9)) return MOE_ERR_INVALID_ARG;
  if (static_scratch) {
    st = permute_scratch_address(&ws);
    if (st != MOE_OK) return st;
  }
  char* w = reinterpret_cast<char*>(ws);
  int32_t* chunks = reinterpret_cast<int32_t*>(w);
  int32_t* order = nullptr;
  hipError_t e = hipSuccess;
  if (priority) {
    const size_t at = round_up((size_t)moe::permute_chunks(T) * E * 4);
    order = reinterpret_cast<int32_t*>(w + at);
    e = moe::launch_priority_order(T, score, score_stride, order, w + at + round_up((size_t)T * 4), stream);
  }
  if (e == hipSuccess)
    e = moe::launch_permute(dt == MOE_BF16, T, d, E, k, cap, x, topk_idx, order, expert_counts,
                            expert_offsets, slot_row, row_slot, x_perm, chunks, stream);
  return hip_status(e);
}

int moe_permute(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt, const void* x,
                const int32_t* topk_idx, int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* slot_row, int32_t* row_slot, void* x_perm, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  return permute_impl(T, d, E, k, cf, dt, x, topk_idx, nullptr, 0, expert_counts, expert_offsets, slot_row,
                      row_slot, x_perm, ws, ws_bytes, stream);
}

int moe_permute_noalloc(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt, const void* x,
                        const int32_t* topk_idx, int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* slot_row, int32_t* row_slot, void* x_perm, hipStream_t stream) {
  return permute_impl(T, d, E, k, cf, dt, x, topk_idx, nullptr, 0, expert_counts, expert_offsets, slot_row,
                      row_slot, x_perm, nullptr, 0, stream, true);
}

size_t moe_permute_noalloc_scratch_bytes(void) { return kPermuteScratchBytes; }

int moe_permute_priority(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt, const void* x,
                         const int32_t* topk_idx, const float* score, int64_t score_stride,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot_row,
                         int32_t* row_slot, void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (score == nullptr) return MOE_ERR_INVALID_ARG;
  return permute_impl(T, d, E, k, cf, dt, x, topk_idx, score, score_stride, expert_counts, expert_offsets,
                      slot_row, row_slot, x_perm, ws, ws_bytes, stream);
}

int moe_grouped_ffn(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                    const void* x_perm, const int32_t* expert_offsets, const void* w_gate,
                    const void* w_up, const void* w_down, void* h_ws, void* out_perm, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !w_gate || !w_up || !w_down || !h_ws || !out_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(expert_offsets) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(h_ws) || !aligned16(out_perm) || !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  const int64_t R_max = rows_max_of(T, E, k, capacity_of(T, E, k, cf));
  const size_t s = elem_bytes(dt);
  const size_t wbytes = (size_t)E * F * d * s;
  const size_t need = ffn_ws_bytes(R_max, E, dt);
  if (ws != nullptr && ws_bytes < need) return MOE_ERR_WORKSPACE;
  const Range all[] = {{h_ws, (size_t)R_max * F * s}, {out_perm, (size_t)R_max * d * s},
                       {ws, need},
                       {x_perm, (size_t)R_max * d * s}, {expert_offsets, (size_t)(E + 1) * 4},
                       {w_gate, wbytes}, {w_up, wbytes}, {w_down, wbytes}};
  if (any_overlap(all, 3, 8)) return MOE_ERR_INVALID_ARG;
  hipError_t e = dt == MOE_BF16
                     ? moe::launch_ffn_bf16(R_max, seg_max_of(capacity_of(T, E, k, cf), R_max), d, E, F, x_perm,
                                            expert_offsets, w_gate, w_up, w_down, h_ws, out_perm,
                                            need ? ws : nullptr, stream)
                     : moe::launch_ffn_f32(R_max, d, E, F, x_perm, expert_offsets, w_gate, w_up,
                                           w_down, h_ws, out_perm, stream);
  return hip_status(e);
}

static int expert_gemm(int which, int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                       int32_t dt, const void* in, const int32_t* expert_offsets, const void* w0,
                       const void* w1, void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!in || !expert_offsets || !w0 || (which == 1 && !w1) || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(expert_offsets) || !aligned16(w0) || !aligned16(w1) || !aligned16(out) ||
      !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  const int64_t R_max = rows_max_of(T, E, k, capacity_of(T, E, k, cf));
  const size_t s = elem_bytes(dt);
  const size_t wbytes = (size_t)E * F * d * s;
  const size_t need = which == 2 ? ffn_ws_bytes(R_max, E, dt) : 0;
  if (which == 2 && ws != nullptr && ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t in_cols = which == 1 ? d : F, out_cols = which == 1 ? F : d;
  const Range all[] = {{out, (size_t)R_max * out_cols * s}, {ws, need}, {in, (size_t)R_max * in_cols * s},
                       {expert_offsets, (size_t)(E + 1) * 4}, {w0, wbytes}, {w1, which == 1 ? wbytes : 0}};
  if (any_overlap(all, 2, 6)) return MOE_ERR_INVALID_ARG;
  hipError_t e = dt == MOE_BF16
                     ? moe::launch_gemm_bf16(which, R_max, seg_max_of(capacity_of(T, E, k, cf), R_max), d, E, F, in,
                                             expert_offsets, w0, w1, out,
                                             need ? ws : nullptr, stream)
                     : moe::launch_gemm_f32(which, R_max, d, E, F, in, expert_offsets, w0, w1, out, stream);
  return hip_status(e);
}

int moe_expert_gate_up(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                       const void* x_perm, const int32_t* expert_offsets, const void* w_gate,
                       const void* w_up, void* h, hipStream_t stream) {
  return expert_gemm(1, T, d, E, k, cf, F, dt, x_perm, expert_offsets, w_gate, w_up, h, nullptr, 0, stream);
}

int moe_expert_down(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                    const void* h, const int32_t* expert_offsets, const void* w_down, void* out_perm,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  return expert_gemm(2, T, d, E, k, cf, F, dt, h, expert_offsets, w_down, nullptr, out_perm, ws, ws_bytes,
                     stream);
}

int moe_unpermute_combine(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                          const void* out_perm, const int32_t* slot_row, const float* topk_gate,
                          void* y, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, -1, dt, false);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!out_perm || !slot_row || !topk_gate || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out_perm) || !aligned16(slot_row) || !aligned16(topk_gate) || !aligned16(y))
    return MOE_ERR_UNSUPPORTED;
  const int64_t R_max = rows_max_of(T, E, k, capacity_of(T, E, k, cf));
  const size_t s = elem_bytes(dt);
  const Range all[] = {{y, (size_t)T * d * s}, {out_perm, (size_t)R_max * d * s},
                       {slot_row, (size_t)T * k * 4}, {topk_gate, (size_t)T * k * 4}};
  if (any_overlap(all, 1, 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(dt == MOE_BF16, T, d, k, out_perm, slot_row, topk_gate, y, stream));
}

int moe_forward_ex(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                   int32_t gating, int32_t fill_order, const void* x, const void* w_router,
                   const void* w_gate, const void* w_up, const void* w_down, void* y, int32_t* topk_idx_opt,
                   float* topk_gate_opt, int32_t* slot_row_opt, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  if (!valid_gating(gating) || !valid_fill(fill_order)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(y) || !aligned16(ws) || !aligned16(topk_idx_opt) ||
      !aligned16(topk_gate_opt) || !aligned16(slot_row_opt))
    return MOE_ERR_UNSUPPORTED;
  const int64_t cap = capacity_of(T, E, k, cf);
  const int64_t R_max = rows_max_of(T, E, k, cap);
  const ForwardLayout L = forward_layout(T, d, E, k, R_max, F, dt);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t s = elem_bytes(dt);
  const size_t wbytes = (size_t)E * F * d * s;
  const Range all[] = {{y, (size_t)T * d * s},        {topk_idx_opt, (size_t)T * k * 4},
                       {topk_gate_opt, (size_t)T * k * 4}, {slot_row_opt, (size_t)T * k * 4},
                       {ws, L.total},                 {x, (size_t)T * d * s},
                       {w_router, (size_t)E * d * s}, {w_gate, wbytes},
                       {w_up, wbytes},                {w_down, wbytes}};
  if (any_overlap(all, 5, 10)) return MOE_ERR_INVALID_ARG;

  char* w = reinterpret_cast<char*>(ws);
  int32_t* idx = topk_idx_opt ? topk_idx_opt : reinterpret_cast<int32_t*>(w + L.topk_idx);
  float* gate = topk_gate_opt ? topk_gate_opt : reinterpret_cast<float*>(w + L.topk_gate);
  int32_t* srow = slot_row_opt ? slot_row_opt : reinterpret_cast<int32_t*>(w + L.slot_row);
  int32_t* rslot = reinterpret_cast<int32_t*>(w + L.row_slot);
  int32_t* counts = reinterpret_cast<int32_t*>(w + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  int32_t* chunks = reinterpret_cast<int32_t*>(w + L.chunks);
  int32_t* order = fill_order == MOE_FILL_PRIORITY ? reinterpret_cast<int32_t*>(w + L.order) : nullptr;
  void* x_perm = w + L.x_perm;
  void* h = w + L.h;
  void* out_perm = w + L.out_perm;
  void* ffn_ws = w + L.ffn;
  const bool bf16 = dt == MOE_BF16;

  // bf16 with 256-row tiles and k >= 4: the gate/up GEMM reads the token
  // rows of x through the row -> slot map, and the permutation writes no x_perm
  const int64_t seg_max = seg_max_of(cap, R_max);
  const bool gather = bf16 && moe::ffn_bf16_gathers(R_max, seg_max, d, E, F, T, k);
  hipError_t e = moe::launch_router(bf16, T, d, E, k, gating, x, w_router, idx, gate, nullptr, stream);
  // Batch Priority Routing: the importance score is each token's top-1 gate
  if (e == hipSuccess && order) e = moe::launch_priority_order(T, gate, k, order, w + L.sort, stream);
  if (e == hipSuccess)
    e = moe::launch_permute(bf16, T, d, E, k, cap, x, idx, order, counts, offsets, srow, rslot,
                            gather ? nullptr : x_perm, chunks, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_ffn_bf16(R_max, seg_max, d, E, F, gather ? x : x_perm, offsets, w_gate, w_up, w_down, h,
                                    out_perm, ffn_ws_bytes(R_max, E, dt) ? ffn_ws : nullptr, stream,
                                    gather ? rslot : nullptr, k, T)
             : moe::launch_ffn_f32(R_max, d, E, F, x_perm, offsets, w_gate, w_up, w_down, h, out_perm,
                                   stream);
  if (e == hipSuccess) e = moe::launch_combine(bf16, T, d, k, out_perm, srow, gate, y, stream);
  return hip_status(e);
}

int moe_forward(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                const void* x, const void* w_router, const void* w_gate, const void* w_up,
                const void* w_down, void* y, int32_t* topk_idx_opt, float* topk_gate_opt,
                int32_t* slot_row_opt, void* ws, size_t ws_bytes, hipStream_t stream) {
  return moe_forward_ex(T, d, E, k, cf, F, dt, MOE_GATING_TOPK_SOFTMAX, MOE_FILL_TOKEN_ORDER, x, w_router,
                        w_gate, w_up, w_down, y, topk_idx_opt, topk_gate_opt, slot_row_opt, ws, ws_bytes,
                        stream);
}

// ---------------------------------------------------------------------------
// expert choice
// ---------------------------------------------------------------------------

// Rows of the expert-choice layer: C tokens per expert (C = capacity).
static int ec_rows(int64_t T, int E, int k, float cf, int64_t* C, int64_t* R) {
  *C = capacity_of(T, E, k, cf);
  *R = (int64_t)E * *C;
  return *R < ((int64_t)1 << 31) ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

int moe_route_expert_choice_workspace_bytes(int64_t T, int32_t E, size_t* bytes) {
  if (bytes == nullptr || T < 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || T >= kMaxTokens) return MOE_ERR_UNSUPPORTED;
  *bytes = round_up(moe::ec_select_bytes(T, E));
  return MOE_OK;
}

int moe_route_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt, const void* x,
                            const void* w_router, float* scores, int32_t* expert_tokens, int32_t* slot,
                            int32_t* expert_offsets, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, -1, dt, false);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !scores || !expert_tokens || !slot || !expert_offsets || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(scores) || !aligned16(expert_tokens) ||
      !aligned16(slot) || !aligned16(expert_offsets) || !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  const size_t need = round_up(moe::ec_select_bytes(T, E));
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const size_t s = elem_bytes(dt);
  const Range all[] = {{scores, (size_t)T * E * 4}, {expert_tokens, (size_t)R * 4}, {slot, (size_t)T * E * 4},
                       {expert_offsets, (size_t)(E + 1) * 4}, {ws, need},
                       {x, (size_t)T * d * s}, {w_router, (size_t)E * d * s}};
  if (any_overlap(all, 5, 7)) return MOE_ERR_INVALID_ARG;
  hipError_t e = moe::launch_router(dt == MOE_BF16, T, d, E, k, 3, x, w_router, nullptr, nullptr, scores, stream);
  if (e == hipSuccess) e = moe::launch_ec_select(T, E, (int)C, scores, ws, expert_tokens, slot, expert_offsets, stream);
  return hip_status(e);
}

int moe_gather_rows(int64_t T, int32_t d, int64_t R, int32_t dt, const void* x, const int32_t* row_token,
                    void* x_perm, hipStream_t stream) {
  if (T < 0 || d < 1 || R < 0 || (dt != MOE_F32 && dt != MOE_BF16)) return MOE_ERR_INVALID_ARG;
  if (d % (dt == MOE_BF16 ? 8 : 4) != 0) return MOE_ERR_UNSUPPORTED;
  if (R == 0) return MOE_OK;
  if (!x || !row_token || !x_perm) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(row_token) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
  const size_t s = elem_bytes(dt);
  const Range all[] = {{x_perm, (size_t)R * d * s}, {x, (size_t)T * d * s}, {row_token, (size_t)R * 4}};
  if (any_overlap(all, 1, 3)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_gather_rows(dt == MOE_BF16, T, R, d, x, row_token, x_perm, stream));
}

int moe_ffn_rows_workspace_bytes(int64_t R_max, int32_t d, int32_t E, int32_t F, int32_t dt, size_t* bytes) {
  if (bytes == nullptr || R_max < 0) return MOE_ERR_INVALID_ARG;
  const int st = check_scalars(0, d, E, 1, 0.0f, F, dt, true);
  if (st != MOE_OK) return st;
  if (R_max >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  *bytes = ffn_ws_bytes(R_max, E, dt);
  return MOE_OK;
}

int moe_grouped_ffn_rows(int64_t R_max, int32_t d, int32_t E, int32_t F, int32_t dt, const void* x_perm,
                         const int32_t* expert_offsets, const void* w_gate, const void* w_up, const void* w_down,
                         void* h_ws, void* out_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (R_max < 0) return MOE_ERR_INVALID_ARG;
  int st = check_scalars(0, d, E, 1, 0.0f, F, dt, true);
  if (st != MOE_OK) return st;
  if (R_max >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
  if (R_max == 0) return MOE_OK;
  if (!x_perm || !expert_offsets || !w_gate || !w_up || !w_down || !h_ws || !out_perm)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x_perm) || !aligned16(expert_offsets) || !aligned16(w_gate) || !aligned16(w_up) ||
      !aligned16(w_down) || !aligned16(h_ws) || !aligned16(out_perm) || !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  const size_t s = elem_bytes(dt);
  const size_t wbytes = (size_t)E * F * d * s;
  const size_t need = ffn_ws_bytes(R_max, E, dt);
  if (ws != nullptr && ws_bytes < need) return MOE_ERR_WORKSPACE;
  const Range all[] = {{h_ws, (size_t)R_max * F * s}, {out_perm, (size_t)R_max * d * s},
                       {ws, need},
                       {x_perm, (size_t)R_max * d * s}, {expert_offsets, (size_t)(E + 1) * 4},
                       {w_gate, wbytes}, {w_up, wbytes}, {w_down, wbytes}};
  if (any_overlap(all, 3, 8)) return MOE_ERR_INVALID_ARG;
  hipError_t e = dt == MOE_BF16
                     ? moe::launch_ffn_bf16(R_max, R_max, d, E, F, x_perm, expert_offsets, w_gate, w_up,
                                            w_down, h_ws, out_perm, need ? ws : nullptr, stream)
                     : moe::launch_ffn_f32(R_max, d, E, F, x_perm, expert_offsets, w_gate, w_up,
                                           w_down, h_ws, out_perm, stream);
  return hip_status(e);
}

int moe_combine_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                              const void* out_perm, const int32_t* slot, const float* scores, void* y,
                              hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, -1, dt, false);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!out_perm || !slot || !scores || !y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(out_perm) || !aligned16(slot) || !aligned16(scores) || !aligned16(y)) return MOE_ERR_UNSUPPORTED;
  const size_t s = elem_bytes(dt);
  const Range all[] = {{y, (size_t)T * d * s}, {out_perm, (size_t)R * d * s}, {slot, (size_t)T * E * 4},
                       {scores, (size_t)T * E * 4}};
  if (any_overlap(all, 1, 4)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_ec_combine(dt == MOE_BF16, T, d, E, R, out_perm, slot, scores, y, stream));
}

struct EcLayout {
  size_t scores, tokens, slot, offsets, select, x_perm, h, out_perm, ffn, total;
};

static EcLayout ec_layout(int64_t T, int d, int E, int64_t R, int F, int dt) {
  EcLayout L;
  const size_t s = elem_bytes(dt);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.scores = take((size_t)T * E * 4);
  L.tokens = take((size_t)R * 4);
  L.slot = take((size_t)T * E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.select = take(moe::ec_select_bytes(T, E));
  L.x_perm = take((size_t)R * d * s);
  L.h = take((size_t)R * F * s);
  L.out_perm = take((size_t)R * d * s);
  L.ffn = take(ffn_ws_bytes(R, E, dt));
  L.total = o;
  return L;
}

int moe_forward_expert_choice_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                                              int32_t dt, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  *bytes = ec_layout(T, d, E, R, F, dt).total;
  return MOE_OK;
}

int moe_forward_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                              const void* x, const void* w_router, const void* w_gate, const void* w_up,
                              const void* w_down, void* y, float* scores_opt, int32_t* slot_opt, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !w_gate || !w_up || !w_down || !y || !ws) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(y) || !aligned16(ws) || !aligned16(scores_opt) || !aligned16(slot_opt))
    return MOE_ERR_UNSUPPORTED;
  const EcLayout L = ec_layout(T, d, E, R, F, dt);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t s = elem_bytes(dt);
  const size_t wbytes = (size_t)E * F * d * s;
  const Range all[] = {{y, (size_t)T * d * s}, {scores_opt, (size_t)T * E * 4}, {slot_opt, (size_t)T * E * 4},
                       {ws, L.total},
                       {x, (size_t)T * d * s}, {w_router, (size_t)E * d * s}, {w_gate, wbytes},
                       {w_up, wbytes}, {w_down, wbytes}};
  if (any_overlap(all, 4, 9)) return MOE_ERR_INVALID_ARG;
  char* w = reinterpret_cast<char*>(ws);
  float* scores = scores_opt ? scores_opt : reinterpret_cast<float*>(w + L.scores);
  int32_t* slot = slot_opt ? slot_opt : reinterpret_cast<int32_t*>(w + L.slot);
  int32_t* tokens = reinterpret_cast<int32_t*>(w + L.tokens);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  const bool bf16 = dt == MOE_BF16;
  hipError_t e = moe::launch_router(bf16, T, d, E, k, 3, x, w_router, nullptr, nullptr, scores, stream);
  if (e == hipSuccess) e = moe::launch_ec_select(T, E, (int)C, scores, w + L.select, tokens, slot, offsets, stream);
  if (e == hipSuccess) e = moe::launch_gather_rows(bf16, T, R, d, x, tokens, w + L.x_perm, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_ffn_bf16(R, C, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w_down, w + L.h,
                                    w + L.out_perm, ffn_ws_bytes(R, E, dt) ? w + L.ffn : nullptr, stream)
             : moe::launch_ffn_f32(R, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w_down, w + L.h,
                                   w + L.out_perm, stream);
  if (e == hipSuccess) e = moe::launch_ec_combine(bf16, T, d, E, R, w + L.out_perm, slot, scores, y, stream);
  return hip_status(e);
}

// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------

struct BwdLayout {
  size_t idx, gate, slot_row, row_slot, counts, offsets, chunks, dl, logits, order, sort, x_perm, a_st, b_st, h, o,
      d_o, dab, dx_perm, router_part, ffn, total;
};

static BwdLayout bwd_layout(int64_t T, int d, int E, int k, int64_t R_max, int F, int dt) {
  const size_t s = elem_bytes(dt);
  BwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.idx = take((size_t)T * k * 4);
  L.gate = take((size_t)T * k * 4);
  L.slot_row = take((size_t)T * k * 4);
  L.row_slot = take((size_t)R_max * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.chunks = take((size_t)moe::permute_chunks(T) * E * 4);
  L.dl = take((size_t)T * (E > k ? E : k) * 4);   // [T, k], or [T, E] under the Switch rules
  L.logits = take((size_t)T * E * 4);             // the Switch rules' softmax input
  L.order = take((size_t)T * 4);                  // Batch Priority Routing: the fill order
  L.sort = take(moe::priority_sort_bytes(T));
  L.x_perm = take((size_t)R_max * d * s);
  L.a_st = take((size_t)R_max * F * s);
  L.b_st = take((size_t)R_max * F * s);
  L.h = take((size_t)R_max * F * s);
  L.o = take((size_t)R_max * d * s);
  L.d_o = take((size_t)R_max * d * s);
  L.dab = take((size_t)R_max * 2 * F * s);
  L.dx_perm = take((size_t)R_max * d * s);
  L.router_part = take(moe::router_wgrad_partial_bytes(T, d, E));
  L.ffn = take(ffn_ws_bytes(R_max, E, dt));
  L.total = o;
  return L;
}

int moe_backward_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                                 size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  *bytes = bwd_layout(T, d, E, k, rows_max_of(T, E, k, capacity_of(T, E, k, cf)), F, dt).total;
  return MOE_OK;
}

int moe_backward_ex(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt, int32_t gating,
                    int32_t fill_order, const void* x, const void* w_router, const void* w_gate, const void* w_up,
                    const void* w_down, const void* dy, void* dx, void* dw_router, void* dw_gate, void* dw_up,
                    void* dw_down, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  if (!valid_gating(gating) || !valid_fill(fill_order)) return MOE_ERR_INVALID_ARG;
  if (T == 0) return MOE_OK;
  const bool bf16 = dt == MOE_BF16;
  const size_t s = elem_bytes(dt);
  if (!x || !w_router || !w_gate || !w_up || !w_down || !dy || !dx || !dw_router || !dw_gate || !dw_up ||
      !dw_down || !ws)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dw_router) || !aligned16(dw_gate) || !aligned16(dw_up) ||
      !aligned16(dw_down) || !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  const int64_t cap = capacity_of(T, E, k, cf);
  const int64_t R_max = rows_max_of(T, E, k, cap);
  // the bf16 GEMMs address one expert's weights, and the kept rows of one activation, with 31-bit offsets
  const int64_t widest = 2 * (int64_t)F > d ? 2 * (int64_t)F : d;
  if (bf16 && (R_max * widest * 2 >= ((int64_t)1 << 31) || (int64_t)d * F * 2 >= ((int64_t)1 << 31)))
    return MOE_ERR_UNSUPPORTED;
  const BwdLayout L = bwd_layout(T, d, E, k, R_max, F, dt);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t wbytes = (size_t)E * F * d * s;
  const Range all[] = {{dx, (size_t)T * d * s},    {dw_router, (size_t)E * d * s}, {dw_gate, wbytes},
                       {dw_up, wbytes},            {dw_down, wbytes},              {ws, L.total},
                       {x, (size_t)T * d * s},     {w_router, (size_t)E * d * s},  {w_gate, wbytes},
                       {w_up, wbytes},             {w_down, wbytes},               {dy, (size_t)T * d * s}};
  if (any_overlap(all, 6, 12)) return MOE_ERR_INVALID_ARG;

  char* w = reinterpret_cast<char*>(ws);
  auto I32 = [&](size_t at) { return reinterpret_cast<int32_t*>(w + at); };
  int32_t* idx = I32(L.idx);
  float* gate = reinterpret_cast<float*>(w + L.gate);
  int32_t* srow = I32(L.slot_row);
  int32_t* offsets = I32(L.offsets);
  float* dl = reinterpret_cast<float*>(w + L.dl);
  void* ffn_ws = ffn_ws_bytes(R_max, E, dt) ? w + L.ffn : nullptr;
  const bool dense = gating != MOE_GATING_TOPK_SOFTMAX;   // the Switch rules: every logit gets gradient
  float* logits = dense ? reinterpret_cast<float*>(w + L.logits) : nullptr;
  const float scale = gating == MOE_GATING_SOFTMAX_TOPK_SCALED ? (float)E / (float)k : 1.f;
  int32_t* order = fill_order == MOE_FILL_PRIORITY ? I32(L.order) : nullptr;

  // recompute: routing (the same gate rule and fill order), permutation, a, b, h and o
  hipError_t e = moe::launch_router(bf16, T, d, E, k, gating, x, w_router, idx, gate, logits, stream);
  if (e == hipSuccess && order != nullptr)
    e = moe::launch_priority_order(T, gate, k, order, w + L.sort, stream);   // score: the top-1 gate
  if (e == hipSuccess)
    e = moe::launch_permute(bf16, T, d, E, k, cap, x, idx, order, I32(L.counts), offsets, srow, I32(L.row_slot),
                            w + L.x_perm, I32(L.chunks), stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_recompute_gate_up(R_max, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w + L.h,
                                                 w + L.a_st, w + L.b_st, stream)
             : moe::launch_bwd_f32_recompute(R_max, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w + L.h,
                                             w + L.a_st, w + L.b_st, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_gemm_bf16(2, R_max, seg_max_of(cap, R_max), d, E, F, w + L.h, offsets, w_down, nullptr,
                                     w + L.o, ffn_ws, stream)
             : moe::launch_gemm_f32(2, R_max, d, E, F, w + L.h, offsets, w_down, nullptr, w + L.o, stream);
  // combine and gate backward: d_o rows, dl
  if (e == hipSuccess)
    e = moe::launch_gate_bwd(T, d, k, dy, w + L.o, srow, gate, w + L.d_o, dl, stream, E, idx, logits, scale, bf16);
  // data gradients through the experts (the weights read as stored)
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_dh(R_max, d, E, F, w + L.d_o, offsets, w_down, w + L.a_st, w + L.b_st, w + L.dab,
                                  stream)
             : moe::launch_bwd_f32_dh(R_max, d, E, F, w + L.d_o, offsets, w_down, w + L.a_st, w + L.b_st, w + L.dab,
                                      stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_dx_perm(R_max, d, E, F, w + L.dab, offsets, w_gate, w_up, w + L.dx_perm, ffn_ws,
                                       stream)
             : moe::launch_bwd_f32_dx_perm(R_max, d, E, F, w + L.dab, offsets, w_gate, w_up, w + L.dx_perm, stream);
  // weight gradients over each expert's rows (the activations as stored)
  if (e == hipSuccess)
    e = bf16 ? moe::launch_wgrad(E, offsets, 2 * F, F, d, 2 * F, d, R_max, w + L.dab, w + L.x_perm, dw_gate, dw_up,
                                 stream)
             : moe::launch_wgrad_f32(E, offsets, 2 * F, F, d, 2 * F, d, w + L.dab, w + L.x_perm, dw_gate, dw_up,
                                     stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_wgrad(E, offsets, d, d, F, d, F, R_max, w + L.d_o, w + L.h, dw_down, nullptr, stream)
             : moe::launch_wgrad_f32(E, offsets, d, d, F, d, F, w + L.d_o, w + L.h, dw_down, nullptr, stream);
  // router weight and input gradients
  if (e == hipSuccess)
    e = moe::launch_router_wgrad(T, d, E, k, x, idx, dl, reinterpret_cast<float*>(w + L.router_part), dw_router,
                                 stream, dense, bf16);
  if (e == hipSuccess)
    e = moe::launch_dx_final(T, d, k, dl, idx, w_router, w + L.dx_perm, srow, dx, stream, dense ? E : 0, bf16);
  return hip_status(e);
}

int moe_backward(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt, const void* x,
                 const void* w_router, const void* w_gate, const void* w_up, const void* w_down, const void* dy,
                 void* dx, void* dw_router, void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  return moe_backward_ex(T, d, E, k, cf, F, dt, MOE_GATING_TOPK_SOFTMAX, MOE_FILL_TOKEN_ORDER, x, w_router, w_gate,
                         w_up, w_down, dy, dx, dw_router, dw_gate, dw_up, dw_down, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// backward pass of the expert-choice layer
// ---------------------------------------------------------------------------

struct EcBwdLayout {
  size_t scores, tokens, slot, offsets, select, dl, x_perm, a_st, b_st, h, o, d_o, dab, dx_perm, router_part, ffn,
      total;
};

static EcBwdLayout ec_bwd_layout(int64_t T, int d, int E, int64_t R, int F, int dt) {
  const size_t s = elem_bytes(dt);
  EcBwdLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += round_up(bytes);
    return at;
  };
  L.scores = take((size_t)T * E * 4);
  L.tokens = take((size_t)R * 4);
  L.slot = take((size_t)T * E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.select = take(moe::ec_select_bytes(T, E));
  L.dl = take((size_t)T * E * 4);
  L.x_perm = take((size_t)R * d * s);
  L.a_st = take((size_t)R * F * s);
  L.b_st = take((size_t)R * F * s);
  L.h = take((size_t)R * F * s);
  L.o = take((size_t)R * d * s);
  L.d_o = take((size_t)R * d * s);
  L.dab = take((size_t)R * 2 * F * s);
  L.dx_perm = take((size_t)R * d * s);
  L.router_part = take(moe::router_wgrad_partial_bytes(T, d, E));
  L.ffn = take(ffn_ws_bytes(R, E, dt));
  L.total = o;
  return L;
}

int moe_backward_expert_choice_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                                               int32_t dt, size_t* bytes) {
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  *bytes = ec_bwd_layout(T, d, E, R, F, dt).total;
  return MOE_OK;
}

int moe_backward_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                               const void* x, const void* w_router, const void* w_gate, const void* w_up,
                               const void* w_down, const void* dy, void* dx, void* dw_router, void* dw_gate,
                               void* dw_up, void* dw_down, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_scalars(T, d, E, k, cf, F, dt, true);
  if (st != MOE_OK) return st;
  int64_t C, R;
  if ((st = ec_rows(T, E, k, cf, &C, &R)) != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const bool bf16 = dt == MOE_BF16;
  const size_t s = elem_bytes(dt);
  if (!x || !w_router || !w_gate || !w_up || !w_down || !dy || !dx || !dw_router || !dw_gate || !dw_up ||
      !dw_down || !ws)
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(dy) || !aligned16(dx) || !aligned16(dw_router) || !aligned16(dw_gate) || !aligned16(dw_up) ||
      !aligned16(dw_down) || !aligned16(ws))
    return MOE_ERR_UNSUPPORTED;
  // the bf16 GEMMs address one expert's weights, and the rows of one activation, with 31-bit offsets
  const int64_t widest = 2 * (int64_t)F > d ? 2 * (int64_t)F : d;
  if (bf16 && (R * widest * 2 >= ((int64_t)1 << 31) || (int64_t)d * F * 2 >= ((int64_t)1 << 31)))
    return MOE_ERR_UNSUPPORTED;
  const EcBwdLayout L = ec_bwd_layout(T, d, E, R, F, dt);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const size_t wbytes = (size_t)E * F * d * s;
  const Range all[] = {{dx, (size_t)T * d * s},    {dw_router, (size_t)E * d * s}, {dw_gate, wbytes},
                       {dw_up, wbytes},            {dw_down, wbytes},              {ws, L.total},
                       {x, (size_t)T * d * s},     {w_router, (size_t)E * d * s},  {w_gate, wbytes},
                       {w_up, wbytes},             {w_down, wbytes},               {dy, (size_t)T * d * s}};
  if (any_overlap(all, 6, 12)) return MOE_ERR_INVALID_ARG;

  char* w = reinterpret_cast<char*>(ws);
  float* scores = reinterpret_cast<float*>(w + L.scores);
  int32_t* tokens = reinterpret_cast<int32_t*>(w + L.tokens);
  int32_t* slot = reinterpret_cast<int32_t*>(w + L.slot);
  int32_t* offsets = reinterpret_cast<int32_t*>(w + L.offsets);
  float* dl = reinterpret_cast<float*>(w + L.dl);
  void* ffn_ws = ffn_ws_bytes(R, E, dt) ? w + L.ffn : nullptr;

  // recompute: scores, selection, gathered rows, a, b, h and o
  hipError_t e = moe::launch_router(bf16, T, d, E, k, 3, x, w_router, nullptr, nullptr, scores, stream);
  if (e == hipSuccess) e = moe::launch_ec_select(T, E, (int)C, scores, w + L.select, tokens, slot, offsets, stream);
  if (e == hipSuccess) e = moe::launch_gather_rows(bf16, T, R, d, x, tokens, w + L.x_perm, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_recompute_gate_up(R, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w + L.h,
                                                 w + L.a_st, w + L.b_st, stream)
             : moe::launch_bwd_f32_recompute(R, d, E, F, w + L.x_perm, offsets, w_gate, w_up, w + L.h, w + L.a_st,
                                             w + L.b_st, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_gemm_bf16(2, R, C, d, E, F, w + L.h, offsets, w_down, nullptr, w + L.o, ffn_ws, stream)
             : moe::launch_gemm_f32(2, R, d, E, F, w + L.h, offsets, w_down, nullptr, w + L.o, stream);
  // combine and gate backward: d_o rows, dl over all E logits
  if (e == hipSuccess)
    e = moe::launch_ec_gate_bwd(bf16, T, d, E, R, dy, w + L.o, slot, scores, w + L.d_o, dl, stream);
  // data gradients through the experts, then the weight gradients over each expert's rows
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_dh(R, d, E, F, w + L.d_o, offsets, w_down, w + L.a_st, w + L.b_st, w + L.dab, stream)
             : moe::launch_bwd_f32_dh(R, d, E, F, w + L.d_o, offsets, w_down, w + L.a_st, w + L.b_st, w + L.dab,
                                      stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_bwd_dx_perm(R, d, E, F, w + L.dab, offsets, w_gate, w_up, w + L.dx_perm, ffn_ws, stream)
             : moe::launch_bwd_f32_dx_perm(R, d, E, F, w + L.dab, offsets, w_gate, w_up, w + L.dx_perm, stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_wgrad(E, offsets, 2 * F, F, d, 2 * F, d, R, w + L.dab, w + L.x_perm, dw_gate, dw_up,
                                 stream)
             : moe::launch_wgrad_f32(E, offsets, 2 * F, F, d, 2 * F, d, w + L.dab, w + L.x_perm, dw_gate, dw_up,
                                     stream);
  if (e == hipSuccess)
    e = bf16 ? moe::launch_wgrad(E, offsets, d, d, F, d, F, R, w + L.d_o, w + L.h, dw_down, nullptr, stream)
             : moe::launch_wgrad_f32(E, offsets, d, d, F, d, F, w + L.d_o, w + L.h, dw_down, nullptr, stream);
  // router weight and input gradients (dl is dense [T, E])
  if (e == hipSuccess)
    e = moe::launch_router_wgrad(T, d, E, k, x, nullptr, dl, reinterpret_cast<float*>(w + L.router_part), dw_router,
                                 stream, true, bf16);
  if (e == hipSuccess)
    e = moe::launch_ec_dx_final(bf16, T, d, E, R, dl, w_router, w + L.dx_perm, slot, dx, stream);
  return hip_status(e);
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, limit or alignment";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
