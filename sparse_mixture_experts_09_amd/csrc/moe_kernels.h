// Kernel launchers of libmoe (internal; the public interface is include/moe.h).
// Every launcher only enqueues work on stream s and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// gating: 0 Softmax(TopK), 1 TopK(Softmax), 2 TopK(Softmax) * E/k,
// 3 expert-choice scores: Softmax over all E written to logits (idx, gate unused)
hipError_t launch_router(bool bf16, int64_t T, int d, int E, int k, int gating, const void* x, const void* wr,
                         int32_t* idx, float* gate, float* logits, hipStream_t s);

// Chunks of tokens used by the permutation's histogram (one int per expert each).
int64_t permute_chunks(int64_t T);

// order: token at each position of the arrival sequence for the capacity
// fill (nullptr: token order)
hipError_t launch_permute(bool bf16, int64_t T, int d, int E, int k, int64_t cap, const void* x,
                          const int32_t* idx, const int32_t* order, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* slot_row, int32_t* row_slot, void* x_perm,
                          int32_t* chunk_counts, hipStream_t s);

// Priority order for Batch Priority Routing: order[0..T) = tokens by score[t * stride]
// descending (as float32), equal scores by ascending token. ws: priority_sort_bytes(T).
size_t priority_sort_bytes(int64_t T);
hipError_t launch_priority_order(int64_t T, const float* score, int64_t stride, int32_t* order, void* ws,
                                 hipStream_t s);

// The two grouped GEMMs (which = 1: gate/up with the SwiGLU epilogue, 2: down).
// R_max bounds the rows in all, seg_max the rows of any one expert.
// ws (bf16 down projection only, may be NULL): ffn_bf16_workspace_bytes() of
// scratch for the partial tiles of its split tail.
// gather_slot (GEMM1 only, when ffn_bf16_can_gather): `in` is the unpermuted
// activations [gather_T, d] and permuted row r reads token gather_slot[r] /
// gather_k (the row -> slot map of the permutation), so no x_perm is needed.
hipError_t launch_gemm_bf16(int which, int64_t R_max, int64_t seg_max, int d, int E, int F, const void* in,
                            const int32_t* offsets, const void* w0, const void* w1, void* out,
                            void* ws, hipStream_t s, const int32_t* gather_slot = nullptr, int gather_k = 0,
                            int64_t gather_T = 0);
bool ffn_bf16_can_gather(int64_t R_max, int64_t seg_max, int d, int E, int F, int64_t T);
// whether moe_forward gathers (it does where that measured faster: k >= 4)
bool ffn_bf16_gathers(int64_t R_max, int64_t seg_max, int d, int E, int F, int64_t T, int k);
size_t ffn_bf16_workspace_bytes(int64_t R_max, int E);
int compute_units();
hipError_t launch_gemm_f32(int which, int64_t R_max, int d, int E, int F, const void* in,
                           const int32_t* offsets, const void* w0, const void* w1, void* out,
                           hipStream_t s);

hipError_t launch_ffn_bf16(int64_t R_max, int64_t seg_max, int d, int E, int F, const void* x_perm,
                           const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                           void* h, void* out, void* ws, hipStream_t s, const int32_t* gather_slot = nullptr,
                           int gather_k = 0, int64_t gather_T = 0);

hipError_t launch_ffn_f32(int64_t R_max, int d, int E, int F, const void* x_perm,
                          const int32_t* offsets, const void* wg, const void* wu, const void* wd,
                          void* h, void* out, hipStream_t s);

hipError_t launch_combine(bool bf16, int64_t T, int d, int k, const void* out_perm,
                          const int32_t* slot_row, const float* gate, void* y, hipStream_t s);

// Expert choice: per-expert selection of C tokens from the [T, E] scores
// (ws: ec_select_bytes), the row gather, and the variable fan-in combine.
size_t ec_select_bytes(int64_t T, int E);
hipError_t launch_ec_select(int64_t T, int E, int C, const float* scores, void* ws, int32_t* tokens,
                            int32_t* slot, int32_t* offsets, hipStream_t s);
hipError_t launch_gather_rows(bool bf16, int64_t T, int64_t R, int d, const void* x, const int32_t* row_token,
                              void* x_perm, hipStream_t s);
hipError_t launch_ec_combine(bool bf16, int64_t T, int d, int E, int64_t R, const void* out_perm,
                             const int32_t* slot, const float* scores, void* y, hipStream_t s);

// Backward pass (bf16): GEMMs on the grouped kernels (ffn_bf16.hip) and the
// transposes and per-token kernels of backward.hip.
hipError_t launch_bwd_recompute_gate_up(int64_t R_max, int d, int E, int F, const void* x_perm,
                                        const int32_t* offsets, const void* wg, const void* wu, void* h,
                                        void* a_st, void* b_st, hipStream_t s);
// dh and dx_perm read the weights as stored ([E, d, F] and [E, F, d]), with
// transposing LDS reads
hipError_t launch_bwd_dh(int64_t R_max, int d, int E, int F, const void* d_o, const int32_t* offsets,
                         const void* w_down, const void* a_st, const void* b_st, void* dab, hipStream_t s);
hipError_t launch_bwd_dx_perm(int64_t R_max, int d, int E, int F, const void* dab, const int32_t* offsets,
                              const void* w_gate, const void* w_up, void* dx_perm, void* ws, hipStream_t s);
// weight gradients over each expert's rows of A [R, lda] and B [R, ldb] (as stored)
hipError_t launch_wgrad(int E, const int32_t* offsets, int M, int M1, int N, int lda, int ldb, int64_t R,
                        const void* A, const void* B, void* C0, void* C1, hipStream_t s);
size_t router_wgrad_partial_bytes(int64_t T, int d, int E);
// logits == nullptr: Softmax(TopK) gates, dl [T, k]; else the Switch rules
// (logits [T, E] of the router, gate scale s), dl dense [T, E].
// Every tensor in the storage type (bf16: true; else fp32); dl, gates, logits fp32.
hipError_t launch_gate_bwd(int64_t T, int d, int k, const void* dy, const void* o, const int32_t* slot_row,
                           const float* gate, void* d_o, float* dl, hipStream_t s, int E = 0,
                           const int32_t* idx = nullptr, const float* logits = nullptr, float scale = 1.f,
                           bool bf16 = true);
hipError_t launch_router_wgrad(int64_t T, int d, int E, int k, const void* x, const int32_t* idx, const float* dl,
                               float* partial, void* dwg, hipStream_t s, bool dense = false, bool bf16 = true);
// dense_E > 0: dl is [T, dense_E]; 0: [T, k] at idx
hipError_t launch_dx_final(int64_t T, int d, int k, const float* dl, const int32_t* idx, const void* wr,
                           const void* dx_perm, const int32_t* slot_row, void* dx, hipStream_t s, int dense_E = 0,
                           bool bf16 = true);
// Expert-choice backward (ec_backward.hip): dS, d_o = S dy and dl [T, E]
// from the [T, E] slots and scores; dx from dl, W_g and the dx_perm rows.
hipError_t launch_ec_gate_bwd(bool bf16, int64_t T, int d, int E, int64_t R, const void* dy, const void* o,
                              const int32_t* slot, const float* scores, void* d_o, float* dl, hipStream_t s);
hipError_t launch_ec_dx_final(bool bf16, int64_t T, int d, int E, int64_t R, const float* dl, const void* wr,
                              const void* dx_perm, const int32_t* slot, void* dx, hipStream_t s);
// fp32 layers: the backward's GEMMs on the vector ALUs (ffn_f32.hip).
//   recompute: h = silu(a) b with a = x_perm W_gate^T, b = x_perm W_up^T, storing h, a and b
//   dh:        dh = d_o W_down[e] ([E, d, F] as stored), then da = dh b silu'(a) and
//              db = dh silu(a) written side by side into dab [R, 2F]
//   dx_perm:   dab [R, 2F] times [W_gate[e]; W_up[e]] ([F, d] each, as stored)
//   wgrad:     C[e] = A^T B over expert e's rows, A [R, lda] columns 0..M-1, B [R, ldb]
//              columns 0..N-1; rows of C below M1 go to C0 ([E, M1, N]), the rest to C1
hipError_t launch_bwd_f32_recompute(int64_t R_max, int d, int E, int F, const void* x_perm, const int32_t* offsets,
                                    const void* wg, const void* wu, void* h, void* a, void* b, hipStream_t s);
hipError_t launch_bwd_f32_dh(int64_t R_max, int d, int E, int F, const void* d_o, const int32_t* offsets,
                             const void* w_down, const void* a, const void* b, void* dab, hipStream_t s);
hipError_t launch_bwd_f32_dx_perm(int64_t R_max, int d, int E, int F, const void* dab, const int32_t* offsets,
                                  const void* w_gate, const void* w_up, void* dx_perm, hipStream_t s);
hipError_t launch_wgrad_f32(int E, const int32_t* offsets, int M, int M1, int N, int lda, int ldb, const void* A,
                            const void* B, void* C0, void* C1, hipStream_t s);

}  // namespace moe
