/*
 * moe.h -- C interface of libmoe: the forward pass of a token-choice
 * Mixture-of-Experts FFN layer on one AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages define it:
 *   - "How do Mixture of Expert Models Work?", section "The Math Behind MoEs":
 *     y = sum_i G(x)_i E_i(x) with G(x) = Softmax(TopK(x.W_g)) -- the softmax
 *     of only the k largest router logits, every other gate 0 -- and, for
 *     Mixtral, SwiGLU experts with Top2.
 *   - "[Paper Club] Upcycling Large Language Models into Mixture of Experts",
 *     the MoE-layer walkthrough: route (the router is a plain matrix multiply),
 *     permute (gather each expert's tokens into one matrix, dropping tokens by
 *     capacity factor), run the experts (a grouped GEMM over any number of
 *     experts and tokens in one operation), un-permute back to the token
 *     order, and scale by the router probability.
 *   - Capacity: "How do Mixture of Expert Models Work?", section "Load
 *     Balancing" (Expert Capacity); "Scaling Vision with Sparse Mixture of
 *     Experts", section "Priority Routing" (a fixed buffer per expert; tokens
 *     beyond it are dropped once the expert is full); "Take a Closer Look at
 *     the MoE LLM Routing", Introduction (drops land towards the end of the
 *     sequence, i.e. buffers fill in token order).
 *
 * Conventions for every entry point:
 *   - Problem scalars: T tokens, hidden size d, E experts, top-k, capacity
 *     factor cf, expert FFN width F.
 *   - Layouts are row-major. Weight matrices are [out, in] with the input
 *     dimension contiguous: w_router [E, d], w_gate and w_up [E, F, d],
 *     w_down [E, d, F].
 *   - dtype: MOE_BF16 stores x, weights, x_perm, h, out_perm and y as
 *     bfloat16 (accumulation in fp32); MOE_F32 stores them as fp32. Logits and
 *     gates are always fp32; indices and row maps are int32.
 *   - Capacity: cap = T if cf == 0 (dropless), else min(T, ceil(cf*T*k/E))
 *     computed in double. Expert e keeps its first min(demand_e, cap)
 *     assignments in token order; later ones are dropped and contribute 0
 *     to y (the remaining gates are not renormalised).
 *   - R_max = min(T*k, E*cap) bounds the number of kept rows R; permuted
 *     buffers (x_perm, h, out_perm, row_slot) have R_max rows. The actual R
 *     = expert_offsets[E] stays on the device; rows at or beyond it are left
 *     untouched.
 *   - Ownership: the caller allocates every device buffer; the library never
 *     allocates or frees device memory and keeps no state between calls.
 *     Device pointers must be 16-byte aligned. Inputs and outputs must not
 *     overlap.
 *   - Asynchrony: every call only enqueues kernels on `stream` (NULL = the
 *     null stream) and returns; it never synchronises. Outputs are valid once
 *     the caller has synchronised the stream.
 *   - Errors: arguments are checked on the host before any launch; a failing
 *     check returns its status and enqueues nothing. MOE_ERR_HIP reports a
 *     launch error (hipGetLastError after the launches); faults during
 *     execution surface at the caller's synchronisation, as usual in HIP.
 *   - T == 0 is a valid empty problem: the call returns MOE_OK and enqueues
 *     nothing (pointers are not inspected).
 *   - Compiled limits (MOE_ERR_UNSUPPORTED beyond them): E <= 256, k <= 8,
 *     T*k < 2^31, d and F at most 2^24; d and F multiples of 8 (bf16) or 4
 *     (fp32); for bf16 the grouped FFN also needs d and F to be multiples of
 *     64. The size queries refuse T >= 2^31 the same way.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Storage type of activations and weights. Entry points take it as an
 * int32_t `dt` holding one of these values, so that any other value is a
 * well-defined MOE_ERR_INVALID_ARG rather than an out-of-range enum. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Gate rule of the router (the chosen experts are the same under every rule;
 * softmax is monotone):
 *   MOE_GATING_TOPK_SOFTMAX        Softmax(TopK(l)): the softmax of the k
 *       chosen logits, summing to 1 ("The Math Behind MoEs"; Mixtral).
 *   MOE_GATING_SOFTMAX_TOPK        TopK(Softmax(l)): the softmax over all E
 *       logits at the chosen experts, which no longer sum to 1 (the
 *       Switch-Transformer order in the upcycling talk, its 0.4 / 0.2
 *       example).
 *   MOE_GATING_SOFTMAX_TOPK_SCALED the same, times E/k: the talk's rescale
 *       of the expert outputs by the number of experts over top-k, applied to
 *       the gates (the combine is linear in them). */
typedef enum {
  MOE_GATING_TOPK_SOFTMAX = 0,
  MOE_GATING_SOFTMAX_TOPK = 1,
  MOE_GATING_SOFTMAX_TOPK_SCALED = 2
} moe_gating;

/* Order in which the expert buffers fill up to capacity:
 *   MOE_FILL_TOKEN_ORDER  by token index (drops land towards the end of the
 *       sequence: "Take a Closer Look at the MoE LLM Routing", Introduction).
 *   MOE_FILL_PRIORITY     Batch Priority Routing ("Scaling Vision with Sparse
 *       Mixture of Experts", section "Priority Routing"): tokens are taken
 *       by descending importance score; equal scores (compared as float32,
 *       -0 equal to +0) keep token order. NaN scores are not supported. */
typedef enum { MOE_FILL_TOKEN_ORDER = 0, MOE_FILL_PRIORITY = 1 } moe_fill_order;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null pointer, bad scalar, overlapping buffers */
  MOE_ERR_UNSUPPORTED = 2,   /* outside the compiled limits, or misaligned pointer */
  MOE_ERR_WORKSPACE = 3,     /* workspace too small */
  MOE_ERR_HIP = 4            /* a HIP runtime call failed */
} moe_status;

/* Per-expert capacity for the given problem (host only, pure).
 * Returns -1 if T < 0, E < 1, k not in [1, E] or cf negative / not finite. */
int64_t moe_capacity(int64_t T, int32_t E, int32_t k, float cf);

/* R_max = min(T*k, E*cap): the row count to allocate for x_perm, h, out_perm
 * and row_slot. Host only. MOE_ERR_INVALID_ARG for invalid scalars (as
 * moe_capacity), MOE_ERR_UNSUPPORTED for T >= 2^31. */
int moe_rows_max(int64_t T, int32_t E, int32_t k, float cf, int64_t* rows);

/* Workspace bytes needed by moe_permute (per-chunk expert histograms). */
int moe_permute_workspace_bytes(int64_t T, int32_t E, size_t* bytes);

/* Workspace bytes needed by moe_permute_priority (the histograms, the
 * priority order and the radix sort's key / value buffers). */
int moe_permute_priority_workspace_bytes(int64_t T, int32_t E, size_t* bytes);

/* Workspace bytes of moe_grouped_ffn / moe_expert_down: fp32 partial tiles
 * for the down projection's split tail (one 256 x 256 tile per compute unit
 * of the current device at most; 0 when the problem uses no split). Query it
 * with the device the calls will run on current. */
int moe_ffn_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                            int32_t dt, size_t* bytes);

/* Workspace bytes needed by moe_forward and moe_forward_ex (routing outputs,
 * row maps, x_perm, h, out_perm, the permutation's histograms, the priority
 * sort's buffers and the FFN's split-tail partials, each 256-byte aligned;
 * depends on the current device). */
int moe_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf,
                        int32_t F, int32_t dt, size_t* bytes);

/* Router: logits l = x . W_g^T (fp32 accumulation), the k largest per token
 * in slot order (descending logit, ties to the lower expert index) and their
 * softmax gates ("The Math Behind MoEs": Softmax(TopK(x.W_g))).
 *   x          [T, d]  dt        input tokens
 *   w_router   [E, d]  dt        router weight
 *   topk_idx   [T, k]  int32     out: chosen experts
 *   topk_gate  [T, k]  fp32      out: gates, summing to 1 per token
 *   logits_opt [T, E]  fp32      out (optional, NULL to skip): router logits */
int moe_route(int64_t T, int32_t d, int32_t E, int32_t k, int32_t dt,
              const void* x, const void* w_router,
              int32_t* topk_idx, float* topk_gate, float* logits_opt,
              hipStream_t stream);

/* moe_route with a selectable gate rule (moe_gating); moe_route is
 * gating = MOE_GATING_TOPK_SOFTMAX. Same indices for every rule; under the
 * softmax-first rules topk_gate[t, j] = p[t, S_j] (times E/k when scaled)
 * with p the softmax over all E logits. An unknown rule is
 * MOE_ERR_INVALID_ARG. */
int moe_route_gating(int64_t T, int32_t d, int32_t E, int32_t k, int32_t dt, int32_t gating,
                     const void* x, const void* w_router,
                     int32_t* topk_idx, float* topk_gate, float* logits_opt,
                     hipStream_t stream);

/* Permutation with token-order capacity (the walkthrough's permute step).
 *   topk_idx        [T, k]      int32  in: from moe_route. A token's k ids
 *                                      must be distinct experts in [0, E)
 *                                      (moe_route guarantees it); an id
 *                                      outside [0, E) is a dropped slot; with
 *                                      a repeated id the call stays inside its
 *                                      buffers but its counts, row maps and
 *                                      x_perm are unspecified
 *   expert_counts   [E]         int32  out: demand, tokens that chose e
 *   expert_offsets  [E + 1]     int32  out: exclusive prefix sum of
 *                                      kept_e = min(demand_e, cap)
 *   slot_row        [T, k]      int32  out: row of (t, j) in x_perm, -1 if dropped
 *   row_slot        [R_max]     int32  out: t*k + j for each kept row
 *   x_perm          [R_max, d]  dt     out: x_perm[slot_row[t,j]] = x[t];
 *                                      expert-major, token order inside an expert
 *   ws, ws_bytes                       scratch, >= moe_permute_workspace_bytes */
int moe_permute(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                const void* x, const int32_t* topk_idx,
                int32_t* expert_counts, int32_t* expert_offsets,
                int32_t* slot_row, int32_t* row_slot, void* x_perm,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_permute for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same arguments, arithmetic and outputs as
 * moe_permute, without ws / ws_bytes: the permutation's scratch (per-chunk
 * expert histograms, ceil(T / 256) * E * 4 bytes rounded up to 256) is a
 * file-scope device array of moe_permute_noalloc_scratch_bytes() = 1 MiB
 * that each GPU holds until the process ends. Problems whose scratch would
 * exceed it return MOE_ERR_WORKSPACE (E = 256 fits up to 262144 tokens,
 * E = 8 up to 8388608). The call allocates nothing: its first call on a device looks
 * up that device's copy of the array (hipGetSymbolAddress, with the device
 * current; MOE_ERR_HIP if that fails) and keeps the address. Every call on
 * a GPU shares that GPU's array, and the array keeps the last call's
 * contents (every histogram entry is rewritten before it is read, so no
 * clearing is needed): calls that overlap in time on one GPU, on different
 * streams, race on it and must be serialised by the caller. `stream` must
 * belong to the current device. */
int moe_permute_noalloc(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                        const void* x, const int32_t* topk_idx,
                        int32_t* expert_counts, int32_t* expert_offsets,
                        int32_t* slot_row, int32_t* row_slot, void* x_perm, hipStream_t stream);

/* Size in bytes of moe_permute_noalloc's device scratch array (host only). */
size_t moe_permute_noalloc_scratch_bytes(void);

/* moe_permute with Batch Priority Routing (MOE_FILL_PRIORITY): token t's
 * importance is score[t * score_stride] (fp32, device; pass topk_gate with
 * stride k for the top-1 gate). Each expert keeps, among the tokens that
 * chose it, the min(demand, cap) of highest score (ties to the lower token
 * index), and its rows in x_perm follow that order instead of token order.
 * Counts and offsets are as for moe_permute.
 *   score, score_stride  fp32 device array, 4-byte aligned; stride >= 1
 *   ws, ws_bytes         scratch, >= moe_permute_priority_workspace_bytes */
int moe_permute_priority(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                         const void* x, const int32_t* topk_idx,
                         const float* score, int64_t score_stride,
                         int32_t* expert_counts, int32_t* expert_offsets,
                         int32_t* slot_row, int32_t* row_slot, void* x_perm,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped SwiGLU expert FFN over the permuted rows, one launch per
 * projection for all experts (the walkthrough's grouped GEMM; Mixtral's
 * SwiGLU experts in "The Math Behind MoEs"). For each expert e and each row r
 * in [expert_offsets[e], expert_offsets[e+1]):
 *   h[r, :]        = store(silu(x_perm[r] . W_gate[e]^T) * (x_perm[r] . W_up[e]^T))
 *   out_perm[r, :] = store(h[r] . W_down[e]^T)
 * silu(a) = a / (1 + exp(-a)); "store" rounds the fp32 accumulator to dt.
 *   x_perm          [R_max, d]  dt
 *   expert_offsets  [E + 1]     int32 (device; read by the kernels)
 *   h_ws            [R_max, F]  dt    caller scratch, holds h on return
 *   out_perm        [R_max, d]  dt    out
 *   ws, ws_bytes                      scratch of moe_ffn_workspace_bytes; NULL
 *                                     runs the down projection without the
 *                                     split tail (same result, longer tail)
 * Scheduling: when the tile count of the down projection leaves a partial
 * last round on the device's compute units, each tile of that round is split
 * into K-slices whose fp32 partial sums are added in slice order before the
 * single rounding to dt, so results are deterministic. */
int moe_grouped_ffn(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                    int32_t dt, const void* x_perm, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, const void* w_down,
                    void* h_ws, void* out_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two launches of moe_grouped_ffn, for callers that schedule (or time)
 * them separately. Same arguments, layouts and arithmetic as above:
 *   moe_expert_gate_up: h = store(silu(x_perm . W_gate^T) * (x_perm . W_up^T))
 *   moe_expert_down:    out_perm = store(h . W_down^T)                       */
int moe_expert_gate_up(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                       int32_t dt, const void* x_perm, const int32_t* expert_offsets,
                       const void* w_gate, const void* w_up, void* h, hipStream_t stream);
int moe_expert_down(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                    int32_t dt, const void* h, const int32_t* expert_offsets,
                    const void* w_down, void* out_perm, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Un-permute and gate-weighted combine ("The Math Behind MoEs":
 * y = sum_i G(x)_i E_i(x); the walkthrough's un-permute then scale):
 *   y[t, :] = store(sum over kept slots j, ascending, of
 *                   topk_gate[t, j] * out_perm[slot_row[t, j], :])
 * summed in fp32 from +0; a token with every slot dropped gets y = 0.
 *   out_perm   [R_max, d]  dt
 *   slot_row   [T, k]      int32
 *   topk_gate  [T, k]      fp32
 *   y          [T, d]      dt    out */
int moe_unpermute_combine(int64_t T, int32_t d, int32_t E, int32_t k, float cf,
                          int32_t dt, const void* out_perm, const int32_t* slot_row,
                          const float* topk_gate, void* y, hipStream_t stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_ffn and
 * moe_unpermute_combine in sequence on one stream, with every intermediate
 * in the caller's workspace (no host synchronisation, no allocation).
 *   y                [T, d]  dt     out
 *   topk_idx_opt     [T, k]  int32  out (optional; NULL keeps it in ws)
 *   topk_gate_opt    [T, k]  fp32   out (optional)
 *   slot_row_opt     [T, k]  int32  out (optional)
 *   ws, ws_bytes                    scratch, >= moe_workspace_bytes */
int moe_forward(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                int32_t dt, const void* x, const void* w_router,
                const void* w_gate, const void* w_up, const void* w_down, void* y,
                int32_t* topk_idx_opt, float* topk_gate_opt, int32_t* slot_row_opt,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_forward with a gate rule (moe_gating) and a capacity fill order
 * (moe_fill_order). With MOE_FILL_PRIORITY the importance score of a token
 * is its top-1 gate under the chosen rule (the pages leave the score open).
 * moe_forward is (MOE_GATING_TOPK_SOFTMAX, MOE_FILL_TOKEN_ORDER). Unknown
 * values are MOE_ERR_INVALID_ARG. */
int moe_forward_ex(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                   int32_t dt, int32_t gating, int32_t fill_order,
                   const void* x, const void* w_router,
                   const void* w_gate, const void* w_up, const void* w_down, void* y,
                   int32_t* topk_idx_opt, float* topk_gate_opt, int32_t* slot_row_opt,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Expert-choice routing ("[Paper Club] Upcycling Large Language Models into
 * Mixture of Experts": the selection is reversed, each expert takes a fixed
 * number of tokens, so a token gets from zero to all E experts).
 *   score[t, e] = Softmax(x_t . W_g^T)[e], the dense gate of "The Math Behind
 *                 MoEs" (fp32; the softmax over all E logits of token t).
 *   C = moe_capacity(T, E, k, cf) tokens per expert, k read as the average
 *                 number of experts per token (cf == 0: C = T, every expert
 *                 takes every token, i.e. dense softmax gating).
 *   Expert e takes the C tokens with the largest score[:, e], compared as
 *   float32, equal scores to the lower token index. Its rows e*C .. e*C+C-1
 *   list them in ascending token order.
 *   y[t] = store(sum over the experts e that chose t, ascending, of
 *                score[t, e] * FFN_e(x_t)), fp32 from +0; y = 0 for a token
 *   no expert chose. Gates are not renormalised.
 * Limit: E * C < 2^31 (MOE_ERR_UNSUPPORTED beyond).
 * ------------------------------------------------------------------------- */

/* Scratch of moe_route_expert_choice (one key row of T per expert). */
int moe_route_expert_choice_workspace_bytes(int64_t T, int32_t E, size_t* bytes);

/* Router scores and the per-expert selection.
 *   scores          [T, E]     fp32   out: the dense gate
 *   expert_tokens   [E * C]    int32  out: token of each row (expert-major,
 *                                     ascending token inside an expert)
 *   slot            [T, E]     int32  out: row of (t, e), -1 if e did not take t
 *   expert_offsets  [E + 1]    int32  out: e * C (for the grouped FFN)
 *   ws, ws_bytes                      scratch, >= moe_route_expert_choice_workspace_bytes */
int moe_route_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                            const void* x, const void* w_router, float* scores,
                            int32_t* expert_tokens, int32_t* slot, int32_t* expert_offsets,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* Row gather: x_perm[r, :] = x[row_token[r], :] for r < R (a token index
 * outside [0, T) gives a zero row). x [T, d], x_perm [R, d], both dt. */
int moe_gather_rows(int64_t T, int32_t d, int64_t R, int32_t dt, const void* x,
                    const int32_t* row_token, void* x_perm, hipStream_t stream);

/* The grouped SwiGLU FFN of moe_grouped_ffn over any expert-major row set of
 * at most R_max rows (expert e owns rows expert_offsets[e] ..
 * expert_offsets[e+1]-1, offsets non-decreasing, expert_offsets[E] <= R_max).
 * Same arithmetic, layouts and split-tail workspace rules; the workspace
 * size comes from moe_ffn_rows_workspace_bytes. */
int moe_ffn_rows_workspace_bytes(int64_t R_max, int32_t d, int32_t E, int32_t F, int32_t dt,
                                 size_t* bytes);
int moe_grouped_ffn_rows(int64_t R_max, int32_t d, int32_t E, int32_t F, int32_t dt,
                         const void* x_perm, const int32_t* expert_offsets,
                         const void* w_gate, const void* w_up, const void* w_down,
                         void* h_ws, void* out_perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* Combine with a variable fan-in (y as above; rows outside [0, E*C) count as
 * not chosen).
 *   out_perm [E*C, d] dt, slot [T, E] int32, scores [T, E] fp32, y [T, d] dt out */
int moe_combine_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t dt,
                              const void* out_perm, const int32_t* slot, const float* scores,
                              void* y, hipStream_t stream);

/* The whole expert-choice layer on one stream, intermediates in ws.
 *   scores_opt [T, E] fp32 and slot_opt [T, E] int32 are optional outputs. */
int moe_forward_expert_choice_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf,
                                              int32_t F, int32_t dt, size_t* bytes);
int moe_forward_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                              int32_t dt, const void* x, const void* w_router,
                              const void* w_gate, const void* w_up, const void* w_down, void* y,
                              float* scores_opt, int32_t* slot_opt,
                              void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward pass of the token-choice layer (Softmax(TopK) gates, token-order
 * capacity), bf16 or fp32 storage ("bf16(...)" below is a rounding to the
 * storage type: a no-op beyond fp32 for MOE_F32, whose products run on the
 * vector ALUs).
 * Gradients of L = <dy, y> by the chain rule of the forward definition. The
 * routing, the permutation and the expert activations are recomputed from
 * the inputs (the upcycling talk's walkthrough recomputes the permutation in
 * the backward pass), then, per kept row r = slot (t, j) of expert e:
 *   d_o[r] = bf16(g_j dy[t]);  dg_j = <dy[t], o[r]> (0 for a dropped slot)
 *   dl_j   = g_j (dg_j - sum_j' g_j' dg_j')     (all k slots, dropped ones too)
 *   da[r]  = bf16(dh b silu'(a)), db[r] = bf16(dh silu(a)), dh = d_o[r] W_down[e],
 *            with a = bf16(x_perm W_gate^T), b = bf16(x_perm W_up^T) recomputed
 *   dx_perm[r] = bf16(da W_gate[e] + db W_up[e])
 *   dw_gate[e] = bf16(sum_r da^T x_perm), dw_up[e] = bf16(sum_r db^T x_perm),
 *   dw_down[e] = bf16(sum_r d_o^T h)   (an expert with no rows gets 0)
 *   dw_router[e] = bf16(sum over (t, j) with S_j = e of dl_j x[t])
 *   dx[t] = bf16(sum_j dl_j W_g[S_j] + sum over kept j of dx_perm[slot (t, j)])
 * All accumulation is fp32. Layouts: dx [T, d], dw_router [E, d],
 * dw_gate / dw_up [E, F, d], dw_down [E, d, F] (as the weights).
 * ws, ws_bytes: scratch of moe_backward_workspace_bytes (routing and
 * permutation maps, the recomputed x_perm, a, b, h and o, d_o, [da | db],
 * dx_perm, fp32 partial sums of the router gradient and the down projection's
 * split-tail partials; the size covers moe_backward_ex under every gate rule
 * and fill order); the GEMMs read weights and activations as stored.
 * Limits (MOE_ERR_UNSUPPORTED beyond), bf16: R_max * max(2F, d) * 2 bytes
 * and one expert's weight (d * F * 2 bytes) below 2^31, R_max the row bound
 * of moe_rows_max.
 * ------------------------------------------------------------------------- */
int moe_backward_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                                 int32_t dt, size_t* bytes);
int moe_backward(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                 const void* x, const void* w_router, const void* w_gate, const void* w_up,
                 const void* w_down, const void* dy,
                 void* dx, void* dw_router, void* dw_gate, void* dw_up, void* dw_down,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_backward for the layer of moe_forward_ex: a gate rule (moe_gating) and a
 * capacity fill order (moe_fill_order); moe_backward is
 * (MOE_GATING_TOPK_SOFTMAX, MOE_FILL_TOKEN_ORDER). The routing, the fill and
 * the activations are recomputed under the same rule and order. The fill
 * order is a discrete decision of the forward pass and carries no gradient;
 * it only decides which slots are kept. Under the Switch rules (gates
 * g_j = s p[S_j], p the softmax over all E logits, s = E/k for
 * MOE_GATING_SOFTMAX_TOPK_SCALED, else 1; the upcycling talk's Switch order)
 * every logit receives gradient, chosen or not:
 *   dl[e] = s p[e] (D[e] - sum_j p[S_j] dg_j),  D[S_j] = dg_j, else 0,
 *   dw_router[e] = bf16(sum_t dl[t, e] x[t]),
 *   dx[t] = bf16(sum_e dl[t, e] W_g[e] + sum over kept j of dx_perm[slot (t, j)]).
 * Everything else, the rounding points and the workspace are as for
 * moe_backward. Unknown rules or orders are MOE_ERR_INVALID_ARG. */
int moe_backward_ex(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F, int32_t dt,
                    int32_t gating, int32_t fill_order,
                    const void* x, const void* w_router, const void* w_gate, const void* w_up,
                    const void* w_down, const void* dy,
                    void* dx, void* dw_router, void* dw_gate, void* dw_up, void* dw_down,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward pass of the expert-choice layer (moe_forward_expert_choice), bf16
 * or fp32 storage. Gradients of L = <dy, y> by the chain rule of that
 * layer's definition. The selection (which tokens each expert takes) is a
 * discrete decision of the forward pass and carries no gradient; the gate of
 * (t, e) is the dense score S[t, e] = Softmax(x_t . W_g^T)[e] ("How do
 * Mixture of Expert Models Work?", "The Math Behind MoEs"), so every logit of
 * a token that some expert chose receives gradient through the softmax over
 * all E experts. The scores, the selection, the gathered rows and the expert
 * activations are recomputed from the inputs, then, per row r = slot[t, e]:
 *   d_o[r] = bf16(S[t, e] dy[t]);  dS[t, e] = <dy[t], o[r]> (0 if e did not take t)
 *   dl[t, :] = S[t, :] (dS[t, :] - sum_e S[t, e] dS[t, e])
 *   da, db, dx_perm, dw_gate, dw_up, dw_down as for moe_backward, over the
 *   E * C selected rows (every expert has C rows)
 *   dw_router[e] = bf16(sum_t dl[t, e] x[t])
 *   dx[t] = bf16(sum_e dl[t, e] W_g[e] + sum over the experts e that took t
 *                of dx_perm[slot[t, e]])   (0 for a token no expert took:
 *                its dS, and so its dl, is 0)
 * All accumulation is fp32; layouts as for moe_backward.
 * ws, ws_bytes: scratch of moe_backward_expert_choice_workspace_bytes (scores,
 * selection, the recomputed rows and activations, d_o, [da | db], dx_perm,
 * dl [T, E], router-gradient partial sums, split-tail partials).
 * Limits (MOE_ERR_UNSUPPORTED beyond): E * C < 2^31; bf16: E * C * max(2F, d)
 * * 2 bytes and one expert's weight (d * F * 2 bytes) below 2^31.
 * ------------------------------------------------------------------------- */
int moe_backward_expert_choice_workspace_bytes(int64_t T, int32_t d, int32_t E, int32_t k, float cf,
                                               int32_t F, int32_t dt, size_t* bytes);
int moe_backward_expert_choice(int64_t T, int32_t d, int32_t E, int32_t k, float cf, int32_t F,
                               int32_t dt, const void* x, const void* w_router, const void* w_gate,
                               const void* w_up, const void* w_down, const void* dy,
                               void* dx, void* dw_router, void* dw_gate, void* dw_up, void* dw_down,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/* Measurement aid, not part of the layer: the shader clock while other work
 * runs. Enqueues one wavefront on `stream` that waits `wall_ticks` ticks of
 * the device's constant-rate wall clock (see moe_wall_clock_khz) and writes
 * out[0] = core clock cycles counted meanwhile (s_memtime), out[1] = wall
 * ticks elapsed, so clock = out[0] / out[1] * wall rate. Run it on a second
 * stream beside a workload to see the clock the workload runs at (a
 * power-limited chip lowers it under dense MFMA work).
 *   out         uint64 [2], device, 16-byte aligned
 *   wall_ticks  1 .. 100000000 (MOE_ERR_INVALID_ARG otherwise) */
int moe_clock_probe(uint64_t* out, int64_t wall_ticks, hipStream_t stream);

/* Rate of the wall clock that moe_clock_probe counts, in kHz, for the
 * current device (hipDeviceAttributeWallClockRate). Host only. */
int moe_wall_clock_khz(int32_t* khz);

/* Static, NUL-terminated description of a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
