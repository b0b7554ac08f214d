"""CPU oracle for the forward pass of a token-choice Mixture-of-Experts FFN layer.

TEST INFRASTRUCTURE ONLY. This module is imported by tests/, by
__graft_entry__.smoke() and by bench.py's cpu_baseline leg, and by nothing
else. The HIP library and its Python binding never import or call it, and it
imports nothing from them: the only code both sides share is the seeded input
generator (moe_inputs), which holds none of the layer's arithmetic.

It is the plain definition of the layer, computed slowly in float64 with numpy
(matrix products use numpy's matmul as a library step; there is no blocking,
fusion or reordering beyond what the definition states). Each function names
the passage it follows. Sources:

  [MATH]  "How do Mixture of Expert Models Work?" (amks.me/notes/moe), section
          "The Math Behind MoEs": the layer output is the sum over experts of
          the gate value times the expert's output; dense gating is
          Softmax(x.W_g); sparse gating is Softmax(TopK(x.W_g)), the softmax
          of only the top-K logits with every other gate set to 0; Mixtral's
          experts are SwiGLU and it routes with Top2.
  [CAPN]  same page, section "Load Balancing", item "Expert Capacity": each
          expert takes at most a set number of tokens; overflow tokens skip
          the layer or are dropped.
  [TALK]  "[Paper Club] Upcycling Large Language Models into Mixture of
          Experts", the MoE-layer walkthrough: routing by a plain matrix
          multiply, permutation of each expert's tokens into one matrix
          (dropping tokens by capacity factor), the original FFN as the
          expert, un-permutation back to the token order, and scaling by the
          router probability. Its upcycling part: TopK then Softmax sums to
          one (0.7/0.3 example); copied identical experts reproduce the dense
          model; top-1 softmax is always one.
  [VMOE]  "Scaling Vision with Sparse Mixture of Experts" (Google Research
          post), section "Priority Routing": a fixed buffer per expert, and
          tokens assigned beyond it are dropped once the expert is full.
  [ROUTE] "Take a Closer Look at the MoE LLM Routing" (OpenMoE), Introduction,
          "Drop-towards-the-End": capacity makes tokens later in the sequence
          drop more often, i.e. the buffers fill in token order.

Readings where the pages are silent (each is listed in the design notes):
  * top-k ties go to the lower expert index; slots are ordered by descending
    logit (ties by ascending index);
  * the top-k decision is taken on float32 logits, the precision in which the
    kernel holds them; gate values use the float64 logits;
  * capacity = ceil(cf*T*k/E) computed in double, clamped to T; cf == 0 means
    dropless (capacity T);
  * a dropped slot contributes 0 and the remaining gates are not renormalised;
  * SwiGLU(x) = W_down (silu(W_gate x) * (W_up x)), silu(a) = a/(1+exp(-a)),
    no biases;
  * Switch gating ([TALK] upcycling part): softmax over all E logits, then
    the k chosen probabilities as gates (no renormalisation); the E/k
    output rescale is applied to each kept gate, which is the same as
    scaling the expert outputs since the combine is linear. The chosen set
    is the same as for Softmax(TopK) (softmax is monotone), decided on the
    float32 logits as above;
  * Batch Priority Routing ([VMOE] "Priority Routing"): the pages do not
    define the importance score; the layer uses each token's top-1 gate.
    Buffers fill in descending score order (the score taken as float32, the
    precision the kernels hold gates in), ties to the lower token index;
    rows inside an expert's segment follow that fill order;
  * expert choice ([TALK] "the selection is reversed": each expert takes a
    fixed number of tokens, so a token gets from zero to all experts): the
    token-expert score is the dense gate Softmax(x.W_g) of [MATH]; expert e
    takes the C = capacity(T, E, k, cf) tokens with the largest score[t, e]
    (k read as the average number of experts per token), compared as
    float32, ties to the lower token index; its rows list them in ascending
    token order; the gate of (t, e) is score[t, e] (not renormalised) and
    y[t] sums over the experts that chose t, in ascending expert order;
  * backward pass ([TALK]: the permutation is recomputed in the backward
    pass instead of being stored): routing, permutation, a = x W_gate^T,
    b = x W_up^T, h and o are recomputed from the inputs; the gradient
    follows the chain rule of the forward definition with these storage
    rounding points: a, b (recomputed, held in the storage type), the
    expert-output gradient d_o = g * dy, the SwiGLU input gradients da, db,
    the permuted input gradient dx_perm, and every returned gradient. The
    router gradient includes dropped slots (their gates still enter the
    softmax of the chosen logits). Under expert choice the selection passes
    no gradient and the gates are the dense scores, so every logit of a
    token that some expert chose gets gradient through the full softmax;
  * "storage" rounding: the layer stores h, o and y in its storage type. In
    "bf16" mode the float64 value is rounded to float32 and then to bfloat16
    (round to nearest even); in "f32" mode to float32; in "f64" mode not at
    all (used by the self-checks).
"""
from __future__ import annotations

import math

import numpy as np

STORAGE_MODES = ("f64", "f32", "bf16")


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def round_to_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32. bfloat16 keeps the top 16 bits of the float32 pattern; adding
    0x7FFF plus the lowest kept bit and truncating is round-half-to-even on the
    dropped 16 bits. Finite inputs only (the layer's inputs are finite)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u << 16).astype(np.uint32).view(np.float32)


def store(v: np.ndarray, storage: str) -> np.ndarray:
    """Value of v after being written in the layer's storage type, as float64."""
    if storage == "f64":
        return np.asarray(v, dtype=np.float64)
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if storage == "f32":
        return v32.astype(np.float64)
    if storage == "bf16":
        return round_to_bf16(v32).astype(np.float64)
    raise ValueError(storage)


def as_f64(a) -> np.ndarray:
    """float64 copy of an input array (torch tensor of any float dtype or numpy)."""
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# routing  [MATH] Softmax(TopK(x.W_g)); [TALK] the router is a matrix multiply
# ---------------------------------------------------------------------------

def router_logits(x, w_router) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_g[e, i]  (x.W_g with W_g stored [E, d]).

    [TALK]: the router is simply a learnable matrix applied to the tokens;
    [MATH]: the gating network's argument is x.W_g. No bias, no noise."""
    return as_f64(x) @ as_f64(w_router).T


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits per token, in slot order.

    [MATH] TopK keeps the k largest logits. The comparison is done on the
    float32 values of the logits; ties go to the lower expert index, and slots
    run from the largest logit down."""
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32)
    order = np.argsort(-l32, axis=1, kind="stable")   # stable: equal values keep index order
    return order[:, :k].astype(np.int32)


def topk_gates(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g[t, j] = exp(l[t, S_j]) / sum_{j'} exp(l[t, S_j']) over the chosen k.

    [MATH] the gate is the softmax of only the top-K values; the others are 0
    (they are not represented in the [T, k] layout). The largest chosen logit
    is subtracted before exp, which leaves the softmax unchanged."""
    v = np.take_along_axis(np.asarray(logits, np.float64), idx.astype(np.int64), axis=1)
    z = np.exp(v - v.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def switch_gates(logits: np.ndarray, idx: np.ndarray, scaled: bool) -> np.ndarray:
    """Switch-Transformer order ([TALK], upcycling part): p = softmax over all
    E logits first, then the gate of slot j is p[t, S_j]. The kept gates no
    longer sum to one (the talk's 0.4 / 0.2 example). With scaled=True every
    kept gate is multiplied by E/k: the talk's fix scales the expert (MLP)
    output by the number of experts over top-k, and the combine is linear in
    the gate, so scaling the gate is the same operation."""
    l = np.asarray(logits, np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    g = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if scaled:
        E, k = l.shape[1], idx.shape[1]
        g = g * (E / k)
    return g


GATINGS = ("topk_softmax", "softmax_topk", "softmax_topk_scaled")


def gates_for(logits: np.ndarray, idx: np.ndarray, gating: str) -> np.ndarray:
    """Gate values of the chosen slots under one of the gating rules:
    topk_softmax        Softmax(TopK(l)) ([MATH]; the layer's default)
    softmax_topk        TopK(Softmax(l)) (Switch order, [TALK])
    softmax_topk_scaled the same times E/k ([TALK]'s rescale)"""
    if gating == "topk_softmax":
        return topk_gates(logits, idx)
    if gating == "softmax_topk":
        return switch_gates(logits, idx, False)
    if gating == "softmax_topk_scaled":
        return switch_gates(logits, idx, True)
    raise ValueError(f"unknown gating {gating!r}")


def dense_gates(logits: np.ndarray, idx: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """The full G(x) of [MATH]: gate values at the chosen experts, 0 elsewhere."""
    T, E = logits.shape
    G = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(G, idx.astype(np.int64), gates, axis=1)
    return G


def near_tie_tokens(logits: np.ndarray, k: int, gap: float = 1e-5) -> np.ndarray:
    """Tokens whose routing could flip under float32 rounding of the logits:
    some adjacent gap among the sorted top-(k+1) float32 logits is below `gap`.
    (The k-th vs (k+1)-th gap decides the chosen set; the gaps inside the top k
    decide the slot order.)"""
    l32 = np.sort(np.asarray(logits, np.float64).astype(np.float32), axis=1)[:, ::-1]
    m = min(k + 1, l32.shape[1])
    if m < 2:
        return np.zeros(l32.shape[0], dtype=bool)
    gaps = l32[:, : m - 1].astype(np.float64) - l32[:, 1:m].astype(np.float64)
    return (gaps < gap).any(axis=1)


# ---------------------------------------------------------------------------
# capacity and permutation  [CAPN] [VMOE] [ROUTE] [TALK]
# ---------------------------------------------------------------------------

def capacity(T: int, E: int, k: int, cf: float) -> int:
    """Per-expert buffer size. [CAPN]/[VMOE] give a pre-set per-expert buffer
    set by a capacity factor (1 to 1.25 typical) but no formula. Reading:
    cap = ceil(cf * T * k / E) in double precision, clamped to T; cf == 0
    means dropless (cap = T). cf is taken as the float32 the C interface
    receives."""
    cf = float(np.float32(cf))
    if cf == 0.0:
        return int(T)
    return int(min(T, math.ceil(cf * T * k / E)))


def fill_in_order(idx: np.ndarray, E: int, cap: int, order):
    """Each expert's buffer fills as the tokens arrive in `order` (a
    permutation of 0..T-1); an assignment that arrives when the expert
    already holds `cap` tokens is dropped ([VMOE] dropped once the expert is
    full). A token's k slots arrive together, in slot order.

    Returns (demand[E], offsets[E+1], slot_row[T,k], row_slot[R]):
      demand[e]    tokens that chose e (kept or not)
      offsets      exclusive prefix sum of kept[e] = min(demand[e], cap):
                   expert e's rows are offsets[e] .. offsets[e+1]-1 ([TALK]
                   "arrange them into a single matrix" per expert)
      slot_row     row of (t, j) in the permuted matrix, -1 if dropped
      row_slot     inverse map: row -> t*k + j
    Rows inside an expert's segment are in arrival order."""
    T, k = idx.shape
    fill = np.zeros(E, dtype=np.int64)
    rank = np.empty((T, k), dtype=np.int64)
    for t in order:
        t = int(t)
        for j in range(k):
            e = int(idx[t, j])
            rank[t, j] = fill[e]
            fill[e] += 1
    kept = np.minimum(fill, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    keep = rank < cap
    slot_row = np.where(keep, offsets[idx.astype(np.int64)] + rank, -1)
    R = int(offsets[E])
    row_slot = np.full(R, -1, dtype=np.int64)
    tt, jj = np.nonzero(keep)
    row_slot[slot_row[tt, jj]] = tt * k + jj
    return (fill.astype(np.int32), offsets.astype(np.int32),
            slot_row.astype(np.int32), row_slot.astype(np.int32))


def layout_from_slot_rows(idx: np.ndarray, E: int, slot_row) -> tuple:
    """The permutation given its slot -> row map instead of a fill: a layout
    decided elsewhere (the routing-conditioned oracle takes the GPU's map where
    float32 ties leave the fill order open). Checks that every expert's kept
    slots occupy one contiguous block of rows, in ascending expert order from
    row 0, and returns (demand, offsets, slot_row, row_slot) like
    fill_in_order."""
    idx = np.asarray(idx)
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, k = idx.shape
    demand = np.bincount(idx.ravel().astype(np.int64), minlength=E)
    kept_e = np.bincount(idx[slot_row >= 0].astype(np.int64), minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept_e)
    R = int(offsets[E])
    row_slot = np.full(R, -1, dtype=np.int64)
    tt, jj = np.nonzero(slot_row >= 0)
    rows = slot_row[tt, jj]
    assert np.all(rows < R), "row beyond the kept rows"
    row_slot[rows] = tt * k + jj
    assert np.all(row_slot >= 0), "kept slots do not fill rows 0..R-1 once each"
    e_of_row = idx[tt, jj]
    assert np.all((rows >= offsets[e_of_row]) & (rows < offsets[e_of_row + 1])), "row outside its expert's block"
    return (demand.astype(np.int32), offsets.astype(np.int32), slot_row.astype(np.int32),
            row_slot.astype(np.int32))


def fill_in_token_order(idx: np.ndarray, E: int, cap: int):
    """Buffers fill in token order ([ROUTE] drops land towards the end of the
    sequence): fill_in_order with the identity order."""
    return fill_in_order(idx, E, cap, range(idx.shape[0]))


def priority_order(score) -> np.ndarray:
    """[VMOE] Batch Priority Routing: tokens are taken by descending
    importance score instead of position. The score is compared as float32
    (the precision of the gates the kernels hold); equal scores keep token
    order (a stable sort of the negated score)."""
    s32 = np.asarray(score, np.float64).astype(np.float32).astype(np.float64)
    return np.argsort(-s32, kind="stable")


def fill_in_priority_order(idx: np.ndarray, E: int, cap: int, score):
    """Batch Priority Routing: fill_in_order in descending score order."""
    return fill_in_order(idx, E, cap, priority_order(score))


# ---------------------------------------------------------------------------
# expert FFN  [MATH] Mixtral's SwiGLU experts; [TALK] the expert is the FFN
# ---------------------------------------------------------------------------

def silu(a: np.ndarray) -> np.ndarray:
    """Swish with beta = 1: a * sigmoid(a) = a / (1 + exp(-a))."""
    with np.errstate(over="ignore"):
        return a / (1.0 + np.exp(-a))


def swiglu_expert(xr, w_gate_e, w_up_e, w_down_e, storage: str):
    """One expert on its rows xr [n, d]:
        h = silu(xr W_gate^T) * (xr W_up^T)     stored   [n, F]
        o = h W_down^T                           stored   [n, d]
    with W_gate, W_up stored [F, d] and W_down stored [d, F]."""
    xr = as_f64(xr)
    a = xr @ as_f64(w_gate_e).T
    b = xr @ as_f64(w_up_e).T
    h = store(silu(a) * b, storage)
    o = store(h @ as_f64(w_down_e).T, storage)
    return h, o


# ---------------------------------------------------------------------------
# un-permute and combine  [MATH] y = sum_i G(x)_i E_i(x); [TALK] scale by the
# router probability after arranging the tokens back; [CAPN] dropped -> 0
# ---------------------------------------------------------------------------

def combine(o_rows: np.ndarray, slot_row: np.ndarray, gates: np.ndarray,
            storage: str, tokens=None) -> np.ndarray:
    """y[t] = sum over kept slots j (ascending) of g[t, j] * o[slot_row[t, j]].
    A token with no kept slot gets y = 0. `tokens` restricts the output to
    those token indices (o_rows must then hold every row they reference)."""
    slot_row = np.asarray(slot_row)
    if tokens is None:
        tokens = np.arange(slot_row.shape[0])
    tokens = np.asarray(tokens, dtype=np.int64)
    d = o_rows.shape[1]
    y = np.zeros((len(tokens), d), dtype=np.float64)
    for j in range(slot_row.shape[1]):
        r = slot_row[tokens, j]
        m = r >= 0
        y[m] += gates[tokens[m], j][:, None] * o_rows[r[m]]
    return store(y, storage)


# ---------------------------------------------------------------------------
# expert choice  [TALK] the experts select the tokens; [MATH] dense gating
# ---------------------------------------------------------------------------

def softmax_scores(logits: np.ndarray) -> np.ndarray:
    """[MATH] dense gating G(x) = Softmax(x.W_g): per token, the softmax over
    all E logits (the largest logit subtracted first)."""
    l = np.asarray(logits, np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def expert_choice_select(scores: np.ndarray, C: int):
    """Each expert takes the C tokens with the largest score in its column,
    compared as float32, equal scores to the lower token index ([TALK]: each
    expert selects a fixed number of tokens). Returns
      tokens [E, C]  the chosen tokens of each expert, ascending
      slot   [T, E]  row of (t, e) in the expert-major matrix (e*C + position
                     in tokens[e]), -1 if e did not choose t."""
    T, E = scores.shape
    s32 = np.asarray(scores, np.float64).astype(np.float32).astype(np.float64)
    tokens = np.empty((E, C), dtype=np.int32)
    slot = np.full((T, E), -1, dtype=np.int32)
    for e in range(E):
        best = np.argsort(-s32[:, e], kind="stable")[:C]
        chosen = np.sort(best)
        tokens[e] = chosen
        slot[chosen, e] = e * C + np.arange(C)
    return tokens, slot


def expert_choice_boundary_ties(scores: np.ndarray, C: int, gap: float = 2e-6) -> np.ndarray:
    """Experts whose C-th and (C+1)-th largest float32 scores are closer than
    `gap` (an ulp of difference in the kernel's float32 score could change
    the chosen set there)."""
    T, E = scores.shape
    if C >= T:
        return np.zeros(E, dtype=bool)
    s32 = np.sort(np.asarray(scores, np.float64).astype(np.float32).astype(np.float64), axis=0)[::-1]
    return (s32[C - 1] - s32[C]) < gap


def expert_choice_forward(x, w_router, w_gate, w_up, w_down, k: int, cf: float, storage: str,
                          tokens=None, slot=None) -> dict:
    """The layer with expert-choice routing. C = capacity(T, E, k, cf) tokens
    per expert (cf == 0: C = T, every expert takes every token).
    y[t] = store(sum over experts e that chose t, ascending, of
                 score[t, e] * FFN_e(x_t)); a token no expert chose gets 0.
    `tokens` restricts y to those tokens (every expert still runs its rows).
    `slot` [T, E] optionally replaces the selection (a choice taken elsewhere
    where float32 scores tie at an expert's C-th place): each expert must take
    exactly C tokens, on rows e*C .. e*C+C-1 in ascending token order."""
    T = x.shape[0]
    E = w_router.shape[0]
    logits = router_logits(x, w_router)
    S = softmax_scores(logits)
    C = capacity(T, E, k, cf)
    if slot is None:
        tok, slot = expert_choice_select(S, C)
    else:
        slot = np.asarray(slot, dtype=np.int32)
        tok = np.empty((E, C), dtype=np.int32)
        for e in range(E):
            chosen = np.nonzero(slot[:, e] >= 0)[0]
            assert len(chosen) == C and np.array_equal(slot[chosen, e], e * C + np.arange(C)), e
            tok[e] = chosen
    d = x.shape[1]
    F = w_gate.shape[1]
    o_rows = np.empty((E * C, d))
    h_rows = np.empty((E * C, F))
    for e in range(E):
        h, o = swiglu_expert(as_f64(x[tok[e]]), w_gate[e], w_up[e], w_down[e], storage)
        o_rows[e * C:(e + 1) * C] = o
        h_rows[e * C:(e + 1) * C] = h
    y = expert_choice_combine(o_rows, slot, S, storage, tokens)
    return dict(logits=logits, scores=S, cap=C, tokens=tok, slot=slot, y=y,
                o_rows=o_rows, h_rows=h_rows, boundary_tie=expert_choice_boundary_ties(S, C))


def expert_choice_combine(o_rows: np.ndarray, slot: np.ndarray, scores: np.ndarray, storage: str,
                          tokens=None) -> np.ndarray:
    """y[t] = store(sum over the experts e that chose t, ascending, of
    score[t, e] * o[slot[t, e]]). The gate is the dense score itself: it is
    not renormalised over the experts that happened to choose t ([TALK]: a
    token may get anywhere from zero to all experts), and a token no expert
    chose gets 0."""
    T, E = slot.shape
    if tokens is None:
        tokens = np.arange(T)
    tokens = np.asarray(tokens, dtype=np.int64)
    y = np.zeros((len(tokens), o_rows.shape[1]))
    for e in range(E):
        r = slot[tokens, e]
        m = r >= 0
        y[m] += scores[tokens[m], e][:, None] * o_rows[r[m]]
    return store(y, storage)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def route(x, w_router, k: int, gating: str = "topk_softmax"):
    """Routing step: logits, top-k indices (slot order), gates, near-tie mask."""
    logits = router_logits(x, w_router)
    idx = select_topk(logits, k)
    gates = gates_for(logits, idx, gating)
    return logits, idx, gates, near_tie_tokens(logits, k)


def forward(x, w_router, w_gate, w_up, w_down, k: int, cf: float, storage: str,
            tokens=None, idx=None, gating: str = "topk_softmax", bpr: bool = False,
            slot_row=None) -> dict:
    """The MoE layer forward pass.

    tokens: optional subset of token indices whose outputs are computed (the
            routing, capacity and permutation always cover all T tokens,
            since capacity depends on every earlier token).
    idx:    optional top-k indices to use instead of the router's choice
            (the gates still come from this oracle's logits at those experts).
    gating: one of GATINGS (see gates_for).
    bpr:    Batch Priority Routing: buffers fill in descending order of each
            token's top-1 gate instead of token order.
    slot_row: optional slot -> row map to use instead of the capacity fill
            (see layout_from_slot_rows); with idx, the layer conditioned on
            routing decisions taken elsewhere.
    Returns a dict with logits, topk_idx, topk_gate, near_tie, demand,
    offsets, slot_row, row_slot, cap, y (for `tokens`, or all tokens), and
    o_rows/h_rows (rows actually computed, indexed by permuted row; NaN
    elsewhere) when tokens is None."""
    T = x.shape[0]
    E = w_router.shape[0]
    logits = router_logits(x, w_router)
    if idx is None:
        idx = select_topk(logits, k)
    gates = gates_for(logits, idx, gating)
    cap = capacity(T, E, k, cf)
    if slot_row is not None:
        demand, offsets, slot_row, row_slot = layout_from_slot_rows(idx, E, slot_row)
    elif bpr:
        demand, offsets, slot_row, row_slot = fill_in_priority_order(idx, E, cap, gates[:, 0])
    else:
        demand, offsets, slot_row, row_slot = fill_in_token_order(idx, E, cap)
    R = int(offsets[E])
    if tokens is None:
        need_rows = np.arange(R)
    else:
        tokens = np.asarray(tokens, dtype=np.int64)
        r = slot_row[tokens].ravel()
        need_rows = np.unique(r[r >= 0])
    xf = x if hasattr(x, "shape") else np.asarray(x)
    d = xf.shape[1]
    F = w_gate.shape[1]
    o_rows = np.full((R, d), np.nan)
    h_rows = np.full((R, F), np.nan) if tokens is None else None
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = need_rows[(need_rows >= lo) & (need_rows < hi)]
        if len(rows) == 0:
            continue
        tok = row_slot[rows] // k
        h, o = swiglu_expert(as_f64(x[tok]), w_gate[e], w_up[e], w_down[e], storage)
        o_rows[rows] = o
        if h_rows is not None:
            h_rows[rows] = h
    y = combine(o_rows, slot_row, gates, storage, tokens)
    return dict(logits=logits, topk_idx=idx, topk_gate=gates,
                near_tie=near_tie_tokens(logits, k), demand=demand, offsets=offsets,
                slot_row=slot_row, row_slot=row_slot, cap=cap, y=y,
                o_rows=o_rows, h_rows=h_rows)


# ---------------------------------------------------------------------------
# backward pass  [TALK] (recomputed permutation); chain rule of the forward
# ---------------------------------------------------------------------------

def silu_grad(a: np.ndarray) -> np.ndarray:
    """d silu / da = sigma(a) * (1 + a * (1 - sigma(a)))."""
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-a))
    return sig * (1.0 + a * (1.0 - sig))


def topk_softmax_grad(gates: np.ndarray, dg: np.ndarray) -> np.ndarray:
    """Gradient through g = softmax(l_S) over the k chosen logits:
    dl_j = g_j (dg_j - sum_j' g_j' dg_j')."""
    return gates * (dg - (gates * dg).sum(axis=1, keepdims=True))


def switch_softmax_grad(logits: np.ndarray, idx: np.ndarray, dg: np.ndarray, scaled: bool) -> np.ndarray:
    """Gradient through the Switch gates g_j = s p[S_j], p = softmax over all E
    logits, s = E/k when scaled else 1 ([TALK] upcycling part). With
    D[e] = dg_j where e = S_j (0 for experts not chosen), the softmax's
    Jacobian gives, for every expert e (chosen or not):
        dl[e] = s p[e] (D[e] - sum_j p[S_j] dg_j).
    Returns the dense [T, E] gradient."""
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    k = idx.shape[1]
    z = np.exp(l - l.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    D = np.zeros((T, E))
    np.put_along_axis(D, idx.astype(np.int64), dg, axis=1)
    s = E / k if scaled else 1.0
    return s * p * (D - (p * D).sum(axis=1, keepdims=True))


def softmax_grad(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """Gradient through p = softmax(l) over the last axis, given dp = dL/dp:
    dl = p (dp - sum p dp) (the softmax's Jacobian diag(p) - p p^T)."""
    return p * (dp - (p * dp).sum(axis=-1, keepdims=True))


def gate_grad_dense(logits: np.ndarray, idx: np.ndarray, gates: np.ndarray, dg: np.ndarray,
                    gating: str) -> np.ndarray:
    """dL/dl [T, E] for a gate rule, given dg [T, k] = dL/dg: Softmax(TopK)
    puts topk_softmax_grad on the chosen logits (the others get 0); the
    Switch rules spread switch_softmax_grad over every logit."""
    T, E = logits.shape
    if gating == "topk_softmax":
        dl = np.zeros((T, E))
        np.put_along_axis(dl, idx.astype(np.int64), topk_softmax_grad(gates, dg), axis=1)
        return dl
    if gating in ("softmax_topk", "softmax_topk_scaled"):
        return switch_softmax_grad(logits, idx, dg, gating == "softmax_topk_scaled")
    raise ValueError(f"unknown gating {gating!r}")


BACKWARD_ROUNDING_POINTS = ("a", "b", "d_o", "da", "db", "dx_perm")


def hold(v: np.ndarray, storage: str, point: str) -> np.ndarray:
    """An intermediate of the backward pass as the layer holds it between its
    steps: written in the storage type like every stored activation. `point`
    names the rounding point (one of BACKWARD_ROUNDING_POINTS); it changes
    nothing here and lets a self-check drop one point at a time."""
    assert point in BACKWARD_ROUNDING_POINTS, point
    return store(v, storage)


def backward(x, w_router, w_gate, w_up, w_down, dy, k: int, cf: float, storage: str,
             weight_grad_experts=None, idx=None, gating: str = "topk_softmax", bpr: bool = False,
             slot_row=None) -> dict:
    """Gradients of L = <dy, y> for the token-choice layer, with respect to x
    and every weight. gating and bpr select the gate rule and the capacity
    fill order as in `forward`; the fill order is a discrete decision of the
    forward pass and passes no gradient.

    Forward (as `forward`): l = x W_g^T; S = TopK(l); g = softmax(l_S);
    a = x_perm W_gate^T, b = x_perm W_up^T; h = st(silu(a) b); o = st(h W_down^T);
    y = st(sum_j g_j o_j).  Backward, per kept row r = slot (t, j) of expert e:
      d_o[r]   = st(g_j dy[t])
      dg[t,j]  = <dy[t], o[r]>                  (0 for a dropped slot)
      dl[t,:]  = gate_grad_dense(l, S, g, dg, gating): for Softmax(TopK)
                 dl[t,S_j] = g_j (dg_j - sum_j' g_j' dg_j') and 0 elsewhere;
                 for the Switch rules every logit gets s p_e (D_e - sum p dg)
      dh[r]    = d_o[r] W_down[e]
      da[r]    = st(dh * b_st * silu'(a_st)),  db[r] = st(dh * silu(a_st))
                 with a_st = st(a), b_st = st(b)
      dx_perm  = st(da W_gate[e] + db W_up[e])
      dW_gate[e] = st(sum_r da[r]^T x_perm[r]),  dW_up[e] = st(sum_r db[r]^T x_perm[r])
      dW_down[e] = st(sum_r d_o[r]^T h[r])
      dW_g[e]  = st(sum_t dl[t, e] x[t])
      dx[t]    = st(sum_e dl[t, e] W_g[e] + sum over kept j of dx_perm[slot (t, j)])

    weight_grad_experts: None for the expert weight gradients of every expert;
    otherwise a list of experts, and dW_gate, dW_up and dW_down hold only theirs,
    in that order (the other results are the same either way).
    idx, slot_row: optional top-k indices and slot -> row layout to use
    instead of the router's choice and the capacity fill (as in `forward`:
    the layer conditioned on routing decisions taken elsewhere).
    """
    x64 = as_f64(x)
    T, d = x64.shape
    E = w_router.shape[0]
    F = w_gate.shape[1]
    wr = as_f64(w_router)
    r = forward(x, w_router, w_gate, w_up, w_down, k, cf, storage, idx=idx, gating=gating, bpr=bpr,
                slot_row=slot_row)
    idx, gates, slot_row, offsets, row_slot = r["topk_idx"], r["topk_gate"], r["slot_row"], r["offsets"], r["row_slot"]
    R = int(offsets[E])
    dy64 = as_f64(dy)
    tok = row_slot // k
    jj = row_slot % k
    a_st = np.empty((R, F))
    b_st = np.empty((R, F))
    h = np.empty((R, F))
    o = np.empty((R, d))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        xr = x64[tok[lo:hi]]
        a = xr @ as_f64(w_gate[e]).T
        b = xr @ as_f64(w_up[e]).T
        a_st[lo:hi] = hold(a, storage, "a")
        b_st[lo:hi] = hold(b, storage, "b")
        h[lo:hi] = store(silu(a) * b, storage)
        o[lo:hi] = store(h[lo:hi] @ as_f64(w_down[e]).T, storage)
    d_o = hold(gates[tok, jj][:, None] * dy64[tok], storage, "d_o")
    dg = np.zeros((T, k))
    kept = slot_row >= 0
    tt, kk = np.nonzero(kept)
    dg[tt, kk] = np.einsum("ij,ij->i", dy64[tt], o[slot_row[tt, kk]])
    dl_dense = gate_grad_dense(r["logits"], idx, gates, dg, gating)
    dl = np.take_along_axis(dl_dense, idx.astype(np.int64), axis=1)   # the chosen experts' entries
    dx_perm = np.empty((R, d))
    da_rows = np.empty((R, F))
    db_rows = np.empty((R, F))
    wg_experts = list(range(E)) if weight_grad_experts is None else [int(e) for e in weight_grad_experts]
    dW_gate = np.zeros((len(wg_experts), F, d))
    dW_up = np.zeros((len(wg_experts), F, d))
    dW_down = np.zeros((len(wg_experts), d, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        dh = d_o[lo:hi] @ as_f64(w_down[e])
        sa = silu(a_st[lo:hi])
        da = hold(dh * b_st[lo:hi] * silu_grad(a_st[lo:hi]), storage, "da")
        db = hold(dh * sa, storage, "db")
        da_rows[lo:hi] = da
        db_rows[lo:hi] = db
        dx_perm[lo:hi] = hold(da @ as_f64(w_gate[e]) + db @ as_f64(w_up[e]), storage, "dx_perm")
        if e in wg_experts:
            i = wg_experts.index(e)
            xr = x64[tok[lo:hi]]
            dW_gate[i] = da.T @ xr
            dW_up[i] = db.T @ xr
            dW_down[i] = d_o[lo:hi].T @ h[lo:hi]
    dW_g = dl_dense.T @ x64
    dx = dl_dense @ wr
    for j in range(k):
        m = slot_row[:, j] >= 0
        dx[m] += dx_perm[slot_row[m, j]]
    return dict(forward=r, dx=store(dx, storage), dW_g=store(dW_g, storage), dW_gate=store(dW_gate, storage),
                dW_up=store(dW_up, storage), dW_down=store(dW_down, storage), dl=dl, dl_dense=dl_dense, dg=dg, d_o=d_o,
                a_st=a_st, b_st=b_st, h=h, o=o, da=da_rows, db=db_rows, dx_perm=dx_perm)


def expert_choice_backward(x, w_router, w_gate, w_up, w_down, dy, k: int, cf: float, storage: str,
                           weight_grad_experts=None, slot=None) -> dict:
    """Gradients of L = <dy, y> for the expert-choice layer (as
    `expert_choice_forward`), with respect to x and every weight. Which tokens
    an expert takes is a discrete decision of the forward pass and passes no
    gradient; the gate of (t, e) is the dense score S[t, e] = softmax(l[t])[e]
    over all E logits ([MATH] dense gating), so every logit of a token that
    some expert chose gets gradient through the softmax.

    Per row r = slot[t, e] (expert e, token t):
      a, b, h, o  recomputed as in the forward (a and b held as stored)
      d_o[r]    = st(S[t, e] dy[t])
      dS[t, e]  = <dy[t], o[r]>                       (0 where e did not choose t)
      dl[t, :]  = S[t, :] (dS[t, :] - sum_e' S[t, e'] dS[t, e'])
      dh, da, db, dx_perm and the expert weight gradients as in `backward`
      dW_g      = st(dl^T x)
      dx[t]     = st(dl[t] W_g + sum over the experts e that chose t of dx_perm[slot[t, e]])

    weight_grad_experts: as in `backward`. slot: optional [T, E] selection to
    use instead of the scores' (as in `expert_choice_forward`)."""
    x64 = as_f64(x)
    T, d = x64.shape
    E = w_router.shape[0]
    F = w_gate.shape[1]
    wr = as_f64(w_router)
    r = expert_choice_forward(x, w_router, w_gate, w_up, w_down, k, cf, storage, slot=slot)
    S, C, tok, slot = r["scores"], r["cap"], r["tokens"], r["slot"]
    R = E * C
    dy64 = as_f64(dy)
    row_tok = tok.reshape(-1).astype(np.int64)   # row e*C + i holds token tokens[e, i]
    row_exp = np.repeat(np.arange(E), C)
    a_st = np.empty((R, F))
    b_st = np.empty((R, F))
    h = np.empty((R, F))
    o = np.empty((R, d))
    for e in range(E):
        lo, hi = e * C, (e + 1) * C
        xr = x64[row_tok[lo:hi]]
        a = xr @ as_f64(w_gate[e]).T
        b = xr @ as_f64(w_up[e]).T
        a_st[lo:hi] = hold(a, storage, "a")
        b_st[lo:hi] = hold(b, storage, "b")
        h[lo:hi] = store(silu(a) * b, storage)
        o[lo:hi] = store(h[lo:hi] @ as_f64(w_down[e]).T, storage)
    d_o = hold(S[row_tok, row_exp][:, None] * dy64[row_tok], storage, "d_o")
    dS = np.zeros((T, E))
    dS[row_tok, row_exp] = np.einsum("ij,ij->i", dy64[row_tok], o)
    dl = softmax_grad(S, dS)
    dx_perm = np.empty((R, d))
    da_rows = np.empty((R, F))
    db_rows = np.empty((R, F))
    wg_experts = list(range(E)) if weight_grad_experts is None else [int(e) for e in weight_grad_experts]
    dW_gate = np.zeros((len(wg_experts), F, d))
    dW_up = np.zeros((len(wg_experts), F, d))
    dW_down = np.zeros((len(wg_experts), d, F))
    for e in range(E):
        lo, hi = e * C, (e + 1) * C
        dh = d_o[lo:hi] @ as_f64(w_down[e])
        da = hold(dh * b_st[lo:hi] * silu_grad(a_st[lo:hi]), storage, "da")
        db = hold(dh * silu(a_st[lo:hi]), storage, "db")
        da_rows[lo:hi] = da
        db_rows[lo:hi] = db
        dx_perm[lo:hi] = hold(da @ as_f64(w_gate[e]) + db @ as_f64(w_up[e]), storage, "dx_perm")
        if e in wg_experts:
            i = wg_experts.index(e)
            xr = x64[row_tok[lo:hi]]
            dW_gate[i] = da.T @ xr
            dW_up[i] = db.T @ xr
            dW_down[i] = d_o[lo:hi].T @ h[lo:hi]
    dW_g = dl.T @ x64
    dx = dl @ wr
    np.add.at(dx, row_tok, dx_perm)
    return dict(forward=r, dx=store(dx, storage), dW_g=store(dW_g, storage), dW_gate=store(dW_gate, storage),
                dW_up=store(dW_up, storage), dW_down=store(dW_down, storage), dl=dl, dS=dS, d_o=d_o,
                a_st=a_st, b_st=b_st, h=h, o=o, da=da_rows, db=db_rows, dx_perm=dx_perm)
