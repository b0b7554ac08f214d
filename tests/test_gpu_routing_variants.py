"""GPU parity for the routing variants: Switch gating (softmax over all
experts, then top-k, optionally times E/k) and Batch Priority Routing
(capacity filled in descending top-1-gate order), each against the CPU oracle
on the same seeded inputs, through the C interface."""
import functools

import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_09_amd as moe
from oracle import moe_oracle as orc
from parity import assert_close_rows, compare_routing, host
from test_gpu_parity import NAMED_SMALL, SMALL, case_id, dev, device_inputs, workload

pytestmark = pytest.mark.gpu

SWITCH = ["softmax_topk", "softmax_topk_scaled"]


@functools.lru_cache(maxsize=None)
def reference_ex(case, gating, bpr):
    w, a = workload(case)
    return orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                       gating=gating, bpr=bpr)


def ambiguous_tokens(score, x):
    """Tokens whose float32 score lies within 2e-6 of another token's with a
    different input row: the kernels' float32 gate may differ from the
    oracle's by an ulp, so such tokens may swap places in the priority order
    (identical rows get bit-identical gates on both sides). A swap changes the
    ranks of the tokens inside such a cluster only."""
    s = np.asarray(score, np.float64).astype(np.float32).astype(np.float64)
    order = np.argsort(-s, kind="stable")
    xs = np.asarray(x.float().numpy() if torch.is_tensor(x) else x)
    amb = np.zeros(len(s), dtype=bool)
    for a_, b_ in zip(order[:-1], order[1:]):
        if abs(s[a_] - s[b_]) <= 2e-6 and not np.array_equal(xs[a_], xs[b_]):
            amb[a_] = amb[b_] = True
    return amb


def check_rows_valid(srow, idx, offsets, k):
    """Kept rows of every expert are exactly its segment, each used once."""
    kept = srow >= 0
    rows = np.sort(srow[kept])
    assert np.array_equal(rows, np.arange(offsets[-1]))
    tt, jj = np.nonzero(kept)
    e = idx[tt, jj]
    assert np.all((srow[tt, jj] >= offsets[e]) & (srow[tt, jj] < offsets[e + 1]))


# ---------------------------------------------------------------------------
# Switch gating in the router
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gating", SWITCH)
@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_route_gating(case, gating):
    w, a = workload(case)
    logits, idx_ref, gate_ref, near = orc.route(a["x"], a["w_router"], w.k, gating=gating)
    g = device_inputs(case)
    idx, gate, lg = moe.moe_route(g["x"], g["w_router"], w.k, want_logits=True, gating=gating)
    torch.cuda.synchronize()
    flips = compare_routing(host(idx), host(gate), {"topk_idx": idx_ref, "topk_gate": gate_ref, "near_tie": near})
    assert flips == 0
    assert np.all(np.abs(host(lg) - logits) <= 1e-5 * (1.0 + np.abs(logits)))
    s = host(gate).sum(1)
    if gating == "softmax_topk":
        assert np.all(s <= 1.0 + 1e-6)
        if w.k == w.E:
            assert np.all(np.abs(s - 1.0) <= 1e-5)


@pytest.mark.parametrize("E,k", [(8, 2), (6, 4), (64, 8), (200, 3)])
def test_route_gating_zero_router(E, k):
    """W_g = 0: every probability is 1/E, so Switch gates are 1/E and the
    rescaled ones 1/k (the talk's "behaves like the dense model")."""
    T, d = 300, 128
    w = mi.Workload("zero", T=T, d=d, E=E, k=k, F=8, cf=0.0, dtype="bf16", seed=40)
    a = mi.generate(w, expert_weights=False)
    x = dev(a["x"])
    wr = torch.zeros((E, d), dtype=torch.bfloat16, device="cuda")
    idx, g1, _ = moe.moe_route(x, wr, k, gating="softmax_topk")
    _, g2, _ = moe.moe_route(x, wr, k, gating="softmax_topk_scaled")
    torch.cuda.synchronize()
    assert np.all(host(idx) == np.arange(k))
    assert np.allclose(host(g1), 1.0 / E, rtol=1e-6, atol=0)
    assert np.allclose(host(g2), 1.0 / k, rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# Batch Priority Routing in the permutation (oracle indices and scores in)
# ---------------------------------------------------------------------------

def run_permute_priority(w, a, idx, score_2d, stride_k):
    x = dev(a["x"])
    idx_d = dev(torch.from_numpy(np.ascontiguousarray(idx)))
    if stride_k:
        sc = dev(torch.from_numpy(np.ascontiguousarray(score_2d, dtype=np.float32)))
        out = moe.moe_permute(x, idx_d, w.E, w.cf, score=sc, score_stride=w.k)
    else:
        sc = dev(torch.from_numpy(np.ascontiguousarray(score_2d[:, 0], dtype=np.float32)))
        out = moe.moe_permute(x, idx_d, w.E, w.cf, score=sc, score_stride=1)
    torch.cuda.synchronize()
    return out


def check_permute_priority(w, a, idx, score_2d, stride_k):
    cap = orc.capacity(w.T, w.E, w.k, w.cf)
    s32 = score_2d[:, 0].astype(np.float32)
    demand, offsets, slot_row, row_slot = orc.fill_in_priority_order(idx, w.E, cap, s32)
    out = run_permute_priority(w, a, idx, score_2d, stride_k)
    R = int(offsets[-1])
    assert np.array_equal(host(out["expert_counts"]), demand)
    assert np.array_equal(host(out["expert_offsets"]), offsets)
    assert np.array_equal(host(out["slot_row"]), slot_row)
    assert np.array_equal(host(out["row_slot"])[:R], row_slot)
    xp = out["x_perm"][:R].cpu()
    assert torch.equal(xp, a["x"][torch.from_numpy(row_slot.astype(np.int64)) // w.k])


@pytest.mark.parametrize("stride_k", [True, False])
@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_permute_priority(case, stride_k):
    w, a = workload(case)
    logits, idx, gates, _ = orc.route(a["x"], a["w_router"], w.k)
    check_permute_priority(w, a, idx, gates.astype(np.float32), stride_k)


@pytest.mark.parametrize("T,E,k,cf,seed", [
    (70000, 16, 2, 0.8, 50),     # 274 chunks, ragged last chunk
    (5000, 64, 8, 0.3, 51),
    (257, 3, 2, 0.5, 52),
    (1, 4, 2, 1.0, 53),
    (16384, 8, 2, 0.5, 54),      # largest single-workgroup sort
    (16385, 8, 2, 0.5, 55),      # smallest radix sort
    (1024, 256, 8, 0.5, 56),     # the largest one-workgroup capacity layout
    (1025, 32, 4, 0.7, 57),      # the smallest chunked layout
])
def test_permute_priority_ties_and_sizes(T, E, k, cf, seed):
    """Many exact ties (a handful of score values, with -0 and +0 equal), the
    top bit of every radix digit used (negative scores), several sizes on both
    sides of the switch from the one-workgroup sort to the radix sort."""
    w = mi.Workload("bpr", T=T, d=64, E=E, k=k, F=8, cf=cf, dtype="f32", seed=seed)
    a = mi.generate(w, expert_weights=False)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    vals = np.array([0.75, 0.5, 0.25, 0.0, -0.0, -0.5, 1e-30, -3.4e38, 2.0 ** -126, 3e38], np.float32)
    score = rng.choice(vals, size=(T, k)).astype(np.float32)
    half = rng.random(T) < 0.5
    score[half, 0] = rng.standard_normal(int(half.sum())).astype(np.float32)
    check_permute_priority(w, a, idx, score, True)


# ---------------------------------------------------------------------------
# the whole layer with a gate rule and a fill order
# ---------------------------------------------------------------------------

def run_forward_ex(w, g, gating, fill):
    T = w.T
    idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    srow = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    y = moe.moe_forward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf,
                        topk_idx=idx, topk_gate=gate, slot_row=srow, gating=gating, fill_order=fill)
    torch.cuda.synchronize()
    return y, idx, gate, srow


VARIANTS = [("softmax_topk", "token"), ("softmax_topk_scaled", "token"), ("topk_softmax", "priority"),
            ("softmax_topk_scaled", "priority")]


@pytest.mark.parametrize("gating,fill", VARIANTS, ids=lambda v: v)
@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_forward_ex(case, gating, fill):
    w, a = workload(case)
    bpr = fill == "priority"
    ref = reference_ex(case, gating, bpr)
    g = device_inputs(case)
    y, idx, gate, srow = run_forward_ex(w, g, gating, fill)
    assert compare_routing(host(idx), host(gate), ref) == 0
    s = host(srow)
    if bpr:
        amb = ambiguous_tokens(ref["topk_gate"][:, 0], a["x"])
        assert np.array_equal(s[~amb], ref["slot_row"][~amb])
        check_rows_valid(s, host(idx), ref["offsets"], w.k)
        assert np.array_equal((s >= 0).sum(), (ref["slot_row"] >= 0).sum())
        print(f"{case_id(case)} {gating}/{fill}: {int(amb.sum())} ambiguous tokens")
        if amb.any() and not np.array_equal(s, ref["slot_row"]):
            # tied priorities: every token against the layer fed the kernel's layout
            ref = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                              gating=gating, idx=host(idx), slot_row=s)
    else:
        assert np.array_equal(s, ref["slot_row"])
    assert_close_rows(host(y), ref["y"], w.dtype)


def test_priority_with_equal_gates_is_token_order():
    """W_g = 0 makes every gate 1/k: the priority order is the token order, so
    BPR must give exactly the vanilla drops (tokens 0..cap-1 kept)."""
    w, a = mi.random_small(200, 128, 8, 2, 128, 0.5, "bf16", 21)
    a = dict(a)
    a["w_router"] = torch.zeros_like(a["w_router"])
    g = {k_: dev(v) for k_, v in a.items() if v is not None}
    y1, _, _, s1 = run_forward_ex(w, g, "topk_softmax", "priority")
    y0, _, _, s0 = run_forward_ex(w, g, "topk_softmax", "token")
    assert torch.equal(s1, s0)
    assert torch.equal(y1, y0)
    assert np.all(host(s1)[25:] == -1)


def test_priority_forward_is_deterministic():
    case = SMALL[0]
    w, _ = workload(case)
    g = device_inputs(case)
    first = [t.clone() for t in run_forward_ex(w, g, "softmax_topk_scaled", "priority")]
    for _ in range(5):
        for a_, b_ in zip(first, run_forward_ex(w, g, "softmax_topk_scaled", "priority")):
            assert torch.equal(a_, b_)


@pytest.mark.parametrize("name,gating,fill", [("openmoe_bf16", "softmax_topk_scaled", "priority"),
                                              ("openmoe_bf16", "topk_softmax", "priority"),
                                              ("mixtral_bf16", "softmax_topk_scaled", "token")])
def test_full_size_forward_ex(name, gating, fill):
    w, a = workload(name)
    bpr = fill == "priority"
    logits, idx_ref, gates, tie = orc.route(a["x"], a["w_router"], w.k, gating=gating)
    cap = orc.capacity(w.T, w.E, w.k, w.cf)
    if bpr:
        _, offsets, slot_row, _ = orc.fill_in_priority_order(idx_ref, w.E, cap, gates[:, 0])
    else:
        _, offsets, slot_row, _ = orc.fill_in_token_order(idx_ref, w.E, cap)
    ref = dict(topk_idx=idx_ref, topk_gate=gates, near_tie=tie, slot_row=slot_row)
    g = device_inputs(name)
    y, idx, gate, srow = run_forward_ex(w, g, gating, fill)
    assert compare_routing(host(idx), host(gate), ref) == 0
    s = host(srow)
    amb = ambiguous_tokens(gates[:, 0], a["x"]) if bpr else np.zeros(w.T, dtype=bool)
    assert np.array_equal(s[~amb], slot_row[~amb])
    check_rows_valid(s, host(idx), offsets, w.k)
    assert (s >= 0).sum() == (slot_row >= 0).sum()
    # every token, against the layer fed the kernel's routing and layout (the
    # two differ only where float32 priorities tie, and the check above bounds that)
    r = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                    gating=gating, idx=host(idx), slot_row=s)
    rel, mae = assert_close_rows(host(y), r["y"], w.dtype)
    print(f"{name} {gating}/{fill}: {int(amb.sum())} ambiguous, {int((s != slot_row).any(1).sum())} placed "
          f"differently, all {w.T} tokens, max-rel {rel:.3g}, MAE {mae:.3g}")
