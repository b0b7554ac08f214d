"""Pins for the CPU oracle: each check ties it to something other than itself
(brute force on tiny inputs, closed forms, library routines in special cases,
values the pages print, invariants the pages state). The last group plants a
plausible mistake in the oracle and shows that some pin fails."""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import moe_inputs as mi
from oracle import moe_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *rest = line.split()
            vals[key] = [float(v) for v in rest]
    return vals


def small_layer(T=40, d=16, E=5, k=2, F=24, seed=7, dtype="f32", identical=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d)) / math.sqrt(d)
    wg = rng.standard_normal((E, F, d)) / math.sqrt(d)
    wu = rng.standard_normal((E, F, d)) / math.sqrt(d)
    wd = rng.standard_normal((E, d, F)) / math.sqrt(d)
    if identical:
        wg[:] = wg[0]
        wu[:] = wu[0]
        wd[:] = wd[0]
    if dtype == "bf16":
        cast = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()
        x, wr, wg, wu, wd = map(cast, (x, wr, wg, wu, wd))
    return x, wr, wg, wu, wd


# ---------------------------------------------------------------------------
# the pins, written as checks so that the planted-mistake tests can reuse them
# ---------------------------------------------------------------------------

def check_bf16_rounding():
    """round_to_bf16 == torch's float32 -> bfloat16 conversion, bit for bit."""
    rng = np.random.default_rng(0)
    parts = [rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32)]
    # exact ties (low 16 bits = 0x8000) with even and odd kept bit, both signs
    hi = rng.integers(0, 0x7F7F, 4000).astype(np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)
    parts += [ties, -ties]
    # just below / above a tie
    parts += [(hi | 0x7FFF).view(np.float32), (hi | 0x8001).view(np.float32)]
    # subnormals, zero, near overflow (rounds to inf)
    sub = rng.integers(1, 0x007FFFFF, 2000).astype(np.uint32).view(np.float32)
    parts += [sub, -sub, np.array([0.0, -0.0, 3.3895314e38, -3.3895314e38,
                                   np.finfo(np.float32).max, -np.finfo(np.float32).max], np.float32)]
    a = np.concatenate(parts).astype(np.float32)
    a = a[np.isfinite(a)]
    mine = orc.round_to_bf16(a).view(np.uint32)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy().view(np.uint32)
    assert np.array_equal(mine, ref), f"{(mine != ref).sum()} mismatches"


def check_silu_library():
    a = np.linspace(-60, 60, 2001)
    assert np.allclose(orc.silu(a), torch.nn.functional.silu(torch.from_numpy(a)).numpy(),
                       rtol=1e-14, atol=1e-300)


def brute_topk(l, k):
    """Max-sum subset of size k, lexicographically smallest among ties."""
    E = len(l)
    best, best_s = None, None
    for s in itertools.combinations(range(E), k):
        v = sum(l[i] for i in s)
        if best is None or v > best:
            best, best_s = v, s
    return best_s


def check_topk_bruteforce():
    rng = np.random.default_rng(1)
    for trial in range(300):
        E = int(rng.integers(1, 6))
        k = int(rng.integers(1, min(3, E) + 1))
        T = int(rng.integers(1, 7))
        # small integers give many exact ties
        logits = rng.integers(-2, 3, (T, E)).astype(np.float64) * 0.5
        if trial % 3 == 0:
            logits = rng.standard_normal((T, E))
        idx = orc.select_topk(logits, k)
        for t in range(T):
            assert tuple(sorted(idx[t].tolist())) == brute_topk(logits[t].astype(np.float32).tolist(), k)
            v = logits[t, idx[t]]
            # slots run from the largest logit down, ties by ascending index
            for j in range(k - 1):
                assert v[j] > v[j + 1] or (v[j] == v[j + 1] and idx[t, j] < idx[t, j + 1])


def check_zero_router_closed_form():
    """W_g = 0: every logit is 0, every token picks experts 0..k-1 with gates 1/k;
    with a finite capacity, experts 0..k-1 keep exactly tokens 0..cap-1."""
    T, d, E, k, F = 30, 8, 6, 3, 8
    x, _, wg, wu, wd = small_layer(T, d, E, k, F)
    wr = np.zeros((E, d))
    r = orc.forward(x, wr, wg, wu, wd, k, 1.0, "f64")
    assert np.array_equal(r["topk_idx"], np.tile(np.arange(k, dtype=np.int32), (T, 1)))
    assert np.all(r["topk_gate"] == 1.0 / k)
    cap = r["cap"]
    assert cap == math.ceil(1.0 * T * k / E) == 15
    assert np.array_equal(r["demand"], np.array([T] * k + [0] * (E - k)))
    assert np.array_equal(r["offsets"], np.array([0] + [cap * (i + 1) for i in range(k)] + [cap * k] * (E - k)))
    for j in range(k):
        kept_tokens = np.nonzero(r["slot_row"][:, j] >= 0)[0]
        assert np.array_equal(kept_tokens, np.arange(cap))
        assert np.array_equal(r["slot_row"][:cap, j], j * cap + np.arange(cap))


def check_gate_invariants():
    for k in (1, 2, 3, 5):
        x, wr, *_ = small_layer(T=50, E=5, k=k)
        logits, idx, g, _ = orc.route(x, wr, k)
        assert np.all(np.abs(g.sum(axis=1) - 1.0) <= k * 2.0 ** -52 * 4)
        if k == 1:
            assert np.all(g == 1.0)
        G = orc.dense_gates(logits, idx, g)
        mask = np.zeros_like(G, dtype=bool)
        np.put_along_axis(mask, idx.astype(np.int64), True, axis=1)
        assert np.all(G[~mask] == 0.0)
        assert np.all(g > 0)
        # gates follow the slot order (largest logit first)
        assert np.all(np.diff(g, axis=1) <= 0)


def check_k_equals_E_is_softmax():
    x, wr, *_ = small_layer(T=50, E=5)
    logits, idx, g, _ = orc.route(x, wr, 5)
    ref = torch.softmax(torch.from_numpy(logits), dim=1).numpy()
    assert np.allclose(np.take_along_axis(ref, idx.astype(np.int64), 1), g, rtol=1e-14, atol=0)


def check_printed_gates():
    u = read_golden("upcycling_top2_gates.txt")
    logits = np.array([u["logits"]])
    idx = orc.select_topk(logits, int(u["k"][0]))
    g = orc.topk_gates(logits, idx)
    assert idx[0].tolist() == [int(v) for v in u["expect_idx"]]
    assert np.allclose(g[0], u["expect_gate"], rtol=1e-12)
    s = read_golden("switch_softmax_then_top2.txt")
    logits = np.array([s["logits"]])
    E = int(s["E"][0])
    idxE = orc.select_topk(logits, E)
    gE = orc.topk_gates(logits, idxE)
    assert idxE[0, :2].tolist() == [int(v) for v in s["expect_dense_top2_idx"]]
    assert np.allclose(gE[0, :2], s["expect_dense_top2_gate"], rtol=1e-12)
    assert gE[0, :2].sum() < 1.0 - 0.3
    idx2 = orc.select_topk(logits, 2)
    assert np.allclose(orc.topk_gates(logits, idx2)[0], s["expect_top2_gate"], rtol=1e-12)


def check_capacity_values():
    assert orc.capacity(64, 4, 1, 1.25) == 20          # the tiny fp32 workload
    assert orc.capacity(8192, 32, 2, 1.25) == 640      # the OpenMoE-shaped workload
    assert orc.capacity(4096, 8, 2, 0.0) == 4096       # dropless
    assert orc.capacity(10, 3, 1, 1.0) == 4            # ceil(3.33)
    assert orc.capacity(7, 2, 1, 1.1) == 4             # ceil(3.85)
    assert orc.capacity(10, 2, 2, 4.0) == 10           # clamped to T
    assert orc.capacity(100, 64, 1, 0.01) == 1         # never below one once cf > 0


def counting_ranks(idx, E):
    """rank(t, e) = #{t' < t : e in S_t'} from the definition, via a cumulative count."""
    T, k = idx.shape
    onehot = np.zeros((T, E), dtype=np.int64)
    for j in range(k):
        onehot[np.arange(T), idx[:, j]] += 1
    before = np.cumsum(onehot, axis=0) - onehot
    return np.take_along_axis(before, idx.astype(np.int64), axis=1)


def check_permutation(idx, E, cap):
    T, k = idx.shape
    demand, offsets, slot_row, row_slot = orc.fill_in_token_order(idx, E, cap)
    rank = counting_ranks(idx, E)
    keep = rank < cap
    assert np.array_equal(slot_row >= 0, keep)
    assert np.array_equal(demand, np.bincount(idx.ravel(), minlength=E))
    kept = np.minimum(demand, cap)
    assert np.array_equal(np.diff(offsets), kept)
    assert offsets[0] == 0 and offsets[E] == keep.sum() == len(row_slot)
    assert np.all(kept <= cap)
    tt, jj = np.nonzero(keep)
    e = idx[tt, jj]
    assert np.array_equal(slot_row[tt, jj], offsets[e] + rank[tt, jj])
    # mutual inverses
    assert np.array_equal(row_slot[slot_row[tt, jj]], tt * k + jj)
    assert np.array_equal(np.sort(slot_row[keep]), np.arange(offsets[E]))
    # segments hold their expert, in token order
    tok = row_slot // k
    for ex in range(E):
        seg = row_slot[offsets[ex]:offsets[ex + 1]]
        assert np.all(idx.ravel()[seg] == ex)
        assert np.all(np.diff(tok[offsets[ex]:offsets[ex + 1]]) > 0)
    # drop-towards-the-end: once (t, e) is dropped every later (t', e) is dropped
    for ex in range(E):
        m = (idx == ex)
        kept_t = np.nonzero((m & keep).any(1))[0]
        drop_t = np.nonzero((m & ~keep).any(1))[0]
        if len(kept_t) and len(drop_t):
            assert kept_t.max() < drop_t.min()


def queue_simulation(idx, E, cap):
    """Brute force: explicit per-expert queues that refuse arrivals once full."""
    T, k = idx.shape
    queues = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            q = queues[idx[t, j]]
            if len(q) < cap:
                q.append(t)
    return queues


def check_permutation_bruteforce():
    rng = np.random.default_rng(3)
    for trial in range(40):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 13))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        for cap in range(1, T + 1):
            check_permutation(idx, E, cap)
            _, offsets, _, row_slot = orc.fill_in_token_order(idx, E, cap)
            q = queue_simulation(idx, E, cap)
            for e in range(E):
                assert (row_slot[offsets[e]:offsets[e + 1]] // k).tolist() == q[e]


def dense_reference_y(x, wr, wg, wu, wd, k, cf, storage, **kw):
    """Every expert on every token (torch, library silu), times the dense G with
    dropped slots set to 0, summed over experts. Shares only the routing
    decision (indices and gates) with the oracle; no permutation at all."""
    r = orc.forward(x, wr, wg, wu, wd, k, cf, storage, **kw)
    T, E = r["logits"].shape
    G = np.zeros((T, E))
    for j in range(k):
        kept = r["slot_row"][:, j] >= 0
        G[np.nonzero(kept)[0], r["topk_idx"][kept, j]] = r["topk_gate"][kept, j]

    def st(t):
        if storage == "f64":
            return t
        t32 = t.to(torch.float32)
        if storage == "bf16":
            t32 = t32.to(torch.bfloat16)
        return t32.to(torch.float64)

    xt = torch.from_numpy(np.asarray(x, np.float64))
    y = torch.zeros_like(xt)
    for e in range(E):
        h = st(torch.nn.functional.silu(xt @ torch.from_numpy(wg[e]).T) * (xt @ torch.from_numpy(wu[e]).T))
        o = st(h @ torch.from_numpy(wd[e]).T)
        y += torch.from_numpy(G[:, e])[:, None] * o
    return r, st(y).numpy()


def check_dense_identity():
    for case in [(40, 5, 2, 0.0, "f64", "f32"), (40, 5, 2, 1.0, "f64", "f32"),
                 (33, 4, 1, 1.25, "f64", "f32"), (40, 6, 3, 0.75, "f64", "f32"),
                 (40, 5, 2, 1.0, "bf16", "bf16"), (40, 4, 4, 0.0, "f32", "f32"),
                 (40, 5, 2, 0.75, "f64", "f32", "softmax_topk_scaled", True),
                 (40, 6, 3, 1.0, "bf16", "bf16", "softmax_topk", True)]:
        T, E, k, cf, storage, dt = case[:6]
        kw = {} if len(case) == 6 else dict(gating=case[6], bpr=case[7])
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k, dtype=dt)
        r, yd = dense_reference_y(x, wr, wg, wu, wd, k, cf, storage, **kw)
        if storage == "f64":
            assert np.allclose(r["y"], yd, rtol=1e-12, atol=1e-14)
        else:
            # same rounding points; summation order differs only in float64
            assert np.allclose(r["y"], yd, rtol=2.0 ** -7, atol=1e-12)
            assert np.mean(r["y"] == yd) > 0.99
        # fully dropped tokens give 0
        dropped = (r["slot_row"] < 0).all(axis=1)
        assert np.all(r["y"][dropped] == 0.0)


def check_identical_experts_dense_ffn():
    """Copies of one FFN with Softmax(TopK) gates reproduce the dense FFN
    (the upcycling property in the talk): the gates sum to one."""
    for (E, k) in [(4, 2), (6, 3), (4, 1), (1, 1)]:
        x, wr, wg, wu, wd = small_layer(T=30, E=E, identical=True)
        r = orc.forward(x, wr, wg, wu, wd, k, 0.0, "f64")
        xt = torch.from_numpy(x)
        dense = (torch.nn.functional.silu(xt @ torch.from_numpy(wg[0]).T)
                 * (xt @ torch.from_numpy(wu[0]).T)) @ torch.from_numpy(wd[0]).T
        # BLAS sums row blocks in its own order, so equality is to float64 rounding
        assert np.allclose(r["y"], dense.numpy(), rtol=1e-13, atol=1e-13)
        if k == 1:
            assert np.all(r["topk_gate"] == 1.0)


def check_near_tie():
    logits = np.array([[1.0, 1.0 + 5e-6, 0.0, -1.0],     # top-2 order near tie
                       [1.0, 0.5, 0.5 + 2e-6, -1.0],     # 2nd vs 3rd near tie
                       [1.0, 0.5, 0.0, -1.0],            # clear
                       [2.0, 0.5, 0.5 - 1e-4, -1.0]])    # 1e-4 apart: clear
    assert orc.near_tie_tokens(logits, 2).tolist() == [True, True, False, False]
    assert orc.near_tie_tokens(logits, 1).tolist() == [True, False, False, False]


# ---------------------------------------------------------------------------
# Switch gating (softmax over all experts, then top-k; optional E/k rescale)
# ---------------------------------------------------------------------------

def check_switch_printed_gates():
    """The talk's Switch example: softmax first over E = 8 experts, then the two
    kept probabilities are 0.4 and 0.2 (they no longer sum to one); the E/k = 4
    rescale multiplies them by 4."""
    s = read_golden("switch_softmax_then_top2.txt")
    logits = np.array([s["logits"]])
    E = int(s["E"][0])
    idx = orc.select_topk(logits, 2)
    assert idx[0].tolist() == [int(v) for v in s["expect_dense_top2_idx"]]
    g = orc.switch_gates(logits, idx, scaled=False)
    assert np.allclose(g[0], s["expect_dense_top2_gate"], rtol=1e-12)
    assert g[0].sum() < 0.61
    gs = orc.switch_gates(logits, idx, scaled=True)
    assert np.allclose(gs[0], np.array(s["expect_dense_top2_gate"]) * E / 2, rtol=1e-12)
    assert np.array_equal(orc.gates_for(logits, idx, "softmax_topk"), g)
    assert np.array_equal(orc.gates_for(logits, idx, "softmax_topk_scaled"), gs)


def check_switch_library_softmax():
    """Library routine: every Switch gate is torch.softmax over all E at the
    chosen expert; k = E gives the whole softmax; and each gate equals the
    Softmax(TopK) gate times the probability mass of the chosen set."""
    for k in (1, 2, 3, 5):
        x, wr, *_ = small_layer(T=50, E=5, k=k)
        logits, idx, g, _ = orc.route(x, wr, k, gating="softmax_topk")
        p = torch.softmax(torch.from_numpy(logits), dim=1).numpy()
        pk = np.take_along_axis(p, idx.astype(np.int64), 1)
        assert np.allclose(g, pk, rtol=1e-14, atol=0)
        assert np.allclose(orc.topk_gates(logits, idx) * pk.sum(1, keepdims=True), g, rtol=1e-13, atol=0)
        _, _, gs, _ = orc.route(x, wr, k, gating="softmax_topk_scaled")
        assert np.allclose(gs, g * 5 / k, rtol=1e-15, atol=0)
        if k == 5:
            assert np.allclose(g.sum(1), 1.0, rtol=1e-14)
        else:
            assert np.all(g.sum(1) < 1.0)


def check_switch_scaled_zero_router_is_dense():
    """The talk's claim for the E/k rescale: with copied experts the model
    behaves like the dense one. With W_g = 0 every probability is 1/E, so the
    rescaled gates are 1/k and k copies of the FFN add up to the dense FFN;
    without the rescale the output is k/E of it. For a general router the
    output is (E/k) * (kept probability mass) * FFN(x)."""
    for (E, k) in [(4, 2), (8, 2), (6, 3), (5, 5)]:
        x, wr, wg, wu, wd = small_layer(T=30, E=E, identical=True)
        xt = torch.from_numpy(x)
        dense = ((torch.nn.functional.silu(xt @ torch.from_numpy(wg[0]).T)
                  * (xt @ torch.from_numpy(wu[0]).T)) @ torch.from_numpy(wd[0]).T).numpy()
        zero = np.zeros_like(wr)
        r = orc.forward(x, zero, wg, wu, wd, k, 0.0, "f64", gating="softmax_topk_scaled")
        assert np.allclose(r["topk_gate"], 1.0 / k, rtol=1e-15, atol=0)
        assert np.allclose(r["y"], dense, rtol=1e-13, atol=1e-13)
        r = orc.forward(x, zero, wg, wu, wd, k, 0.0, "f64", gating="softmax_topk")
        assert np.allclose(r["topk_gate"], 1.0 / E, rtol=1e-15, atol=0)
        assert np.allclose(r["y"], dense * k / E, rtol=1e-13, atol=1e-13)
        r = orc.forward(x, wr, wg, wu, wd, k, 0.0, "f64", gating="softmax_topk_scaled")
        p = torch.softmax(torch.from_numpy(r["logits"]), dim=1).numpy()
        mass = np.take_along_axis(p, r["topk_idx"].astype(np.int64), 1).sum(1, keepdims=True)
        assert np.allclose(r["y"], dense * mass * E / k, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Batch Priority Routing (buffers fill in descending score order)
# ---------------------------------------------------------------------------

def bpr_sets(idx, E, cap, score):
    """Brute force from the definition, per expert and without a sequential
    fill: among the tokens that chose e, the kept ones are the cap best by
    (float32 score descending, token ascending), in that order."""
    T, k = idx.shape
    s32 = np.asarray(score, np.float64).astype(np.float32).tolist()
    out = []
    for e in range(E):
        dem = [t for t in range(T) if e in idx[t].tolist()]
        dem.sort(key=lambda t: (-s32[t], t))
        out.append(dem[:cap])
    return out


def check_bpr_bruteforce():
    rng = np.random.default_rng(5)
    for trial in range(60):
        E = int(rng.integers(1, 7))
        k = int(rng.integers(1, E + 1))
        T = int(rng.integers(1, 14))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        if trial % 2:
            score = rng.integers(0, 3, T).astype(np.float64) * 0.25   # many exact ties
        else:
            score = rng.random(T)
        for cap in range(1, T + 1):
            demand, offsets, slot_row, row_slot = orc.fill_in_priority_order(idx, E, cap, score)
            sets = bpr_sets(idx, E, cap, score)
            assert np.array_equal(demand, np.bincount(idx.ravel(), minlength=E))
            assert np.array_equal(np.diff(offsets), np.minimum(demand, cap))
            for e in range(E):
                assert (row_slot[offsets[e]:offsets[e + 1]] // k).tolist() == sets[e]
            keep = slot_row >= 0
            tt, jj = np.nonzero(keep)
            assert np.array_equal(row_slot[slot_row[tt, jj]], tt * k + jj)
            assert np.array_equal(np.sort(slot_row[keep]), np.arange(offsets[E]))


def check_bpr_reduces_to_token_order():
    """Equal scores: priority order is token order, so BPR is the vanilla fill."""
    rng = np.random.default_rng(6)
    for trial in range(20):
        E, k, T = 5, 2, 37
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        for cap in (1, 5, 9, 37):
            a = orc.fill_in_priority_order(idx, E, cap, np.full(T, 0.5))
            b = orc.fill_in_token_order(idx, E, cap)
            for u, v in zip(a, b):
                assert np.array_equal(u, v)
    # and a strictly decreasing score is token order too, an increasing one reverses it
    idx = np.zeros((6, 1), dtype=np.int32)
    _, _, sr, _ = orc.fill_in_priority_order(idx, 1, 2, np.arange(6, 0, -1))
    assert sr[:, 0].tolist() == [0, 1, -1, -1, -1, -1]
    _, _, sr, _ = orc.fill_in_priority_order(idx, 1, 2, np.arange(6))
    assert sr[:, 0].tolist() == [-1, -1, -1, -1, 1, 0]


def check_bpr_float32_decision():
    """Scores are compared as float32: two scores equal in float32 tie, and
    the tie goes to the lower token index even if the float64 values differ."""
    idx = np.zeros((3, 1), dtype=np.int32)
    score = np.array([0.5, 0.5 + 1e-12, 0.25])
    _, _, sr, _ = orc.fill_in_priority_order(idx, 1, 1, score)
    assert sr[:, 0].tolist() == [0, -1, -1]
    _, _, sr, _ = orc.fill_in_priority_order(idx, 1, 2, np.array([0.25, 0.5 + 1e-12, 0.5]))
    assert sr[:, 0].tolist() == [-1, 0, 1]


def check_bpr_forward_keeps_high_gates():
    """Forward with BPR on a capacity-bound layer: for every expert, no dropped
    assignment has a larger top-1 gate than a kept one."""
    x, wr, wg, wu, wd = small_layer(T=60, E=4, k=2)
    r = orc.forward(x, wr, wg, wu, wd, 2, 0.5, "f64", bpr=True)
    s = r["topk_gate"][:, 0].astype(np.float32)
    assert (r["slot_row"] < 0).any()
    for e in range(4):
        m = r["topk_idx"] == e
        kept = s[(m & (r["slot_row"] >= 0)).any(1)]
        drop = s[(m & (r["slot_row"] < 0)).any(1)]
        if len(kept) and len(drop):
            assert kept.min() >= drop.max()


# ---------------------------------------------------------------------------
# expert choice (each expert takes its C best tokens by softmax score)
# ---------------------------------------------------------------------------

def check_ec_bruteforce():
    rng = np.random.default_rng(8)
    for trial in range(60):
        E = int(rng.integers(1, 6))
        T = int(rng.integers(1, 12))
        if trial % 2:
            logits = rng.integers(-1, 2, (T, E)).astype(np.float64)   # many exact ties
        else:
            logits = rng.standard_normal((T, E))
        S = orc.softmax_scores(logits)
        assert np.allclose(S, torch.softmax(torch.from_numpy(logits), dim=1).numpy(), rtol=1e-14, atol=0)
        s32 = S.astype(np.float32).tolist()
        for C in range(1, T + 1):
            tok, slot = orc.expert_choice_select(S, C)
            assert tok.shape == (E, C)
            for e in range(E):
                want = sorted(sorted(range(T), key=lambda t: (-s32[t][e], t))[:C])
                assert tok[e].tolist() == want
                for i, t in enumerate(want):
                    assert slot[t, e] == e * C + i
            assert (slot >= 0).sum() == E * C
            assert np.array_equal(np.sort(slot[slot >= 0]), np.arange(E * C))


def check_ec_selects_by_score_not_logit():
    """Token A has logits (5, 5), token B (1, -5). Expert 0 with C = 1 takes B:
    its score 1/(1+e^-6) = 0.9975 beats A's 0.5, although A's logit is larger;
    expert 1 takes A (0.5 against B's 0.0025)."""
    logits = np.array([[5.0, 5.0], [1.0, -5.0]])
    S = orc.softmax_scores(logits)
    assert abs(S[1, 0] - 1.0 / (1.0 + math.exp(-6.0))) < 1e-15 and S[0, 0] == 0.5
    tok, slot = orc.expert_choice_select(S, 1)
    assert tok[:, 0].tolist() == [1, 0]
    assert slot.tolist() == [[-1, 1], [0, -1]]


def check_ec_full_capacity_is_dense_gating():
    """C = T (cf = 0): every expert takes every token, so the layer is the dense
    softmax-gated mixture of [MATH]: y = sum_e Softmax(x.W_g)_e FFN_e(x),
    evaluated densely with torch (library softmax and silu)."""
    for (E, k) in [(4, 2), (3, 1), (5, 5)]:
        x, wr, wg, wu, wd = small_layer(T=25, E=E)
        r = orc.expert_choice_forward(x, wr, wg, wu, wd, k, 0.0, "f64")
        assert r["cap"] == 25
        xt = torch.from_numpy(x)
        G = torch.softmax(xt @ torch.from_numpy(wr).T, dim=1)
        y = torch.zeros_like(xt)
        for e in range(E):
            h = torch.nn.functional.silu(xt @ torch.from_numpy(wg[e]).T) * (xt @ torch.from_numpy(wu[e]).T)
            y += G[:, e:e + 1] * (h @ torch.from_numpy(wd[e]).T)
        assert np.allclose(r["y"], y.numpy(), rtol=1e-12, atol=1e-13)


def check_ec_zero_router():
    """W_g = 0: every score is 1/E, so every expert takes tokens 0..C-1; with
    copied experts those tokens get exactly the dense FFN (E gates of 1/E) and
    the others 0."""
    T, E, k, cf = 30, 4, 2, 0.5
    x, _, wg, wu, wd = small_layer(T=T, E=E, identical=True)
    wr = np.zeros((E, x.shape[1]))
    r = orc.expert_choice_forward(x, wr, wg, wu, wd, k, cf, "f64")
    C = r["cap"]
    assert C == math.ceil(cf * T * k / E) == 8
    assert np.array_equal(r["tokens"], np.tile(np.arange(C), (E, 1)))
    xt = torch.from_numpy(x)
    dense = ((torch.nn.functional.silu(xt @ torch.from_numpy(wg[0]).T) * (xt @ torch.from_numpy(wu[0]).T))
             @ torch.from_numpy(wd[0]).T).numpy()
    assert np.allclose(r["y"][:C], dense[:C], rtol=1e-13, atol=1e-13)
    assert np.all(r["y"][C:] == 0.0)


def check_ec_partial_capacity_dense_eval():
    """C < T: experts take different numbers of each token, so tokens get
    zero, one or several experts ([TALK] expert-choice Q&A). The layer must be
    y[t] = sum over the experts e that chose t of Softmax(x.W_g)[t, e] *
    FFN_e(x_t): the dense score, not renormalised over the choosing experts.
    The selection here is a brute-force column sort (float32 scores, lower
    token first) and the experts run densely in torch (library softmax, silu)."""
    for (T, E, k, cf, seed) in [(30, 5, 2, 0.5, 11), (24, 4, 1, 1.0, 12), (40, 6, 3, 0.3, 13)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, seed=seed)
        wr = wr * 3.0                      # sharper scores: choosers differ a lot between tokens
        r = orc.expert_choice_forward(x, wr, wg, wu, wd, k, cf, "f64")
        C = r["cap"]
        assert C == math.ceil(float(np.float32(cf)) * T * k / E) < T
        xt = torch.from_numpy(x)
        S = torch.softmax(xt @ torch.from_numpy(wr).T, dim=1)
        s32 = S.to(torch.float32).tolist()
        chosen = np.zeros((T, E), dtype=bool)
        for e in range(E):
            best = sorted(range(T), key=lambda t: (-s32[t][e], t))[:C]
            chosen[best, e] = True
        per_token = chosen.sum(axis=1)
        assert (per_token == 0).any() and (per_token == 1).any() and (per_token >= 2).any(), per_token
        y = torch.zeros_like(xt)
        for e in range(E):
            h = torch.nn.functional.silu(xt @ torch.from_numpy(wg[e]).T) * (xt @ torch.from_numpy(wu[e]).T)
            w = S[:, e:e + 1] * torch.from_numpy(chosen[:, e:e + 1].astype(np.float64))
            y += w * (h @ torch.from_numpy(wd[e]).T)
        assert np.allclose(r["y"], y.numpy(), rtol=1e-12, atol=1e-13)
        assert np.all(r["y"][per_token == 0] == 0.0)


def check_ec_float32_decision():
    """Scores equal in float32 tie (lower token wins) even if float64 differs."""
    S = np.array([[0.5, 0.5], [0.5 + 1e-12, 0.5 - 1e-12], [0.25, 0.75]])
    tok, _ = orc.expert_choice_select(S, 1)
    assert tok[:, 0].tolist() == [0, 2]


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------

def _loss(x, wr, wg, wu, wd, dy, k, cf, gating="topk_softmax", bpr=False):
    return float((orc.forward(x, wr, wg, wu, wd, k, cf, "f64", gating=gating, bpr=bpr)["y"] * dy).sum())


def _fd_check(x, wr, wg, wu, wd, dy, k, cf, gating="topk_softmax", bpr=False, eps=1e-6):
    """Every gradient entry against a central difference of L = <dy, y>; the
    routing, the drops and (with bpr) the fill order must not move under the
    step, which the caller's inputs make sure of and this checks."""
    g = orc.backward(x, wr, wg, wu, wd, dy, k, cf, "f64", gating=gating, bpr=bpr)
    base = g["forward"]["slot_row"]
    params = {"dx": x, "dW_g": wr, "dW_gate": wg, "dW_up": wu, "dW_down": wd}
    for name, arr in params.items():
        flat = arr.reshape(-1)
        num = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            vals = []
            for sgn in (1, -1):
                flat[i] = keep + sgn * eps
                vals.append(_loss(x, wr, wg, wu, wd, dy, k, cf, gating, bpr))
            flat[i] = keep
            num[i] = (vals[0] - vals[1]) / (2 * eps)
        assert np.allclose(g[name].reshape(-1), num, rtol=1e-6, atol=1e-7), (name, gating, bpr)
    again = orc.forward(x, wr, wg, wu, wd, k, cf, "f64", gating=gating, bpr=bpr)
    assert np.array_equal(again["slot_row"], base)
    return g


def check_backward_finite_differences():
    """Every gradient entry of a tiny layer (with and without drops) against a
    central difference of L = <dy, y> through the forward oracle (float64, no
    rounding). The step is far below every routing gap, so the routing and the
    drops stay fixed."""
    for (T, d, E, k, F, cf, seed) in [(12, 6, 4, 2, 5, 0.75, 1), (9, 4, 3, 3, 4, 0.0, 2), (10, 5, 4, 1, 6, 0.5, 3)]:
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((T, d))
        wr = rng.standard_normal((E, d))
        wg = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wu = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wd = rng.standard_normal((E, d, F)) / math.sqrt(F)
        dy = rng.standard_normal((T, d))
        g = orc.backward(x, wr, wg, wu, wd, dy, k, cf, "f64")
        if cf > 0:
            assert (g["forward"]["slot_row"] < 0).any()
        params = {"dx": x, "dW_g": wr, "dW_gate": wg, "dW_up": wu, "dW_down": wd}
        eps = 1e-6
        for name, arr in params.items():
            flat = arr.reshape(-1)
            num = np.empty(flat.size)
            for i in range(flat.size):
                keep = flat[i]
                flat[i] = keep + eps
                lp = _loss(x, wr, wg, wu, wd, dy, k, cf)
                flat[i] = keep - eps
                lm = _loss(x, wr, wg, wu, wd, dy, k, cf)
                flat[i] = keep
                num[i] = (lp - lm) / (2 * eps)
            assert np.allclose(g[name].reshape(-1), num, rtol=1e-6, atol=1e-7), name


def check_backward_gating_finite_differences():
    """The Switch gate rules (every logit gets gradient through the softmax
    over all experts; rescaled by E/k or not) and Batch Priority Routing
    (fill order by the top-1 gate: a discrete decision, no gradient), each on
    tiny layers with capacity drops, against central differences."""
    for (T, d, E, k, F, cf, seed, gating, bpr) in [
            (12, 6, 4, 2, 5, 0.75, 31, "softmax_topk", False),
            (10, 5, 4, 1, 6, 0.5, 32, "softmax_topk_scaled", False),
            (12, 6, 5, 2, 5, 0.6, 33, "topk_softmax", True),
            (11, 5, 4, 2, 4, 0.75, 34, "softmax_topk_scaled", True)]:
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((T, d))
        wr = rng.standard_normal((E, d))
        wg = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wu = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wd = rng.standard_normal((E, d, F)) / math.sqrt(F)
        dy = rng.standard_normal((T, d))
        g = _fd_check(x, wr, wg, wu, wd, dy, k, cf, gating, bpr)
        assert (g["forward"]["slot_row"] < 0).any()
        if gating != "topk_softmax":
            # under the Switch rules every logit of a token with a kept slot gets gradient,
            # chosen or not; a token with every slot dropped gets none
            live = (g["forward"]["slot_row"] >= 0).any(axis=1)
            assert np.all(np.abs(g["dl_dense"][live]) > 0) and np.all(g["dl_dense"][~live] == 0)


def check_backward_gating_autograd():
    """torch autograd through a dense evaluation with the oracle's routing,
    fill and drops held fixed, for the Switch rules and Batch Priority
    Routing (gates s * softmax(l)[S_j] from the library softmax)."""
    for (T, E, k, cf, gating, bpr) in [(30, 5, 2, 0.75, "softmax_topk", False), (25, 4, 1, 0.5, "softmax_topk_scaled", True),
                                       (28, 6, 3, 0.8, "topk_softmax", True)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k)
        dy = np.random.default_rng(7).standard_normal(x.shape)
        g = orc.backward(x, wr, wg, wu, wd, dy, k, cf, "f64", gating=gating, bpr=bpr)
        fw = g["forward"]
        idx = torch.from_numpy(fw["topk_idx"].astype(np.int64))
        kept = torch.from_numpy(fw["slot_row"] >= 0)
        tx, twr, twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (x, wr, wg, wu, wd))
        l = tx @ twr.T
        if gating == "topk_softmax":
            gate = torch.softmax(torch.gather(l, 1, idx), dim=1)
        else:
            gate = torch.gather(torch.softmax(l, dim=1), 1, idx) * (E / k if gating.endswith("scaled") else 1.0)
        y = torch.zeros_like(tx)
        for e in range(E):
            h = torch.nn.functional.silu(tx @ twg[e].T) * (tx @ twu[e].T)
            w = ((idx == e) & kept).double() * gate
            y = y + w.sum(1, keepdim=True) * (h @ twd[e].T)
        (y * torch.from_numpy(dy)).sum().backward()
        for name, t in [("dx", tx), ("dW_g", twr), ("dW_gate", twg), ("dW_up", twu), ("dW_down", twd)]:
            assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), (name, gating, bpr)


def check_backward_autograd():
    """torch.autograd through a dense evaluation with the oracle's routing and
    drop decisions held fixed (every expert on every token, masked by the
    kept slots; gates = softmax of the chosen logits): the same five gradients."""
    for (T, E, k, cf) in [(30, 5, 2, 0.75), (25, 4, 1, 0.0), (20, 6, 3, 1.0)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k)
        dy = np.random.default_rng(4).standard_normal(x.shape)
        g = orc.backward(x, wr, wg, wu, wd, dy, k, cf, "f64")
        fw = g["forward"]
        idx = torch.from_numpy(fw["topk_idx"].astype(np.int64))
        kept = torch.from_numpy(fw["slot_row"] >= 0)
        tx, twr, twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (x, wr, wg, wu, wd))
        l = tx @ twr.T
        gate = torch.softmax(torch.gather(l, 1, idx), dim=1)
        y = torch.zeros_like(tx)
        for e in range(E):
            h = torch.nn.functional.silu(tx @ twg[e].T) * (tx @ twu[e].T)
            oe = h @ twd[e].T
            w = ((idx == e) & kept).double() * gate
            y = y + w.sum(1, keepdim=True) * oe
        (y * torch.from_numpy(dy)).sum().backward()
        for name, t in [("dx", tx), ("dW_g", twr), ("dW_gate", twg), ("dW_up", twu), ("dW_down", twd)]:
            assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), name


def check_backward_storage_rounding():
    """bf16 storage: the returned gradients are bf16 values, and they match the
    float64 gradients to bf16 precision (the rounding points only perturb)."""
    x, wr, wg, wu, wd = small_layer(T=30, E=4, k=2, dtype="bf16")
    dy = torch.from_numpy(np.random.default_rng(5).standard_normal(x.shape)).to(torch.bfloat16).double().numpy()
    gb = orc.backward(x, wr, wg, wu, wd, dy, 2, 1.0, "bf16")
    g64 = orc.backward(x, wr, wg, wu, wd, dy, 2, 1.0, "f64")
    for name in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
        v = gb[name]
        assert np.array_equal(orc.round_to_bf16(v.astype(np.float32)).astype(np.float64), v), name
        scale = np.abs(g64[name]).max()
        assert np.abs(v - g64[name]).max() <= 0.05 * scale, name


def bf16_ordinal(v):
    """Signed position of each bf16 value on the bf16 number line (0 for both
    zeros), so that adjacent bf16 values differ by 1."""
    b = (np.asarray(v, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_bf16_close(mine, ref, what, min_equal=0.99):
    """Both sides hold bf16 values; they differ by at most one bf16 step, and
    at least `min_equal` of them are identical (the two sides round the same
    float64 values, which differ only by float64 summation order)."""
    mine = np.asarray(mine, np.float64)
    ref = np.asarray(ref, np.float64)
    as_bf16 = lambda a: torch.from_numpy(a).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(as_bf16(mine), mine), f"{what}: oracle value is not a bf16 value"
    assert np.array_equal(as_bf16(ref), ref), f"{what}: reference value is not a bf16 value"
    steps = np.abs(bf16_ordinal(mine) - bf16_ordinal(ref))
    assert steps.max(initial=0) <= 1, f"{what}: {int(steps.max())} bf16 steps apart"
    eq = float((steps == 0).mean()) if steps.size else 1.0
    assert eq >= min_equal, f"{what}: only {eq:.4f} identical"


def torch_backward_bf16(x, wr, wg, wu, wd, dy, k, cf, gating="topk_softmax", bpr=False):
    """The backward pass of a bf16 layer, evaluated slot by slot in torch
    float64, rounding to bf16 (torch's float32 -> bfloat16 conversion) at the
    points where the layer holds a value in its storage type: a and b as the
    SwiGLU backward reads them, h and o (recomputed as the forward stores
    them), d_o = g*dy, da, db, dx_perm, and each returned gradient. The
    derivatives of silu and of the softmax over the chosen logits come from
    torch autograd, the routing from a stable torch sort and counting ranks."""
    bf = lambda v: v.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    X, WR, WG, WU, WD, DY = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wr, wg, wu, wd, dy))
    T, d = X.shape
    E, F = WG.shape[0], WG.shape[1]
    l = X @ WR.T
    idx = torch.sort(l.to(torch.float32), dim=1, descending=True, stable=True).indices[:, :k]
    if gating == "topk_softmax":
        lS = torch.gather(l, 1, idx).detach().requires_grad_(True)
        g = torch.softmax(lS, dim=1)
    else:
        lS = l.detach().clone().requires_grad_(True)
        g = torch.gather(torch.softmax(lS, dim=1), 1, idx) * (E / k if gating.endswith("scaled") else 1.0)
    cap = T if np.float32(cf) == 0 else min(T, math.ceil(float(np.float32(cf)) * T * k / E))
    # arrival order: token order, or (BPR) by descending float32 top-1 gate, ties by token
    order = (torch.sort(-g.detach()[:, 0].to(torch.float32), stable=True).indices if bpr
             else torch.arange(T))
    onehot = torch.zeros((T, E), dtype=torch.int64)
    onehot.scatter_(1, idx, 1)
    oh = onehot[order]
    before_in_order = torch.cumsum(oh, 0) - oh
    before = torch.empty_like(before_in_order)
    before[order] = before_in_order
    rank = torch.gather(before, 1, idx)
    kept = rank < cap
    gd = g.detach()
    out = {n: {} for n in ("a", "b", "h", "o", "d_o", "da", "db", "dx_perm")}
    dg = torch.zeros((T, k), dtype=torch.float64)
    dWgate = torch.zeros_like(WG)
    dWup = torch.zeros_like(WU)
    dWdown = torch.zeros_like(WD)
    dx = torch.zeros_like(X)
    for t in range(T):
        for j in range(k):
            if not bool(kept[t, j]):
                continue
            e = int(idx[t, j])
            a = WG[e] @ X[t]
            b = WU[e] @ X[t]
            h = bf(torch.nn.functional.silu(a) * b)
            o = bf(WD[e] @ h)
            d_o = bf(gd[t, j] * DY[t])
            dg[t, j] = torch.dot(DY[t], o)
            dh = WD[e].T @ d_o
            a_st, b_st = bf(a), bf(b)
            a_req = a_st.clone().requires_grad_(True)
            s = torch.nn.functional.silu(a_req)
            s.sum().backward()
            da = bf(dh * b_st * a_req.grad)
            db = bf(dh * s.detach())
            dxp = bf(WG[e].T @ da + WU[e].T @ db)
            dWgate[e] += torch.outer(da, X[t])
            dWup[e] += torch.outer(db, X[t])
            dWdown[e] += torch.outer(d_o, h)
            dx[t] += dxp
            for n, v in (("a", a_st), ("b", b_st), ("h", h), ("o", o), ("d_o", d_o), ("da", da), ("db", db),
                         ("dx_perm", dxp)):
                out[n][(t, j)] = v.numpy()
    g.backward(dg)
    dl = torch.zeros((T, E), dtype=torch.float64)
    if gating == "topk_softmax":
        dl.scatter_(1, idx, lS.grad)
    else:
        dl = lS.grad
    dWg = dl.T @ X
    dx += dl @ WR
    res = dict(dx=bf(dx).numpy(), dW_g=bf(dWg).numpy(), dW_gate=bf(dWgate).numpy(), dW_up=bf(dWup).numpy(),
               dW_down=bf(dWdown).numpy(), dl=dl.numpy(), idx=idx.numpy(), kept=kept.numpy(),
               rank=rank.numpy())
    res.update(out)
    return res


def check_backward_rounding_points_bf16():
    """The bf16 backward's rounding points, pinned by an independent slot-by-slot
    torch evaluation (torch_backward_bf16): every intermediate the oracle holds
    (a, b, h, o, d_o, da, db, dx_perm) and every returned gradient are bf16
    values within one bf16 step of torch's, and almost all identical. With a
    rounding point left out, the intermediate is no bf16 value, or the
    gradients drift by more than rounding-order noise."""
    for (T, E, k, cf, seed, gating, bpr) in [(24, 4, 2, 0.75, 21, "topk_softmax", False),
                                             (16, 3, 1, 0.0, 22, "topk_softmax", False),
                                             (20, 5, 3, 1.0, 23, "topk_softmax", False),
                                             (24, 4, 2, 0.75, 24, "softmax_topk_scaled", True),
                                             (20, 5, 2, 0.6, 25, "softmax_topk", False)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k, seed=seed, dtype="bf16")
        dy = torch.from_numpy(np.random.default_rng(seed).standard_normal(x.shape)).to(torch.bfloat16).double().numpy()
        g = orc.backward(x, wr, wg, wu, wd, dy, k, cf, "bf16", gating=gating, bpr=bpr)
        ref = torch_backward_bf16(x, wr, wg, wu, wd, dy, k, cf, gating, bpr)
        fw = g["forward"]
        assert np.array_equal(fw["topk_idx"], ref["idx"])
        assert np.array_equal(fw["slot_row"] >= 0, ref["kept"])
        if cf > 0 and k > 1:
            assert (~ref["kept"]).any()          # the case has drops
        slots = sorted(ref["a"])
        rows = np.array([fw["slot_row"][t, j] for (t, j) in slots])
        for name in ("a", "b", "h", "o", "d_o", "da", "db", "dx_perm"):
            mine = {"a": g["a_st"], "b": g["b_st"]}.get(name, g.get(name))
            assert_bf16_close(mine[rows], np.stack([ref[name][s] for s in slots]), name)
        assert np.allclose(g["dl_dense"], ref["dl"], rtol=1e-9, atol=1e-12)
        for name in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
            assert_bf16_close(g[name], ref[name], name)


def check_backward_expert_subset_and_sub_batch():
    """The identities the full-size GPU test relies on. (1) Asking for some
    experts' weight gradients returns exactly theirs. (2) A token's routing,
    gates and rows depend on that token alone (only whether a slot is kept
    depends on the tokens before it), so a drop-free backward over a sub-batch
    gives the same dx for tokens that kept every slot, and one over the tokens
    an expert kept gives that expert's weight gradients."""
    x, wr, wg, wu, wd = small_layer(T=40, E=4, k=2, dtype="bf16")
    dy = torch.from_numpy(np.random.default_rng(6).standard_normal(x.shape)).to(torch.bfloat16).double().numpy()
    full = orc.backward(x, wr, wg, wu, wd, dy, 2, 0.0, "bf16")
    part = orc.backward(x, wr, wg, wu, wd, dy, 2, 0.0, "bf16", weight_grad_experts=[3, 1])
    for name in ("dW_gate", "dW_up", "dW_down"):
        assert np.array_equal(part[name], full[name][[3, 1]]), name
    assert np.array_equal(part["dx"], full["dx"]) and np.array_equal(part["dW_g"], full["dW_g"])
    toks = np.array([0, 7, 21, 39])
    sub = orc.backward(x[toks], wr, wg, wu, wd, dy[toks], 2, 0.0, "bf16", weight_grad_experts=[])
    assert np.array_equal(sub["dx"], full["dx"][toks])
    idx = full["forward"]["topk_idx"]
    te = np.nonzero((idx == 2).any(axis=1))[0]
    sub = orc.backward(x[te], wr, wg, wu, wd, dy[te], 2, 0.0, "bf16", weight_grad_experts=[2])
    for name in ("dW_gate", "dW_up", "dW_down"):
        assert np.allclose(sub[name][0], full[name][2], rtol=0, atol=1e-12 * np.abs(full[name][2]).max()), name
    # With capacity drops: a token none of whose slots was dropped has the same
    # dx as in a drop-free backward over it alone, and expert e's weight
    # gradients are those of a drop-free backward over the tokens it kept.
    cf = 0.6
    full = orc.backward(x, wr, wg, wu, wd, dy, 2, cf, "bf16")
    srow, idx = full["forward"]["slot_row"], full["forward"]["topk_idx"]
    kept_all = np.nonzero((srow >= 0).all(axis=1))[0]
    assert 0 < len(kept_all) < len(x)
    sub = orc.backward(x[kept_all], wr, wg, wu, wd, dy[kept_all], 2, 0.0, "bf16", weight_grad_experts=[])
    assert np.array_equal(sub["dx"], full["dx"][kept_all])
    for e in range(4):
        te = np.nonzero(((idx == e) & (srow >= 0)).any(axis=1))[0]
        sub = orc.backward(x[te], wr, wg, wu, wd, dy[te], 2, 0.0, "bf16", weight_grad_experts=[e])
        for name in ("dW_gate", "dW_up", "dW_down"):
            scale = max(np.abs(full[name][e]).max(), 1e-300)
            assert np.allclose(sub[name][0], full[name][e], rtol=0, atol=1e-12 * scale), (name, e)


def _ec_loss(x, wr, wg, wu, wd, dy, k, cf):
    return float((orc.expert_choice_forward(x, wr, wg, wu, wd, k, cf, "f64")["y"] * dy).sum())


def check_ec_backward_finite_differences():
    """Expert choice: every gradient entry of tiny layers (experts taking part
    of the tokens, and all of them) against a central difference of
    L = <dy, y> through the forward oracle (float64). The step is far below
    every score gap at an expert's C-th place, so the selection stays fixed,
    which this checks."""
    for (T, d, E, k, F, cf, seed) in [(10, 4, 3, 1, 4, 0.5, 41), (8, 5, 4, 2, 3, 0.0, 42), (12, 4, 3, 2, 5, 0.6, 43)]:
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((T, d))
        wr = rng.standard_normal((E, d))
        wg = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wu = rng.standard_normal((E, F, d)) / math.sqrt(d)
        wd = rng.standard_normal((E, d, F)) / math.sqrt(F)
        dy = rng.standard_normal((T, d))
        g = orc.expert_choice_backward(x, wr, wg, wu, wd, dy, k, cf, "f64")
        base = g["forward"]["slot"]
        if cf > 0:
            assert (base < 0).any()
        params = {"dx": x, "dW_g": wr, "dW_gate": wg, "dW_up": wu, "dW_down": wd}
        eps = 1e-6
        for name, arr in params.items():
            flat = arr.reshape(-1)
            num = np.empty(flat.size)
            for i in range(flat.size):
                keep = flat[i]
                flat[i] = keep + eps
                lp = _ec_loss(x, wr, wg, wu, wd, dy, k, cf)
                flat[i] = keep - eps
                lm = _ec_loss(x, wr, wg, wu, wd, dy, k, cf)
                flat[i] = keep
                num[i] = (lp - lm) / (2 * eps)
            assert np.allclose(g[name].reshape(-1), num, rtol=1e-6, atol=1e-7), (name, T, E, cf)
        assert np.array_equal(orc.expert_choice_forward(x, wr, wg, wu, wd, k, cf, "f64")["slot"], base)


def check_ec_backward_autograd():
    """Expert choice: torch autograd through a dense evaluation (every expert
    on every token, masked by the oracle's selection, gates from torch's
    softmax over all experts) gives the same five gradients. The cases give
    tokens no expert, one expert and several experts."""
    for (T, E, k, cf, seed) in [(30, 5, 2, 0.6, 44), (24, 4, 1, 0.0, 45), (20, 6, 3, 0.4, 46)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k, seed=seed)
        dy = np.random.default_rng(seed).standard_normal(x.shape)
        g = orc.expert_choice_backward(x, wr, wg, wu, wd, dy, k, cf, "f64")
        chosen = g["forward"]["slot"] >= 0
        per_token = chosen.sum(axis=1)
        if cf > 0:
            assert (per_token == 0).any() and (per_token == 1).any() and (per_token >= 2).any()
        mask = torch.from_numpy(chosen).double()
        tx, twr, twg, twu, twd = (torch.tensor(a, requires_grad=True) for a in (x, wr, wg, wu, wd))
        S = torch.softmax(tx @ twr.T, dim=1)
        y = torch.zeros_like(tx)
        for e in range(E):
            h = torch.nn.functional.silu(tx @ twg[e].T) * (tx @ twu[e].T)
            y = y + (mask[:, e] * S[:, e])[:, None] * (h @ twd[e].T)
        (y * torch.from_numpy(dy)).sum().backward()
        for name, t in [("dx", tx), ("dW_g", twr), ("dW_gate", twg), ("dW_up", twu), ("dW_down", twd)]:
            assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), (name, cf)


def check_ec_backward_full_capacity_is_switch_backward():
    """With C = T every expert takes every token, so the expert-choice layer is
    the dense-gated layer: the token-choice layer with k = E under the Switch
    rule without rescale (gates p[e], nothing dropped). Their gradients agree
    (they differ only in row order, hence summation order)."""
    x, wr, wg, wu, wd = small_layer(T=18, E=4, k=2, seed=47)
    dy = np.random.default_rng(47).standard_normal(x.shape)
    ec = orc.expert_choice_backward(x, wr, wg, wu, wd, dy, 2, 0.0, "f64")
    tc = orc.backward(x, wr, wg, wu, wd, dy, 4, 0.0, "f64", gating="softmax_topk")
    assert (ec["forward"]["slot"] >= 0).all()
    for name in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
        assert np.allclose(ec[name], tc[name], rtol=1e-12, atol=1e-13), name


def torch_ec_backward_bf16(x, wr, wg, wu, wd, dy, k, cf):
    """The expert-choice backward of a bf16 layer, evaluated pair by pair in
    torch float64 and rounded to bf16 where the layer holds a value in its
    storage type (as torch_backward_bf16). The selection (each expert's C
    largest float32 scores, ties to the lower token) comes from a stable torch
    sort, the softmax's derivative from torch autograd."""
    bf = lambda v: v.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    X, WR, WG, WU, WD, DY = (torch.from_numpy(np.asarray(a, np.float64)) for a in (x, wr, wg, wu, wd, dy))
    T, d = X.shape
    E = WG.shape[0]
    lS = (X @ WR.T).detach().requires_grad_(True)
    S = torch.softmax(lS, dim=1)
    C = T if np.float32(cf) == 0 else min(T, math.ceil(float(np.float32(cf)) * T * k / E))
    chosen = torch.zeros((T, E), dtype=torch.bool)
    for e in range(E):
        chosen[torch.sort(-S.detach()[:, e].to(torch.float32), stable=True).indices[:C], e] = True
    out = {n: {} for n in ("a", "b", "h", "o", "d_o", "da", "db", "dx_perm")}
    dS = torch.zeros((T, E), dtype=torch.float64)
    dWgate = torch.zeros_like(WG)
    dWup = torch.zeros_like(WU)
    dWdown = torch.zeros_like(WD)
    dx = torch.zeros_like(X)
    for t in range(T):
        for e in range(E):
            if not bool(chosen[t, e]):
                continue
            a = WG[e] @ X[t]
            b = WU[e] @ X[t]
            h = bf(torch.nn.functional.silu(a) * b)
            o = bf(WD[e] @ h)
            d_o = bf(S.detach()[t, e] * DY[t])
            dS[t, e] = torch.dot(DY[t], o)
            dh = WD[e].T @ d_o
            a_st, b_st = bf(a), bf(b)
            a_req = a_st.clone().requires_grad_(True)
            s = torch.nn.functional.silu(a_req)
            s.sum().backward()
            da = bf(dh * b_st * a_req.grad)
            db = bf(dh * s.detach())
            dxp = bf(WG[e].T @ da + WU[e].T @ db)
            dWgate[e] += torch.outer(da, X[t])
            dWup[e] += torch.outer(db, X[t])
            dWdown[e] += torch.outer(d_o, h)
            dx[t] += dxp
            for n, v in (("a", a_st), ("b", b_st), ("h", h), ("o", o), ("d_o", d_o), ("da", da), ("db", db),
                         ("dx_perm", dxp)):
                out[n][(t, e)] = v.numpy()
    S.backward(dS)
    dl = lS.grad
    dx += dl @ WR
    res = dict(dx=bf(dx).numpy(), dW_g=bf(dl.T @ X).numpy(), dW_gate=bf(dWgate).numpy(),
               dW_up=bf(dWup).numpy(), dW_down=bf(dWdown).numpy(), dl=dl.numpy(), chosen=chosen.numpy())
    res.update(out)
    return res


def check_ec_backward_rounding_points_bf16():
    """The bf16 expert-choice backward's rounding points, pinned by the
    independent pair-by-pair torch evaluation: every held intermediate and
    every returned gradient within one bf16 step of torch's, almost all
    identical."""
    for (T, E, k, cf, seed) in [(24, 4, 2, 0.5, 48), (16, 3, 1, 0.0, 49), (20, 5, 2, 0.8, 50)]:
        x, wr, wg, wu, wd = small_layer(T=T, E=E, k=k, seed=seed, dtype="bf16")
        dy = torch.from_numpy(np.random.default_rng(seed).standard_normal(x.shape)).to(torch.bfloat16).double().numpy()
        g = orc.expert_choice_backward(x, wr, wg, wu, wd, dy, k, cf, "bf16")
        ref = torch_ec_backward_bf16(x, wr, wg, wu, wd, dy, k, cf)
        slot = g["forward"]["slot"]
        assert np.array_equal(slot >= 0, ref["chosen"])
        pairs = sorted(ref["a"])
        rows = np.array([slot[t, e] for (t, e) in pairs])
        for name in ("a", "b", "h", "o", "d_o", "da", "db", "dx_perm"):
            mine = {"a": g["a_st"], "b": g["b_st"]}.get(name, g.get(name))
            assert_bf16_close(mine[rows], np.stack([ref[name][p] for p in pairs]), name)
        assert np.allclose(g["dl"], ref["dl"], rtol=1e-9, atol=1e-12)
        for name in ("dx", "dW_g", "dW_gate", "dW_up", "dW_down"):
            assert_bf16_close(g[name], ref[name], name)


ALL_PINS = [check_bf16_rounding, check_silu_library, check_topk_bruteforce,
            check_zero_router_closed_form, check_gate_invariants, check_k_equals_E_is_softmax,
            check_printed_gates, check_capacity_values, check_permutation_bruteforce,
            check_dense_identity, check_identical_experts_dense_ffn, check_near_tie,
            check_switch_printed_gates, check_switch_library_softmax,
            check_switch_scaled_zero_router_is_dense, check_bpr_bruteforce,
            check_bpr_reduces_to_token_order, check_bpr_float32_decision,
            check_bpr_forward_keeps_high_gates, check_ec_bruteforce, check_ec_selects_by_score_not_logit,
            check_ec_full_capacity_is_dense_gating, check_ec_zero_router, check_ec_float32_decision,
            check_ec_partial_capacity_dense_eval,
            check_backward_finite_differences, check_backward_autograd, check_backward_storage_rounding,
            check_backward_rounding_points_bf16, check_backward_gating_finite_differences,
            check_backward_gating_autograd,
            check_backward_expert_subset_and_sub_batch,
            check_ec_backward_finite_differences, check_ec_backward_autograd,
            check_ec_backward_full_capacity_is_switch_backward, check_ec_backward_rounding_points_bf16]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_permutation_random_mid():
    rng = np.random.default_rng(11)
    for (T, E, k) in [(500, 8, 2), (300, 64, 8), (257, 3, 3)]:
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        for cap in (1, 7, T * k // E, T):
            check_permutation(idx, E, cap)


def test_skewed_workload_drops_towards_the_end():
    """The Zipf token-id workload: capacity 640, imbalanced demand, and the
    drops fall in the later part of the sequence (Drop-towards-the-End)."""
    w = mi.WORKLOADS["openmoe_bf16"]
    a = mi.generate(w, expert_weights=False)
    logits, idx, g, tie = orc.route(a["x"], a["w_router"], w.k)
    cap = orc.capacity(w.T, w.E, w.k, w.cf)
    assert cap == 640
    demand, offsets, slot_row, row_slot = orc.fill_in_token_order(idx, w.E, cap)
    assert demand.max() > cap                   # imbalanced: some expert overflows
    dropped = slot_row < 0
    n_drop = int(dropped.sum())
    assert 0 < n_drop < w.T * w.k // 4
    drop_tokens = np.nonzero(dropped.any(1))[0]
    assert np.median(drop_tokens) > w.T * 0.6
    assert drop_tokens.min() > w.T // 4


def test_workload_shapes_and_seeds():
    w = mi.WORKLOADS["tiny_fp32"]
    a = mi.generate(w)
    b = mi.generate(w)
    for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
        assert torch.equal(a[key], b[key])
    assert a["x"].shape == (64, 64) and a["w_gate"].shape == (4, 128, 64)
    assert a["w_down"].shape == (4, 64, 128)
    # scale: weights ~ N(0, 1/d)
    assert abs(a["w_gate"].double().std().item() * math.sqrt(64) - 1.0) < 0.05


# ---------------------------------------------------------------------------
# planted mistakes: each must make some pin fail
# ---------------------------------------------------------------------------

def _swap_gate_up(xr, w_gate_e, w_up_e, w_down_e, storage, _orig=orc.swiglu_expert):
    return _orig(xr, w_up_e, w_gate_e, w_down_e, storage)


MUTANTS = {
    "topk_smallest": ("select_topk", lambda logits, k: np.argsort(np.asarray(logits, np.float32), axis=1, kind="stable")[:, :k].astype(np.int32),
                      [check_topk_bruteforce]),
    "ties_to_higher_index": ("select_topk", lambda logits, k: (logits.shape[1] - 1 - np.argsort(-np.asarray(logits, np.float32)[:, ::-1], axis=1, kind="stable"))[:, :k].astype(np.int32),
                             [check_zero_router_closed_form]),
    "softmax_then_topk": ("topk_gates", lambda logits, idx: np.take_along_axis(
        np.exp(logits - logits.max(1, keepdims=True)) / np.exp(logits - logits.max(1, keepdims=True)).sum(1, keepdims=True),
        idx.astype(np.int64), 1), [check_gate_invariants]),
    "capacity_floor": ("capacity", lambda T, E, k, cf: T if cf == 0 else int(min(T, math.floor(cf * T * k / E))),
                       [check_capacity_values]),
    "silu_sign": ("silu", lambda a: a / (1.0 + np.exp(a)), [check_silu_library, check_identical_experts_dense_ffn]),
    "gate_up_swapped": ("swiglu_expert", _swap_gate_up, [check_dense_identity]),
    "combine_ignores_gates": ("combine", lambda o_rows, slot_row, gates, storage, tokens=None, _o=orc.combine:
                              _o(o_rows, slot_row, np.ones_like(gates), storage, tokens), [check_dense_identity]),
    "bf16_truncates": ("round_to_bf16", lambda a: (np.ascontiguousarray(a, np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32),
                       [check_bf16_rounding]),
}


def _fill_reverse(idx, E, cap, _orig=orc.fill_in_token_order):
    T = idx.shape[0]
    demand, offsets, slot_row, row_slot = _orig(idx[::-1].copy(), E, cap)
    return demand, offsets, slot_row[::-1].copy(), (T - 1 - row_slot // idx.shape[1]) * idx.shape[1] + row_slot % idx.shape[1]


MUTANTS["fill_from_the_end"] = ("fill_in_token_order", _fill_reverse, [check_permutation_bruteforce])
MUTANTS["switch_renormalised"] = ("switch_gates", lambda logits, idx, scaled: orc.topk_gates(logits, idx),
                                  [check_switch_printed_gates])
MUTANTS["switch_scale_k_over_E"] = ("switch_gates", lambda logits, idx, scaled, _o=orc.switch_gates:
                                    _o(logits, idx, False) * (idx.shape[1] / logits.shape[1] if scaled else 1.0),
                                    [check_switch_scaled_zero_router_is_dense])
MUTANTS["bpr_ascending"] = ("priority_order", lambda score: np.argsort(
    np.asarray(score, np.float64).astype(np.float32), kind="stable"), [check_bpr_bruteforce])
MUTANTS["bpr_ties_to_later_token"] = ("priority_order", lambda score: np.lexsort(
    (-np.arange(len(score)), -np.asarray(score, np.float64).astype(np.float32).astype(np.float64))),
    [check_bpr_bruteforce])
MUTANTS["ec_selects_by_logit"] = ("softmax_scores", lambda logits: np.asarray(logits, np.float64),
                                  [check_ec_selects_by_score_not_logit])
MUTANTS["ec_ties_to_later_token"] = ("expert_choice_select", lambda S, C, _o=orc.expert_choice_select:
                                     _ec_reversed(S, C, _o), [check_ec_zero_router])
MUTANTS["ec_rows_in_score_order"] = ("expert_choice_select", lambda S, C: _ec_score_order(S, C),
                                     [check_ec_bruteforce])
MUTANTS["silu_grad_is_sigmoid"] = ("silu_grad", lambda a: 1.0 / (1.0 + np.exp(-a)),
                                   [check_backward_autograd])
MUTANTS["softmax_grad_without_the_mean"] = ("topk_softmax_grad", lambda gates, dg: gates * dg,
                                            [check_backward_autograd])
MUTANTS["bpr_score_as_float64"] = ("priority_order", lambda score: np.argsort(
    -np.asarray(score, np.float64), kind="stable"), [check_bpr_float32_decision])


def _ec_combine_renormalised(o_rows, slot, scores, storage, tokens=None, _o=orc.expert_choice_combine):
    """Gates renormalised over the experts that chose the token."""
    chosen = slot >= 0
    mass = np.where(chosen, scores, 0.0).sum(axis=1, keepdims=True)
    s = np.where(chosen, scores / np.where(mass > 0, mass, 1.0), 0.0)
    return _o(o_rows, slot, s, storage, tokens)


MUTANTS["ec_combine_renormalised"] = ("expert_choice_combine", _ec_combine_renormalised,
                                      [check_ec_partial_capacity_dense_eval])


MUTANTS["switch_grad_chosen_logits_only"] = (
    "switch_softmax_grad",
    lambda logits, idx, dg, scaled, _o=orc.switch_softmax_grad: _mask_chosen(_o(logits, idx, dg, scaled), idx),
    [check_backward_gating_finite_differences, check_backward_gating_autograd])
MUTANTS["switch_grad_without_rescale"] = (
    "switch_softmax_grad", lambda logits, idx, dg, scaled, _o=orc.switch_softmax_grad: _o(logits, idx, dg, False),
    [check_backward_gating_finite_differences, check_backward_gating_autograd])


def _mask_chosen(dl, idx):
    """Keep dl only at each token's chosen experts."""
    m = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(m, idx.astype(np.int64), True, axis=1)
    return np.where(m, dl, 0.0)


def _hold_skipping(skip):
    def hold(v, storage, point, _o=orc.hold):
        return np.asarray(v, np.float64) if point in skip else _o(v, storage, point)
    return hold


MUTANTS["backward_no_intermediate_rounding"] = ("hold", _hold_skipping(set(orc.BACKWARD_ROUNDING_POINTS)),
                                                [check_backward_rounding_points_bf16])
for _p in orc.BACKWARD_ROUNDING_POINTS:
    MUTANTS[f"backward_{_p}_unrounded"] = ("hold", _hold_skipping({_p}), [check_backward_rounding_points_bf16])


MUTANTS["ec_grad_chosen_logits_only"] = (
    "softmax_grad", lambda p, dp, _o=orc.softmax_grad: np.where(dp != 0, _o(p, dp), 0.0),
    [check_ec_backward_finite_differences, check_ec_backward_autograd])
MUTANTS["ec_grad_without_the_mean"] = ("softmax_grad", lambda p, dp: p * dp,
                                       [check_ec_backward_finite_differences, check_ec_backward_autograd])
for _p in orc.BACKWARD_ROUNDING_POINTS:
    MUTANTS[f"ec_backward_{_p}_unrounded"] = ("hold", _hold_skipping({_p}), [check_ec_backward_rounding_points_bf16])


def _ec_reversed(S, C, orig):
    """Ties to the later token: select on the reversed token order."""
    T = S.shape[0]
    tok, _ = orig(S[::-1].copy(), C)
    tok = np.sort(T - 1 - tok, axis=1)
    slot = np.full(S.shape, -1, dtype=np.int32)
    for e in range(S.shape[1]):
        slot[tok[e], e] = e * C + np.arange(C)
    return tok.astype(np.int32), slot


def _ec_score_order(S, C):
    """Rows in descending score order instead of token order."""
    s32 = np.asarray(S, np.float64).astype(np.float32).astype(np.float64)
    T, E = S.shape
    tok = np.empty((E, C), dtype=np.int32)
    slot = np.full((T, E), -1, dtype=np.int32)
    for e in range(E):
        tok[e] = np.argsort(-s32[:, e], kind="stable")[:C]
        slot[tok[e], e] = e * C + np.arange(C)
    return tok, slot


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn, pins = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = False
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught = True
    assert caught, f"planted mistake {name} passed every pin"


def test_routing_conditioned_oracle_reduces_to_the_oracle():
    """forward(idx=, slot_row=) with the oracle's own decisions is the oracle;
    any other valid layout (rows reordered inside each expert's block) gives
    the same y (the combine follows the slots, not the row order); a layout
    with a row outside its expert's block is refused. The same for expert
    choice with its own selection."""
    x, wr, wg, wu, wd = small_layer(T=40, E=5, k=2)
    ref = orc.forward(x, wr, wg, wu, wd, 2, 0.75, "f64")
    again = orc.forward(x, wr, wg, wu, wd, 2, 0.75, "f64", idx=ref["topk_idx"], slot_row=ref["slot_row"])
    for key in ("demand", "offsets", "slot_row", "row_slot"):
        assert np.array_equal(again[key], ref[key]), key
    assert np.array_equal(again["y"], ref["y"])
    # reverse the rows of every expert's block
    off = ref["offsets"]
    new_row = np.arange(int(off[-1]))
    for e in range(5):
        new_row[off[e]:off[e + 1]] = new_row[off[e]:off[e + 1]][::-1]
    srow = np.where(ref["slot_row"] >= 0, new_row[np.maximum(ref["slot_row"], 0)], -1)
    rev = orc.forward(x, wr, wg, wu, wd, 2, 0.75, "f64", idx=ref["topk_idx"], slot_row=srow)
    assert np.allclose(rev["y"], ref["y"], rtol=1e-13, atol=1e-14)
    bad = ref["slot_row"].copy()
    swap = np.nonzero((bad >= 0) & (ref["topk_idx"] == 0))
    other = np.nonzero((bad >= 0) & (ref["topk_idx"] == 1))
    bad[swap[0][0], swap[1][0]], bad[other[0][0], other[1][0]] = bad[other[0][0], other[1][0]], bad[swap[0][0], swap[1][0]]
    with pytest.raises(AssertionError):
        orc.forward(x, wr, wg, wu, wd, 2, 0.75, "f64", idx=ref["topk_idx"], slot_row=bad)
    ec = orc.expert_choice_forward(x, wr, wg, wu, wd, 2, 0.5, "f64")
    ec2 = orc.expert_choice_forward(x, wr, wg, wu, wd, 2, 0.5, "f64", slot=ec["slot"])
    assert np.array_equal(ec2["y"], ec["y"]) and np.array_equal(ec2["tokens"], ec["tokens"])
