"""GPU parity: every entry point of libmoe against the CPU oracle, on the same
seeded inputs. Stage tests feed each entry point the oracle's own inputs for
that stage; forward tests run the whole layer. Small cases span several tiles
and a ragged tail; the named workloads run at full size with every output row
compared (y of every token, h and o of every kept row)."""
import functools

import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_09_amd as moe
from oracle import moe_oracle as orc
from parity import assert_close_rows, compare_routing, host

pytestmark = pytest.mark.gpu

# (T, d, E, k, F, cf, dtype, seed)
SMALL = [
    (300, 256, 8, 2, 320, 1.25, "bf16", 10),     # drops, several row tiles, ragged tail
    (517, 128, 6, 3, 192, 0.0, "bf16", 11),      # dropless, k = 3
    (1000, 512, 16, 4, 256, 1.0, "bf16", 12),
    (700, 256, 64, 8, 192, 1.0, "bf16", 18),     # many experts, k = 8
    (100, 128, 8, 8, 128, 0.0, "bf16", 16),      # k = E: dense softmax gating
    (130, 64, 1, 1, 64, 0.0, "bf16", 15),        # one expert: the dense FFN
    (1, 128, 8, 2, 128, 0.0, "bf16", 17),        # a single token
    (333, 64, 4, 2, 64, 0.5, "bf16", 19),        # heavy dropping
    (32, 512, 8, 2, 256, 0.0, "bf16", 21),       # decode-sized: 64 rows, weight-streaming GEMMs
    (20, 64, 4, 3, 192, 0.0, "bf16", 22),        # 60 rows, one 64-deep K step in the gate/up GEMM
    (64, 192, 1, 1, 128, 0.0, "bf16", 23),       # one expert with 64 rows: two full token tiles
    (48, 128, 4, 1, 128, 0.5, "bf16", 24),       # decode-sized with drops
    (600, 128, 256, 8, 64, 1.0, "bf16", 27),     # the most experts and slots: E = 256, k = 8
    (40, 128, 256, 8, 64, 1.0, "bf16", 25),      # E = 256 with 78 empty experts, capacity 2
    (200, 64, 8, 2, 64, 0.01, "bf16", 26),       # capacity 1: every expert keeps one token
    (257, 64, 4, 1, 128, 1.25, "f32", 13),
    (200, 100, 5, 2, 72, 0.8, "f32", 14),        # fp32: d, F not multiples of the tiles
    (90, 32, 3, 3, 36, 0.0, "f32", 20),
]
NAMED_SMALL = ["tiny_fp32"]
FULL = ["mixtral_bf16", "openmoe_bf16", "finegrained_bf16", "decode_bf16"]


def case_id(c):
    return c if isinstance(c, str) else "T{}_d{}_E{}_k{}_F{}_cf{}_{}".format(*c[:7])


@functools.lru_cache(maxsize=None)
def workload(case):
    if isinstance(case, str):
        w = mi.WORKLOADS[case]
        return w, mi.generate(w)
    return mi.random_small(*case)


@functools.lru_cache(maxsize=None)
def reference(case):
    """Full oracle forward (small cases only)."""
    w, a = workload(case)
    return orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)


def dev(t):
    return t.to("cuda").contiguous()


def tdtype(w):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def as_storage(arr, w):
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(tdtype(w))


@functools.lru_cache(maxsize=2)
def device_inputs(case):
    w, a = workload(case)
    return {k: dev(v) for k, v in a.items() if v is not None and k != "token_ids"}


# ---------------------------------------------------------------------------
# stage by stage, small cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_route(case):
    w, a = workload(case)
    ref = reference(case)
    g = device_inputs(case)
    idx, gate, logits = moe.moe_route(g["x"], g["w_router"], w.k, want_logits=True)
    torch.cuda.synchronize()
    flips = compare_routing(host(idx), host(gate), ref)
    assert flips == 0
    l = host(logits)
    assert np.all(np.abs(l - ref["logits"]) <= 1e-5 * (1.0 + np.abs(ref["logits"])))
    gs = host(gate).sum(axis=1)
    assert np.all(np.abs(gs - 1.0) <= 1e-6 * w.k)
    if w.k == 1:
        assert np.all(host(gate) == 1.0)


# Router-only shapes: every expert-tile width of the bf16 kernel (E up to 256),
# one- and two-tile token blocks with a ragged last block, d down to one
# 16-byte piece and d ending inside a 128-column step; fp32 with large E.
ROUTE_SHAPES = [
    (1000, 200, 256, 8, "bf16", 30),
    (8200, 264, 200, 2, "bf16", 31),
    (9000, 136, 100, 3, "bf16", 32),
    (8193, 64, 40, 5, "bf16", 33),
    (5000, 8, 2, 2, "bf16", 34),
    (17, 1032, 16, 1, "bf16", 35),
    (70, 72, 200, 8, "f32", 36),
]


@pytest.mark.parametrize("case", ROUTE_SHAPES, ids=lambda c: "T{}_d{}_E{}_k{}_{}".format(*c[:5]))
def test_route_shapes(case):
    T, d, E, k, dtype, seed = case
    w = mi.Workload(f"route_T{T}_d{d}_E{E}", T=T, d=d, E=E, k=k, F=8, cf=0.0, dtype=dtype, seed=seed)
    a = mi.generate(w, expert_weights=False)
    logits, idx_ref, gate_ref, near = orc.route(a["x"], a["w_router"], k)
    idx, gate, lg = moe.moe_route(dev(a["x"]), dev(a["w_router"]), k, want_logits=True)
    torch.cuda.synchronize()
    flips = compare_routing(host(idx), host(gate), {"topk_idx": idx_ref, "topk_gate": gate_ref, "near_tie": near})
    assert flips <= int(near.sum())
    l = host(lg)
    assert np.all(np.abs(l - logits) <= 1e-5 * (1.0 + np.abs(logits)))


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_permute(case):
    w, a = workload(case)
    ref = reference(case)
    g = device_inputs(case)
    idx = dev(torch.from_numpy(ref["topk_idx"]))
    out = moe.moe_permute(g["x"], idx, w.E, w.cf)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1])
    assert np.array_equal(host(out["expert_counts"]), ref["demand"])
    assert np.array_equal(host(out["expert_offsets"]), ref["offsets"])
    assert np.array_equal(host(out["slot_row"]), ref["slot_row"])
    assert np.array_equal(host(out["row_slot"])[:R], ref["row_slot"])
    xp = out["x_perm"][:R].cpu()
    assert torch.equal(xp, a["x"][torch.from_numpy(ref["row_slot"].astype(np.int64)) // w.k])


# Token counts on both sides of the one-workgroup layout (up to 1024 tokens)
# and of the scatter's switch from a wavefront per 1 KB piece to a wavefront
# per row (2048 tokens); rows of 1200 bytes end inside their second piece.
@pytest.mark.parametrize("T,d,E,k,cf,dtype,seed", [
    (1024, 600, 256, 8, 1.0, "bf16", 60),   # the largest one-workgroup layout, E = 256
    (1025, 600, 16, 2, 0.7, "bf16", 61),    # the smallest chunked layout
    (2047, 300, 8, 2, 1.0, "f32", 62),
    (2048, 600, 8, 3, 0.9, "bf16", 63),
    (999, 64, 1, 1, 0.5, "bf16", 64),       # one expert, half the tokens dropped
])
def test_permute_layout_sizes(T, d, E, k, cf, dtype, seed):
    w = mi.Workload("perm_sizes", T=T, d=d, E=E, k=k, F=8, cf=cf, dtype=dtype, seed=seed)
    a = mi.generate(w, expert_weights=False)
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    cap = orc.capacity(T, E, k, cf)
    demand, offsets, slot_row, row_slot = orc.fill_in_token_order(idx, E, cap)
    out = moe.moe_permute(dev(a["x"]), dev(torch.from_numpy(idx)), E, cf)
    torch.cuda.synchronize()
    R = int(offsets[-1])
    assert np.array_equal(host(out["expert_counts"]), demand)
    assert np.array_equal(host(out["expert_offsets"]), offsets)
    assert np.array_equal(host(out["slot_row"]), slot_row)
    assert np.array_equal(host(out["row_slot"])[:R], row_slot)
    assert torch.equal(out["x_perm"][:R].cpu(), a["x"][torch.from_numpy(row_slot.astype(np.int64)) // k])


@pytest.mark.parametrize("T", [300, 3000])
def test_permute_repeated_or_out_of_range_ids_stay_in_bounds(T):
    """Caller-supplied indices outside the contract (a repeated expert id in a
    token, ids outside [0, E)): the layout is unspecified, but every row the
    call reports lies inside x_perm, kept rows are a prefix of it, every kept
    row holds its token's row of x and an out-of-range id is a dropped slot.
    Both layout paths (one workgroup up to 1024 tokens, chunked above)."""
    E, k, d, cf = 8, 3, 64, 0.0
    rng = np.random.default_rng(T)
    idx = rng.integers(0, E, (T, k)).astype(np.int32)
    idx[::7, 1] = idx[::7, 0]                   # repeats
    idx[::11, 2] = E + 5                        # out of range
    idx[::13, 0] = -3
    x = torch.from_numpy(rng.standard_normal((T, d)).astype(np.float32)).to(torch.bfloat16)
    R_max = moe.moe_rows_max(T, E, k, cf)
    out = moe.moe_permute(dev(x), dev(torch.from_numpy(idx)), E, cf)
    torch.cuda.synchronize()
    off = host(out["expert_offsets"])
    R = int(off[-1])
    assert 0 <= R <= R_max and np.all(np.diff(off) >= 0)
    srow = host(out["slot_row"])
    assert np.all((srow >= -1) & (srow < R))
    bad = (idx < 0) | (idx >= E)
    assert np.all(srow[bad] == -1)
    tt, jj = np.nonzero(srow >= 0)
    xp = out["x_perm"][:R].cpu()
    assert torch.equal(xp[torch.from_numpy(srow[tt, jj].astype(np.int64))], x[torch.from_numpy(tt)])


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_grouped_ffn(case):
    w, a = workload(case)
    ref = reference(case)
    g = device_inputs(case)
    R = int(ref["offsets"][-1])
    R_max = moe.moe_rows_max(w.T, w.E, w.k, w.cf)
    x_perm = torch.zeros((max(R_max, 1), w.d), dtype=tdtype(w))
    x_perm[:R] = a["x"][torch.from_numpy(ref["row_slot"].astype(np.int64)) // w.k]
    offsets = dev(torch.from_numpy(ref["offsets"]))
    h, o = moe.moe_grouped_ffn(dev(x_perm), offsets, g["w_gate"], g["w_up"], g["w_down"], w.T, w.k, w.cf)
    torch.cuda.synchronize()
    if R == 0:
        return
    assert_close_rows(host(h[:R]), ref["h_rows"], w.dtype, "h")
    assert_close_rows(host(o[:R]), ref["o_rows"], w.dtype, "o")


# Expert row counts that give the 256-row-tile GEMMs every tile shape: last
# row tiles of 1 and 64 rows (the 64-row body), 65 and 128 (the 128-row
# body), 129, 255 and 256 (full), an empty expert and experts of several
# tiles; the down projection with and without its split tail (the tail tiles
# of each XCD cut into K-slices when the workspace is given).
TILE_COUNTS = [1, 64, 65, 128, 129, 255, 256, 257, 300, 0, 511, 640]


@pytest.mark.parametrize("split", [True, False], ids=["split_tail", "whole_tiles"])
def test_grouped_ffn_tile_shapes(split):
    E, d, F = len(TILE_COUNTS), 512, 384
    offsets = np.concatenate([[0], np.cumsum(TILE_COUNTS)]).astype(np.int32)
    R = int(offsets[-1])
    assert R >= 128 * E   # the 256-row tiles
    w = mi.Workload("tile_shapes", T=R, d=d, E=E, k=1, F=F, cf=0.0, dtype="bf16", seed=70)
    a = mi.generate(w)
    xp = dev(a["x"])
    h, o = moe.moe_grouped_ffn_rows(xp, dev(torch.from_numpy(offsets)), dev(a["w_gate"]), dev(a["w_up"]),
                                    dev(a["w_down"]), R, ws=None if split else False)
    torch.cuda.synchronize()
    hs, os_ = [], []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        he, oe = orc.swiglu_expert(a["x"][lo:hi], a["w_gate"][e], a["w_up"][e], a["w_down"][e], "bf16")
        hs.append(he)
        os_.append(oe)
    assert_close_rows(host(h[:R]), np.concatenate(hs), "bf16", "h")
    assert_close_rows(host(o[:R]), np.concatenate(os_), "bf16", "o")


# The most experts with 256-row tiles (at least 128 rows per expert on
# average): every thread of the per-XCD plan's block scan holds an expert,
# and most experts end in a ragged tile of at most 128 rows.
@pytest.mark.parametrize("E,R,seed", [(256, 32768, 80), (255, 33000, 81)])
def test_grouped_ffn_many_experts(E, R, seed):
    d, F = 128, 128
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(R, np.full(E, 1.0 / E))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    assert R >= 128 * E   # the 256-row tiles
    w = mi.Workload("many_experts", T=R, d=d, E=E, k=1, F=F, cf=0.0, dtype="bf16", seed=seed)
    a = mi.generate(w)
    h, o = moe.moe_grouped_ffn_rows(dev(a["x"]), dev(torch.from_numpy(offsets)), dev(a["w_gate"]), dev(a["w_up"]),
                                    dev(a["w_down"]), R)
    torch.cuda.synchronize()
    hs, os_ = [], []
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        he, oe = orc.swiglu_expert(a["x"][lo:hi], a["w_gate"][e], a["w_up"][e], a["w_down"][e], "bf16")
        hs.append(he)
        os_.append(oe)
    assert_close_rows(host(h[:R]), np.concatenate(hs), "bf16", "h")
    assert_close_rows(host(o[:R]), np.concatenate(os_), "bf16", "o")


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_unpermute_combine(case):
    w, a = workload(case)
    ref = reference(case)
    R = int(ref["offsets"][-1])
    R_max = moe.moe_rows_max(w.T, w.E, w.k, w.cf)
    o = torch.zeros((max(R_max, 1), w.d), dtype=tdtype(w))
    o[:R] = as_storage(ref["o_rows"], w)
    gate32 = ref["topk_gate"].astype(np.float32)
    y = moe.moe_unpermute_combine(dev(o), dev(torch.from_numpy(ref["slot_row"])), dev(torch.from_numpy(gate32)),
                                  w.E, w.cf)
    torch.cuda.synchronize()
    y_ref = orc.combine(ref["o_rows"], ref["slot_row"], gate32.astype(np.float64), w.dtype)
    assert_close_rows(host(y), y_ref, w.dtype)


# ---------------------------------------------------------------------------
# the whole layer, small cases
# ---------------------------------------------------------------------------

def run_forward(w, g):
    T = w.T
    idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    gate = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    srow = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    y = moe.moe_forward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf,
                        topk_idx=idx, topk_gate=gate, slot_row=srow)
    torch.cuda.synchronize()
    return y, idx, gate, srow


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_forward(case):
    w, a = workload(case)
    ref = reference(case)
    g = device_inputs(case)
    y, idx, gate, srow = run_forward(w, g)
    assert compare_routing(host(idx), host(gate), ref) == 0
    assert np.array_equal(host(srow), ref["slot_row"])
    rel, mae = assert_close_rows(host(y), ref["y"], w.dtype)
    print(f"{case_id(case)}: row max-rel {rel:.3g}, MAE {mae:.3g}")
    if w.dtype == "bf16":
        # transparency: distance to a float32-storage oracle (no bf16 rounding of h, o)
        ref32 = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, "f32")
        d = np.abs(host(y) - ref32["y"])
        print(f"  vs fp32-storage oracle: MAE {d.mean():.3g}")


def test_forward_is_deterministic():
    case = SMALL[3]
    w, _ = workload(case)
    g = device_inputs(case)
    first = [t.clone() for t in run_forward(w, g)]
    for _ in range(9):
        again = run_forward(w, g)
        for a_, b_ in zip(first, again):
            assert torch.equal(a_, b_)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_zero_router_drops_in_token_order(dtype):
    """W_g = 0: every token picks experts 0..k-1 with gates 1/k; with cf = 0.5
    those experts keep exactly tokens 0..cap-1; later tokens are dropped and
    their output is exactly zero."""
    w, a = mi.random_small(200, 128, 8, 2, 128, 0.5, dtype, 21)
    a = dict(a)
    a["w_router"] = torch.zeros_like(a["w_router"])
    ref = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)
    cap = ref["cap"]
    assert cap == 25   # ceil(0.5 * 200 * 2 / 8)
    g = {k: dev(v) for k, v in a.items() if v is not None}
    y, idx, gate, srow = run_forward(w, g)
    assert np.all(host(idx) == np.arange(w.k))
    assert np.all(host(gate) == np.float32(1.0 / w.k))
    s = host(srow)
    assert np.array_equal(s, ref["slot_row"])
    assert np.all(s[:cap] >= 0) and np.all(s[cap:] == -1)
    yy = host(y)
    assert np.all(yy[cap:] == 0.0)
    assert_close_rows(yy, ref["y"], w.dtype)


def test_identical_experts_reproduce_the_dense_ffn():
    """Copies of one FFN with Softmax(TopK) gates give the dense FFN (the
    upcycling property), here within bf16 rounding of h, o and y."""
    w, a = mi.random_small(256, 256, 8, 2, 256, 0.0, "bf16", 22)
    a = dict(a)
    for key in ("w_gate", "w_up", "w_down"):
        a[key] = a[key][:1].expand_as(a[key]).contiguous()
    g = {k: dev(v) for k, v in a.items() if v is not None}
    y, *_ = run_forward(w, g)
    x = a["x"].double()
    dense = (torch.nn.functional.silu(x @ a["w_gate"][0].double().T) * (x @ a["w_up"][0].double().T)) \
        @ a["w_down"][0].double().T
    rel = ((host(y) - dense.numpy()).__abs__().max(axis=1) / np.abs(dense.numpy()).max(axis=1)).max()
    assert rel < 3e-2


# ---------------------------------------------------------------------------
# the named workloads at full size (every output row compared)
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=1)
def full_reference(name):
    w, a = workload(name)
    logits, idx, gates, tie = orc.route(a["x"], a["w_router"], w.k)
    cap = orc.capacity(w.T, w.E, w.k, w.cf)
    demand, offsets, slot_row, row_slot = orc.fill_in_token_order(idx, w.E, cap)
    return dict(logits=logits, topk_idx=idx, topk_gate=gates, near_tie=tie, cap=cap, demand=demand,
                offsets=offsets, slot_row=slot_row, row_slot=row_slot)


@functools.lru_cache(maxsize=None)
def full_oracle(name):
    """The whole oracle forward of a named workload: y of every token, h and o
    of every kept row (a few seconds each on the host's BLAS threads)."""
    w, a = workload(name)
    return orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)


@pytest.mark.parametrize("name", FULL)
def test_full_size_forward(name):
    """moe_forward at full size: routing bit-exact (near ties counted), the
    permutation bit-exact and y of every token within tolerance. A near-tie
    token the kernel routed the other way is not left out: the oracle is then
    conditioned on the kernel's indices (the same layer fed those decisions),
    which fixes every slot row and every output, flipped token included."""
    w, a = workload(name)
    ref = full_oracle(name)
    g = device_inputs(name)
    y, idx, gate, srow = run_forward(w, g)
    flips = compare_routing(host(idx), host(gate), ref)
    print(f"{name}: near-tie tokens {int(ref['near_tie'].sum())}, flipped {flips}")
    if flips:
        ref = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                          idx=host(idx))
        assert compare_routing(host(idx), host(gate), ref) == 0
    assert np.array_equal(host(srow), ref["slot_row"])
    rel, mae = assert_close_rows(host(y), ref["y"], w.dtype)
    print(f"{name}: all {w.T} tokens, row max-rel {rel:.3g}, MAE {mae:.3g}")


@pytest.mark.parametrize("name", FULL)
def test_full_size_permute(name):
    w, a = workload(name)
    ref = full_reference(name)
    g = device_inputs(name)
    out = moe.moe_permute(g["x"], dev(torch.from_numpy(ref["topk_idx"])), w.E, w.cf)
    torch.cuda.synchronize()
    R = int(ref["offsets"][-1])
    assert np.array_equal(host(out["expert_counts"]), ref["demand"])
    assert np.array_equal(host(out["expert_offsets"]), ref["offsets"])
    assert np.array_equal(host(out["slot_row"]), ref["slot_row"])
    assert np.array_equal(host(out["row_slot"])[:R], ref["row_slot"])
    rows = torch.from_numpy(ref["row_slot"].astype(np.int64)) // w.k
    assert torch.equal(out["x_perm"][:R].cpu(), a["x"][rows])


@pytest.mark.parametrize("name", FULL)
def test_full_size_grouped_ffn(name):
    """moe_grouped_ffn at full size on the oracle's permutation: every kept
    row of h and of o."""
    w, a = workload(name)
    ref = full_oracle(name)
    g = device_inputs(name)
    R = int(ref["offsets"][-1])
    R_max = moe.moe_rows_max(w.T, w.E, w.k, w.cf)
    rows_tok = torch.from_numpy(ref["row_slot"].astype(np.int64)) // w.k
    x_perm = torch.zeros((R_max, w.d), dtype=tdtype(w), device="cuda")
    x_perm[:R] = g["x"][rows_tok.cuda()]
    h, o = moe.moe_grouped_ffn(x_perm, dev(torch.from_numpy(ref["offsets"])), g["w_gate"], g["w_up"],
                               g["w_down"], w.T, w.k, w.cf)
    torch.cuda.synchronize()
    rel_h, _ = assert_close_rows(host(h[:R]), ref["h_rows"], w.dtype, "h")
    rel_o, _ = assert_close_rows(host(o[:R]), ref["o_rows"], w.dtype, "o")
    print(f"{name}: all {R} rows, h max-rel {rel_h:.3g}, o max-rel {rel_o:.3g}")


@pytest.mark.parametrize("name", FULL)
def test_full_size_combine(name):
    """Combine at full size with synthetic expert outputs (bf16 N(0,1))."""
    w, a = workload(name)
    ref = full_reference(name)
    R = int(ref["offsets"][-1])
    R_max = moe.moe_rows_max(w.T, w.E, w.k, w.cf)
    gen = torch.Generator().manual_seed(5)
    o = torch.randn((R_max, w.d), generator=gen).to(tdtype(w))
    gate32 = ref["topk_gate"].astype(np.float32)
    y = moe.moe_unpermute_combine(dev(o), dev(torch.from_numpy(ref["slot_row"])), dev(torch.from_numpy(gate32)),
                                  w.E, w.cf)
    torch.cuda.synchronize()
    y_ref = orc.combine(o[:R].double().numpy(), ref["slot_row"], gate32.astype(np.float64), w.dtype)
    assert_close_rows(host(y), y_ref, w.dtype)


# ---------------------------------------------------------------------------
# the down projection's split tail (256-row tiles): every output row compared
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    (2048, 512, 8, 2, 1024, 0.0, "bf16", 31),    # fewer tiles than compute units: every tile split
    (4096, 2048, 8, 2, 1024, 0.0, "bf16", 32),   # whole rounds plus a split tail
    (3000, 1024, 6, 2, 512, 1.1, "bf16", 33),    # drops, ragged experts
], ids=case_id)
def test_grouped_ffn_split_tail(case):
    w, a = mi.random_small(*case)
    logits, idx, gates, tie = orc.route(a["x"], a["w_router"], w.k)
    cap = orc.capacity(w.T, w.E, w.k, w.cf)
    demand, offsets, slot_row, row_slot = orc.fill_in_token_order(idx, w.E, cap)
    R = int(offsets[-1])
    R_max = moe.moe_rows_max(w.T, w.E, w.k, w.cf)
    assert R_max >= 128 * w.E   # the 256-row tile path
    rows_tok = torch.from_numpy(row_slot.astype(np.int64)) // w.k
    x_perm = torch.zeros((R_max, w.d), dtype=torch.bfloat16)
    x_perm[:R] = a["x"][rows_tok]
    g = {n: dev(a[n]) for n in ("w_gate", "w_up", "w_down")}
    xp, off = dev(x_perm), dev(torch.from_numpy(offsets))
    h1, o1 = moe.moe_grouped_ffn(xp, off, g["w_gate"], g["w_up"], g["w_down"], w.T, w.k, w.cf)
    h2, o2 = moe.moe_grouped_ffn(xp, off, g["w_gate"], g["w_up"], g["w_down"], w.T, w.k, w.cf)
    h3, o3 = moe.moe_grouped_ffn(xp, off, g["w_gate"], g["w_up"], g["w_down"], w.T, w.k, w.cf, ws=False)
    torch.cuda.synchronize()
    assert torch.equal(o1[:R], o2[:R])          # deterministic
    hh = np.empty((R, w.F))
    oo = np.empty((R, w.d))
    for e in range(w.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            hh[lo:hi], oo[lo:hi] = orc.swiglu_expert(a["x"][rows_tok[lo:hi]], a["w_gate"][e], a["w_up"][e],
                                                     a["w_down"][e], "bf16")
    assert_close_rows(host(h1[:R]), hh, "bf16", "h")
    assert_close_rows(host(o1[:R]), oo, "bf16", "o (split tail)")
    assert_close_rows(host(o3[:R]), oo, "bf16", "o (no split)")


@pytest.mark.parametrize("fill", ["token", "priority"])
@pytest.mark.parametrize("case", [
    (3000, 1024, 6, 4, 512, 1.1, "bf16", 33),    # drops, ragged experts
    (2048, 512, 16, 8, 256, 0.0, "bf16", 31),    # dropless, k = 8
    (1000, 512, 16, 4, 256, 1.0, "bf16", 12),    # k = 4, 16 experts
    (2048, 512, 8, 2, 1024, 0.0, "bf16", 34),    # k = 2: no gather, same check
], ids=case_id)
def test_forward_gather_equals_stage_path(case, fill):
    """With 256-row tiles and k >= 4, moe_forward's gate/up GEMM reads the token
    rows of x through the row -> slot map instead of a scattered x_perm; the
    staged path (moe_permute's scatter, then moe_grouped_ffn) must give the
    same bits, and both must match the oracle."""
    w, a = workload(case)
    assert moe.moe_rows_max(w.T, w.E, w.k, w.cf) >= 128 * w.E   # 256-row tiles
    g = device_inputs(case)
    y = moe.moe_forward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf, fill_order=fill)
    idx, gate, _ = moe.moe_route(g["x"], g["w_router"], w.k)
    perm = moe.moe_permute(g["x"], idx, w.E, w.cf, score=gate if fill == "priority" else None, score_stride=w.k)
    h, o = moe.moe_grouped_ffn(perm["x_perm"], perm["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"],
                               w.T, w.k, w.cf)
    y2 = moe.moe_unpermute_combine(o, perm["slot_row"], gate, w.E, w.cf)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    ref = orc.forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                      bpr=fill == "priority")
    assert_close_rows(host(y), ref["y"], w.dtype)
