"""GPU parity for expert-choice routing (each expert takes its C best tokens
by the dense gate Softmax(x.W_g)) against the CPU oracle, through the C
interface: scores, the per-expert selection, the row gather, the grouped FFN
over the selected rows, the variable fan-in combine, and the whole layer."""
import functools

import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_09_amd as moe
from oracle import moe_oracle as orc
from parity import assert_close_rows, host
from test_gpu_parity import NAMED_SMALL, SMALL, case_id, dev, device_inputs, workload

pytestmark = pytest.mark.gpu

BAND = 1e-5   # relative: the kernel's float32 score can differ from the oracle's by a few ulps


@functools.lru_cache(maxsize=None)
def ec_reference(case):
    w, a = workload(case)
    return orc.expert_choice_forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)


def boundary_bands(S, C):
    """Per expert: the C-th largest float32 score b, and the tokens whose score
    lies within BAND (relative) of b. Where that band holds only the C-th token
    itself and the (C+1)-th lies outside, the chosen set is decided the same
    way by any float32 evaluation that is within a few ulps."""
    s32 = np.asarray(S, np.float64).astype(np.float32).astype(np.float64)
    T, E = s32.shape
    amb_expert = np.zeros(E, dtype=bool)
    in_band = np.zeros((T, E), dtype=bool)
    if C >= T:
        return amb_expert, in_band
    srt = np.sort(s32, axis=0)[::-1]
    for e in range(E):
        b = srt[C - 1, e]
        band = np.abs(s32[:, e] - b) <= BAND * abs(b)
        in_band[:, e] = band
        amb_expert[e] = band.sum() > 1
    return amb_expert, in_band


def check_selection(S, C, tokens_gpu, slot_gpu, offsets_gpu, tok_ref, slot_ref):
    T, E = S.shape
    assert np.array_equal(offsets_gpu, np.arange(E + 1) * C)
    amb, band = boundary_bands(S, C)
    s32 = np.asarray(S, np.float64).astype(np.float32).astype(np.float64)
    srt = np.sort(s32, axis=0)[::-1]
    tg = tokens_gpu[:E * C].reshape(E, C)
    for e in range(E):
        assert np.all(np.diff(tg[e]) > 0), f"expert {e}: rows not in ascending token order"
        assert np.array_equal(slot_gpu[tg[e], e], e * C + np.arange(C))
        assert (slot_gpu[:, e] >= 0).sum() == C
        if not amb[e]:
            assert np.array_equal(tg[e], tok_ref[e]), f"expert {e}"
            assert np.array_equal(slot_gpu[:, e], slot_ref[:, e])
        else:
            b = srt[C - 1, e]
            must = np.nonzero(s32[:, e] > b * (1 + BAND))[0]
            never = np.nonzero(s32[:, e] < b * (1 - BAND))[0]
            chosen = set(tg[e].tolist())
            assert set(must.tolist()) <= chosen and not (set(never.tolist()) & chosen)
    return amb, band


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_ec_route(case):
    w, a = workload(case)
    ref = ec_reference(case)
    g = device_inputs(case)
    out = moe.moe_route_expert_choice(g["x"], g["w_router"], w.k, w.cf)
    torch.cuda.synchronize()
    C = out["C"]
    assert C == ref["cap"]
    sc = host(out["scores"])
    assert np.all(np.abs(sc - ref["scores"]) <= 1e-5 * ref["scores"] + 1e-7)
    assert np.allclose(sc.sum(1), 1.0, rtol=0, atol=1e-5)
    amb, _ = check_selection(ref["scores"], C, host(out["expert_tokens"]), host(out["slot"]),
                             host(out["expert_offsets"]), ref["tokens"], ref["slot"])
    print(f"{case_id(case)}: C={C}, experts with a near tie at the boundary: {int(amb.sum())}")


@pytest.mark.parametrize("T,E,k,cf,seed", [(40000, 8, 2, 1.0, 60), (3000, 64, 8, 0.5, 61), (5, 3, 1, 1.0, 62),
                                           (1, 4, 2, 1.0, 63), (2048, 256, 4, 2.0, 64)])
def test_ec_route_sizes(T, E, k, cf, seed):
    """Selection over several sizes: a 40000-token column, one token, C = 1."""
    w = mi.Workload("ec", T=T, d=128, E=E, k=k, F=64, cf=cf, dtype="bf16", seed=seed)
    a = mi.generate(w, expert_weights=False)
    logits = orc.router_logits(a["x"], a["w_router"])
    S = orc.softmax_scores(logits)
    C = orc.capacity(T, E, k, cf)
    tok, slot = orc.expert_choice_select(S, C)
    out = moe.moe_route_expert_choice(dev(a["x"]), dev(a["w_router"]), k, cf)
    torch.cuda.synchronize()
    assert out["C"] == C
    check_selection(S, C, host(out["expert_tokens"]), host(out["slot"]), host(out["expert_offsets"]), tok, slot)


def test_ec_zero_router():
    """W_g = 0: all scores are 1/E, so every expert takes tokens 0..C-1 exactly
    and every later token's output is exactly zero."""
    w, a = mi.random_small(200, 128, 8, 2, 128, 0.5, "bf16", 65)
    a = dict(a)
    a["w_router"] = torch.zeros_like(a["w_router"])
    g = {k_: dev(v) for k_, v in a.items() if v is not None}
    C = orc.capacity(w.T, w.E, w.k, w.cf)
    out = moe.moe_route_expert_choice(g["x"], g["w_router"], w.k, w.cf)
    y = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf)
    torch.cuda.synchronize()
    assert np.array_equal(host(out["expert_tokens"])[:w.E * C].reshape(w.E, C), np.tile(np.arange(C), (w.E, 1)))
    assert np.all(host(out["scores"]) == np.float32(1.0 / w.E))
    ref = orc.expert_choice_forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)
    yy = host(y)
    assert np.all(yy[C:] == 0.0)
    assert_close_rows(yy, ref["y"], w.dtype)


def excluded_tokens(ref):
    """Tokens in a near-tie band of some expert with an ambiguous boundary."""
    amb, band = boundary_bands(ref["scores"], ref["cap"])
    return (band & amb[None, :]).any(axis=1)


@pytest.mark.parametrize("case", SMALL + NAMED_SMALL, ids=case_id)
def test_ec_forward(case):
    w, a = workload(case)
    ref = ec_reference(case)
    g = device_inputs(case)
    T, E = w.T, w.E
    scores = torch.empty((T, E), dtype=torch.float32, device="cuda")
    slot = torch.empty((T, E), dtype=torch.int32, device="cuda")
    y = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf,
                                      scores=scores, slot=slot)
    torch.cuda.synchronize()
    skip = excluded_tokens(ref)
    s = host(slot)
    assert np.array_equal(s[~skip], ref["slot"][~skip])
    rel, mae = assert_close_rows(host(y)[~skip], ref["y"][~skip], w.dtype)
    print(f"{case_id(case)}: {int(skip.sum())} tokens next to a near-tie boundary, max-rel {rel:.3g}")


@pytest.mark.parametrize("case", [SMALL[0], SMALL[2], SMALL[3], "tiny_fp32"], ids=case_id)
def test_ec_stages_match_forward(case):
    """route -> gather -> grouped FFN over rows -> combine, stage by stage, gives
    bit-for-bit the fused forward; the gather copies rows exactly; the FFN on
    the oracle's own selection matches the oracle's expert outputs."""
    w, a = workload(case)
    ref = ec_reference(case)
    g = device_inputs(case)
    out = moe.moe_route_expert_choice(g["x"], g["w_router"], w.k, w.cf)
    C = out["C"]
    R = w.E * C
    xp = moe.moe_gather_rows(g["x"], out["expert_tokens"], R)
    h, o = moe.moe_grouped_ffn_rows(xp, out["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"], R)
    y = moe.moe_combine_expert_choice(o, out["slot"], out["scores"], w.k, w.cf)
    y_fused = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf)
    torch.cuda.synchronize()
    assert torch.equal(y, y_fused)
    tok = out["expert_tokens"][:R].long().cpu()
    assert torch.equal(xp[:R].cpu(), a["x"][tok])
    # the oracle's own selection through the gather and the FFN
    tref = dev(torch.from_numpy(ref["tokens"].reshape(-1).astype(np.int32)))
    xp2 = moe.moe_gather_rows(g["x"], tref, R)
    _, o2 = moe.moe_grouped_ffn_rows(xp2, out["expert_offsets"], g["w_gate"], g["w_up"], g["w_down"], R)
    torch.cuda.synchronize()
    assert_close_rows(host(o2)[:R], ref["o_rows"], w.dtype, "o_rows")


def test_ec_gather_out_of_range_rows_are_zero():
    x = torch.randn((10, 64), device="cuda").to(torch.bfloat16)
    rt = torch.tensor([3, -1, 10, 9, 1 << 30, 0], dtype=torch.int32, device="cuda")
    xp = moe.moe_gather_rows(x, rt, 6)
    torch.cuda.synchronize()
    assert torch.equal(xp[0], x[3]) and torch.equal(xp[3], x[9]) and torch.equal(xp[5], x[0])
    for r in (1, 2, 4):
        assert torch.all(xp[r] == 0)


def test_ec_dense_capacity():
    """cf = 0: C = T, every expert takes every token: dense softmax gating."""
    w, a = mi.random_small(300, 128, 4, 2, 128, 0.0, "bf16", 66)
    g = {k_: dev(v) for k_, v in a.items() if v is not None}
    y = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf)
    torch.cuda.synchronize()
    ref = orc.expert_choice_forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype)
    assert ref["cap"] == w.T
    assert_close_rows(host(y), ref["y"], w.dtype)


def test_ec_forward_is_deterministic():
    case = SMALL[3]
    w, _ = workload(case)
    g = device_inputs(case)
    first = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf)
    for _ in range(5):
        again = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf)
        assert torch.equal(first, again)


@pytest.mark.parametrize("name", ["openmoe_bf16"])
def test_ec_full_size_forward(name):
    """Full-size expert choice (OpenMoE shape: C = 640 tokens per expert): the
    selection bit-exact outside float32 near-tie bands at an expert's C-th
    place, and y of every token against the oracle fed the kernel's selection
    (which differs from its own only inside those bands)."""
    w, a = workload(name)
    logits = orc.router_logits(a["x"], a["w_router"])
    S = orc.softmax_scores(logits)
    C = orc.capacity(w.T, w.E, w.k, w.cf)
    tok_ref, slot_ref = orc.expert_choice_select(S, C)
    g = device_inputs(name)
    scores = torch.empty((w.T, w.E), dtype=torch.float32, device="cuda")
    slot = torch.empty((w.T, w.E), dtype=torch.int32, device="cuda")
    y = moe.moe_forward_expert_choice(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], w.k, w.cf,
                                      scores=scores, slot=slot)
    torch.cuda.synchronize()
    amb, band = boundary_bands(S, C)
    skip = (band & amb[None, :]).any(axis=1)
    s = host(slot)
    assert np.array_equal(s[~skip], slot_ref[~skip])
    r = orc.expert_choice_forward(a["x"], a["w_router"], a["w_gate"], a["w_up"], a["w_down"], w.k, w.cf, w.dtype,
                                  slot=s)
    rel, mae = assert_close_rows(host(y), r["y"], w.dtype)
    toks = np.arange(w.T)
    print(f"{name}: C={C}, {int(amb.sum())} experts with a near-tie boundary, {int((s != slot_ref).any(1).sum())} "
          f"tokens selected differently, all {len(toks)} tokens, max-rel {rel:.3g}, MAE {mae:.3g}")
