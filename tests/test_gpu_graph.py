"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed:
the library allocates nothing, synchronises nothing and issues no memset, so
the whole layer is one capturable sequence of kernel launches. Every replay,
with eager work and host synchronisations between replays, must give the
eager result bit for bit."""
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_09_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("case,gating,fill", [
    ((300, 256, 8, 2, 320, 1.25, "bf16", 10), "topk_softmax", "token"),
    ((2048, 512, 16, 4, 256, 0.0, "bf16", 31), "softmax_topk_scaled", "priority"),
    ((32, 512, 8, 2, 256, 0.0, "bf16", 21), "topk_softmax", "token"),
    ((200, 100, 5, 2, 72, 0.8, "f32", 14), "topk_softmax", "token"),
], ids=["small", "gather_priority", "decode_sized", "f32"])
def test_forward_graph_replays_equal_eager(case, gating, fill):
    w, a = mi.random_small(*case)
    g = {k: v.cuda() for k, v in a.items() if v is not None}
    T, d, E, k, F, cf = w.T, w.d, w.E, w.k, w.F, w.cf
    ws = torch.empty(moe.moe_workspace_bytes(T, d, E, k, cf, F, g["x"].dtype), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(g["x"])

    def fwd():
        moe.moe_forward(g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"], k, cf, y=y, ws=ws,
                        gating=gating, fill_order=fill)

    fwd()                         # eager first: one-time launch set-up happens outside the capture
    torch.cuda.synchronize()
    ref = y.clone()
    side = torch.cuda.Stream()    # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    torch.cuda.synchronize()
    for i in range(4):
        y.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {i} differs"
        assert torch.isfinite(junk)


@pytest.mark.parametrize("kind", ["backward", "backward_switch_priority", "expert_choice_forward",
                                  "expert_choice_backward", "backward_f32"])
def test_other_layers_graph_replays_equal_eager(kind):
    """The backward passes and the expert-choice layer captured the same way:
    every output of every replay equals the eager call's, bit for bit."""
    case = (200, 100, 5, 2, 72, 0.8, "f32", 14) if kind.endswith("f32") else (300, 256, 8, 2, 320, 1.25, "bf16", 10)
    w, a = mi.random_small(*case)
    g = {k: v.cuda() for k, v in a.items() if v is not None}
    k, cf = w.k, w.cf
    gen = torch.Generator().manual_seed(5)
    dy = torch.randn((w.T, w.d), generator=gen).to(g["x"].dtype).cuda()
    args = (g["x"], g["w_router"], g["w_gate"], g["w_up"], g["w_down"])

    def run():
        if kind in ("backward", "backward_f32"):
            return moe.moe_backward(*args, dy, k, cf)
        if kind == "backward_switch_priority":
            return moe.moe_backward(*args, dy, k, cf, gating="softmax_topk_scaled", fill_order="priority")
        if kind == "expert_choice_forward":
            return {"y": moe.moe_forward_expert_choice(*args, k, cf)}
        return moe.moe_backward_expert_choice(*args, dy, k, cf)

    ref = {n: t.clone() for n, t in run().items()}   # eager first (one-time launch set-up)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()    # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = run()
    torch.cuda.synchronize()
    for i in range(3):
        for t in out.values():
            t.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for n, t in out.items():
            assert torch.equal(t, ref[n]), f"{kind}: {n} differs in replay {i}"
        assert torch.isfinite(junk)
