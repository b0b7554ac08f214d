"""The allocation-free permutation (moe_permute_noalloc) against moe_permute,
through the C interface: the same routing in, bit-identical counts, offsets,
row maps and permuted rows out, on two calls in a row (the second smaller, so
it runs on the scratch the first one left behind), and the documented error
for a problem whose scratch exceeds the static array."""
import numpy as np
import pytest
import torch

import moe_inputs as mi
import sparse_mixture_experts_09_amd as moe
from sparse_mixture_experts_09_amd import moe as binding

pytestmark = pytest.mark.gpu

# (T, d, E, k, F, cf, dtype, seed): chunked layout (several 256-token chunks,
# ragged last chunk) with capacity drops, then a smaller chunked case with
# more experts, then the one-workgroup layout (T <= 1024)
CASES = [
    (3000, 256, 8, 2, 64, 1.25, "bf16", 31),
    (1300, 128, 32, 4, 64, 1.0, "bf16", 32),
    (700, 64, 16, 2, 64, 0.0, "f32", 33),
]


def outputs(T, d, E, k, cf, dtype, dev):
    R_max = moe.moe_rows_max(T, E, k, cf)
    return dict(expert_counts=torch.full((E,), -7, dtype=torch.int32, device=dev),
                expert_offsets=torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                slot_row=torch.full((T, k), -7, dtype=torch.int32, device=dev),
                row_slot=torch.full((max(R_max, 1),), -7, dtype=torch.int32, device=dev),
                x_perm=torch.full((max(R_max, 1), d), 3.0, dtype=dtype, device=dev))


def test_noalloc_permute_matches_workspace_permute():
    dev = torch.device("cuda:0")
    for (T, d, E, k, F, cf, dt, seed) in CASES:
        print(f"noalloc permute: T={T} d={d} E={E} k={k} cf={cf} {dt}", flush=True)
        w, a = mi.random_small(T, d, E, k, F, cf, dt, seed)
        x = a["x"].to(dev).contiguous()
        wr = a["w_router"].to(dev).contiguous()
        idx, gate, _ = moe.moe_route(x, wr, k)
        ref = moe.moe_permute(x, idx, E, cf)
        got = moe.moe_permute_noalloc(x, idx, E, cf, outputs(T, d, E, k, cf, x.dtype, dev))
        torch.cuda.synchronize()
        R = int(ref["expert_offsets"][E])
        assert R > 0
        if cf > 0:
            assert int(ref["expert_counts"].sum()) == T * k
        for name in ("expert_counts", "expert_offsets", "slot_row"):
            assert torch.equal(got[name], ref[name]), name
        assert torch.equal(got["row_slot"][:R], ref["row_slot"][:R])
        assert torch.equal(got["x_perm"][:R].view(torch.int16 if dt == "bf16" else torch.int32),
                           ref["x_perm"][:R].view(torch.int16 if dt == "bf16" else torch.int32))
        # rows past R are left untouched
        assert bool((got["row_slot"][R:] == -7).all())


def test_noalloc_permute_rejects_too_large():
    """262145 tokens over 256 experts need more than the 1 MiB scratch: the
    host check returns MOE_ERR_WORKSPACE before anything is enqueued."""
    dev = torch.device("cuda:0")
    T, d, E, k, cf = 262145, 8, 256, 1, 0.0
    x = torch.zeros((T, d), dtype=torch.bfloat16, device=dev)
    idx = torch.zeros((T, k), dtype=torch.int32, device=dev)
    with pytest.raises(binding.MoeError) as err:
        moe.moe_permute_noalloc(x, idx, E, cf, outputs(T, d, E, k, cf, x.dtype, dev))
    assert err.value.status == binding.MOE_ERR_WORKSPACE
