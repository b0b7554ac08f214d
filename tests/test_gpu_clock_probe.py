"""The clock probe (a measurement aid of the benchmark): it waits the asked
number of wall-clock ticks and counts a plausible number of core cycles."""
import pytest
import torch

import sparse_mixture_experts_09_amd as moe
from sparse_mixture_experts_09_amd import moe as binding

pytestmark = pytest.mark.gpu


def test_clock_probe_counts_core_cycles():
    khz = binding.moe_wall_clock_khz()
    assert 1_000 <= khz <= 10_000_000
    out = torch.zeros((3, 2), dtype=torch.int64, device="cuda")
    for i, ms in enumerate((0.05, 0.2, 1.0)):
        binding.moe_clock_probe(out[i], int(khz * ms), stream=torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i, ms in enumerate((0.05, 0.2, 1.0)):
        cyc, wall = int(out[i, 0]), int(out[i, 1])
        assert wall >= int(khz * ms)
        mhz = cyc / wall * khz / 1e3
        print(f"probe {ms} ms: {wall} wall ticks, {cyc} core cycles, {mhz:.0f} MHz")
        assert 100 <= mhz <= 3000
