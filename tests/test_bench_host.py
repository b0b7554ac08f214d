"""Host-side contract of bench.py: no multi-GPU runs, and the HBM-traffic field only
while the counters describe the kernel that is built (the GEMM file and every header
it includes unchanged)."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_digest_covers_the_included_headers():
    names = [os.path.basename(p) for p in bench.DOMINANT_KERNEL_SRC]
    assert names[0] == "ffn_bf16.hip"
    src = open(bench.DOMINANT_KERNEL_SRC[0]).read()
    included = [line.split('"')[1] for line in src.splitlines() if line.startswith('#include "')]
    assert included and set(included) <= set(names[1:])


@pytest.mark.parametrize("workload", ["mixtral_bf16", "decode_bf16"])
def test_traffic_only_for_the_sources_it_was_taken_on(workload, tmp_path, monkeypatch):
    with open(os.path.join(ROOT, "profiles", f"traffic_gate_up_{workload}.json")) as f:
        rec = json.load(f)
    # the committed counters describe the committed sources
    assert rec["source_sha256"] == bench.source_digest(bench.DOMINANT_KERNEL_SRC)
    assert bench.load_traffic(workload) == pytest.approx(rec["bytes_per_launch"])
    # a change to any one of the files, the headers included, drops the field
    copies = []
    for p in bench.DOMINANT_KERNEL_SRC:
        q = tmp_path / os.path.basename(p)
        shutil.copyfile(p, q)
        copies.append(str(q))
    monkeypatch.setattr(bench, "DOMINANT_KERNEL_SRC", copies)
    assert bench.load_traffic(workload) == pytest.approx(rec["bytes_per_launch"])
    for q in copies:
        orig = open(q).read()
        with open(q, "a") as f:
            f.write("\n// changed\n")
        assert bench.load_traffic(workload) is None, q
        with open(q, "w") as f:
            f.write(orig)
    assert bench.load_traffic(workload) == pytest.approx(rec["bytes_per_launch"])
