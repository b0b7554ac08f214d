"""The C interface's host code under AddressSanitizer and
UndefinedBehaviorSanitizer: every csrc/*.hip is compiled with the host pass
instrumented (the device code is unchanged and never runs here), linked into
a separate libmoe, and tests/test_abi.py runs against it in a child Python
with the sanitizer runtime preloaded. That exercises the argument checks and
the capacity, size and workspace arithmetic of every entry point, including
sizes near the integer limits, on the CPU; any sanitizer report aborts the
child and fails this test."""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_09_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def build_sanitized():
    from sparse_mixture_experts_09_amd.build import FLAGS
    os.makedirs(OUT, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(OUT, os.path.basename(s)[:-4] + ".o") for s in srcs]
    flags = [f for f in FLAGS if f != "-O3"] + ["-O1"]

    def cc(so):
        r = subprocess.run([HIPCC, *flags, *SAN_HOST, "-c", so[0], "-o", so[1]], capture_output=True, text=True)
        assert r.returncode == 0, r.stdout + r.stderr

    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(cc, zip(srcs, objs)))
    lib = os.path.join(OUT, "libmoe_sanitized.so")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-shared-libsan",
                        "-fsanitize=address,undefined", "-o", lib, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return lib


@pytest.mark.skipif(not os.path.exists(HIPCC) or asan_runtime() is None, reason="needs hipcc and the ASan runtime")
def test_abi_under_address_and_undefined_behaviour_sanitizers():
    lib = build_sanitized()
    env = dict(os.environ)
    env.update(MOE_LIBRARY=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-s",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
