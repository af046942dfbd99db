"""The library's host logic under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU).

api.hip -- argument validation, the ring-share plan, dead sub-call pruning,
scratch layout and the parameters each kernel launch receives -- is compiled
host-only with both sanitizers and linked with tests/host_asan_driver.cpp,
which stands in for the HIP runtime calls and for every kernel launcher (each
stand-in touches every row its kernel would read or write).  The driver runs
invalid-argument cases, every entry point on small ragged shapes, ring plans
for P up to 8 (every rank, both placements, with and without causal order,
windows and ALiBi), scratch sizes against the formulas of include/attn.h, and
allocation and launch failures.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"
# host-only translation units: the sanitizer flags apply to host code only
FLAGS = ["--cuda-host-only", "-x", "hip", "-O1", "-g", "-std=c++17",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=undefined"]


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="ROCm toolchain not installed")
def test_host_logic_under_asan_and_ubsan(tmp_path):
    objs = []
    for src, name in ((os.path.join(ROOT, "blockwise_online_softmax_attn_amd", "csrc", "api.hip"), "api.o"),
                      (os.path.join(ROOT, "tests", "host_asan_driver.cpp"), "driver.o")):
        obj = str(tmp_path / name)
        r = subprocess.run([HIPCC, *FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "harness")
    r = subprocess.run([CLANG, "-fsanitize=address,undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0 and "all checks passed" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
