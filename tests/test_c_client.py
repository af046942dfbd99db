"""The C ABI from C itself: a C99 program (tests/c_client.c) compiled with
gcc -std=c99 -pedantic -Werror against include/attn.h and linked against the
built libattn.so, calling the entry points that make no HIP call (the ring
plan and argument validation), so it runs without a GPU."""
import os
import shutil
import subprocess

import pytest

import blockwise_online_softmax_attn_amd as bosa
from blockwise_online_softmax_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_program_uses_the_header_and_the_library(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib = _lib.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libattn.so not built")
    exe = tmp_path / "c_client"
    libdir = os.path.dirname(lib)
    cmd = [gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_client.c"), "-o", str(exe), "-L", libdir, "-l:" + os.path.basename(lib),
           "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    plan = bosa.attn_ring_plan(131072, 8, 0, True, True)
    assert lines["plan"] == (f"{len(plan)} merges {sum(c.accumulate for c in plan)} first_block {plan[0].block} "
                             f"last_kv_pos0 {plan[-1].kv_pos0}")
    assert lines["rc"] == f"{_lib.ATTN_ERR_UNSUPPORTED} unsupported 1"
    assert "96" in lines["message"]
    assert lines["version"] == str(_lib.load().attn_version())
