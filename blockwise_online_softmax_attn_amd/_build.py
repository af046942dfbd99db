"""Build libattn.so (gfx950) from csrc/*.hip with hipcc, and the matrix-core
rate probe (probe/mfma_rate.hip, a stand-alone program bench.py runs as a
yardstick) next to its source.

Every call recompiles.  Objects go to <repo>/_build/, the shared library to
this package directory, where the ctypes binding loads it.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(os.path.dirname(PKG), "_build")
LIB = os.path.join(PKG, "libattn.so")
PROBE_SRC = os.path.join(PKG, "probe", "mfma_rate.hip")
PROBE = os.path.join(PKG, "probe", "mfma_rate")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
# Packed fp32 VALU ops are disabled (hipcc otherwise forms v_pk_*_f32 from
# scalar float code); the host pass warns that it does not know the feature.
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l and "--hip-link" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(SRC) if f.endswith(".hip"))
    jobs = []
    for f in srcs:
        obj = os.path.join(BUILD, f[:-4] + ".o")
        jobs.append((obj, [HIPCC, *CFLAGS, "-c", os.path.join(SRC, f), "-o", obj]))
    jobs.append((PROBE + ".tmp", [HIPCC, *CFLAGS, "-o", PROBE + ".tmp", PROBE_SRC]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for (obj, cmd), warn in zip(jobs, ex.map(lambda j: _run(j[1]), jobs)):
            if verbose and warn.strip():
                print(warn, file=sys.stderr)
    shutil.move(PROBE + ".tmp", PROBE)
    jobs.pop()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in jobs]])
    shutil.move(tmp, LIB)
    if verbose:
        print(f"built {LIB} and {PROBE}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
