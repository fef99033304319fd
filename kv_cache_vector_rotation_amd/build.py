"""Builds libturboquant.so in-tree with hipcc for gfx950.

Usage: python -m kv_cache_vector_rotation_amd.build  (or build() from Python).
Every call recompiles. The library links only the HIP runtime.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libturboquant.so")
SOURCES = ["tq_host.cpp", "tq_quantize.hip", "tq_decode.hip", "tq_decode_bf16.hip", "tq_search.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 instructions are disabled for all device code: the compiler
# would otherwise form v_pk_*_f32 from ordinary float code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    tmp = os.path.join(HERE, "_build")
    os.makedirs(tmp, exist_ok=True)
    cmds, objs = [], []
    for src in SOURCES:
        obj = os.path.join(tmp, src + ".o")
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
               "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = DEVICE_FLAGS
        else:
            cmd += ["-x", "c++"]
        cmds.append(cmd)
        objs.append(obj)
    # the translation units are independent: compile them side by side
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    out_tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs, verbose)
    os.replace(out_tmp, LIB)
    return LIB


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd)}")


if __name__ == "__main__":
    print(build(verbose=True))
