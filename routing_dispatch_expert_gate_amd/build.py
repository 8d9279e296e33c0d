"""Build ``libmoe.so`` (gfx950) in-tree with hipcc.

Every HIP source under ``csrc/`` is compiled for gfx950 only and linked into
one shared library next to this file.  Packed fp32 instructions are disabled
(``-packed-fp32-ops``) and fp32 division and square root are correctly
rounded, which the per-token int8 quantisation relies on for bit-exact codes.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmoe.so")
# bench-only diagnostics (a dense MFMA loop), outside the library's ABI
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
ARCH = "gfx950"

SOURCES = ["route.hip", "align.hip", "ffn.hip", "combine.hip", "moe_api.cpp"]
PROBE_SOURCES = ["probe.hip"]

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-x", "hip", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the MoE library needs ROCm's hipcc to build")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(jobs: int | None = None) -> str:
    """Compile every source and link ``libmoe.so`` (and the bench-only
    ``libmoe_probe.so``); returns the path of ``libmoe.so``."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        _run([hipcc, *CFLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    srcs = SOURCES + PROBE_SOURCES
    n = jobs or min(len(srcs), max(1, (os.cpu_count() or 2)))
    with ThreadPoolExecutor(n) as ex:
        objs = dict(zip(srcs, ex.map(compile_one, srcs)))
    for lib, names in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *(objs[s] for s in names)])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
