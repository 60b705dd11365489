"""Builds libringsim.so in-tree with hipcc for gfx950.

Usage: python -m ring_all_reduce_allreduce_amd.build [--verbose]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libringsim.so")
# (source, object name, extra defines): the line kernel's instantiation unit
# is compiled once per line mode.
SOURCES = [
    ("ringsim_api.hip", "ringsim_api", []),
    ("ring_bulk.hip", "ring_bulk", []),
    ("ring_lines_inst.hip", "ring_lines_half", ["-DRINGSIM_LINE_MODE=kLinesHalf", "-DRINGSIM_LINE_NAME=half"]),
    ("ring_lines_inst.hip", "ring_lines_one", ["-DRINGSIM_LINE_MODE=kLinesOne", "-DRINGSIM_LINE_NAME=one"]),
    ("ring_lines_inst.hip", "ring_lines_multi", ["-DRINGSIM_LINE_MODE=kLinesMulti", "-DRINGSIM_LINE_NAME=multi"]),
    ("tree.hip", "tree", []),
    ("copy.hip", "copy", []),
]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming packed fp32 instructions.
# -ffp-contract=off: every hop is one rounded add or multiply, never fused.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libringsim")


def build(verbose: bool = False) -> str:
    """Compiles every source to an object, links libringsim.so, returns its path."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="ringsim_build_") as tmp:
        objs = []
        procs = []
        for src, name, defines in SOURCES:
            obj = os.path.join(tmp, name + ".o")
            cmd = [cc, *HIP_FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((name, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            out, _ = p.communicate()
            if out and (verbose or p.returncode):
                sys.stderr.write(out)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError(f"hipcc failed for {failed}")
        tmp_lib = LIB + ".tmp"
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_lib, *objs]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp_lib, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
