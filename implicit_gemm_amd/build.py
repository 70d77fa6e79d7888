"""Compile the gfx950 weight-gradient library (libconvwgrad.so) in-tree with hipcc,
and beside it the measurement probes (libcwprobes.so, not part of the C ABI).

    python -m implicit_gemm_amd.build
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libconvwgrad.so")
PROBES_DIR = os.path.join(HERE, "probes")
PROBES_LIB = os.path.join(PROBES_DIR, "libcwprobes.so")
OBJ_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    # No packed-fp32 VALU instructions in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.cpp")) + glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s%s" % (src, res.stdout, res.stderr))
    return obj


def _link(objs, out):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s%s" % (res.stdout, res.stderr))
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source, link libconvwgrad.so and libcwprobes.so; returns the library path."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    probe_srcs = sorted(glob.glob(os.path.join(PROBES_DIR, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(probe_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBES_LIB)
    if verbose:
        print("built", LIB, "and", PROBES_LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
