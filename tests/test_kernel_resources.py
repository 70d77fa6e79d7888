"""Register, scratch and LDS use of every gfx950 kernel (CPU only: hipcc
cross-compiles).  Each HIP source is compiled with the library's flags and
-Rpass-analysis=kernel-resource-usage; every kernel instantiation must use no
scratch (no register spills, no private arrays in memory) and fit the 160 KB
of LDS a CU has."""
import glob
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from implicit_gemm_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = sorted(glob.glob(os.path.join(ROOT, "implicit_gemm_amd", "csrc", "*.hip")) +
                 glob.glob(os.path.join(ROOT, "implicit_gemm_amd", "probes", "*.hip")))


def _resources(src, tmpdir):
    obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
    cmd = [B.HIPCC] + B.FLAGS + ["-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    kernels = []
    cur = None
    for line in res.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        if cur is None:
            continue
        for key, pat in (("vgpr", r"VGPRs: (\d+)"), ("agpr", r"AGPRs: (\d+)"),
                         ("scratch", r"ScratchSize \[bytes/lane\]: (\d+)"),
                         ("lds", r"LDS Size \[bytes/block\]: (\d+)"), ("occupancy", r"Occupancy \[waves/SIMD\]: (\d+)")):
            m = re.search(pat, line)
            if m:
                cur[key] = int(m.group(1))
    return kernels


def test_every_kernel_has_no_scratch_and_fits_lds(tmp_path):
    with ThreadPoolExecutor(8) as ex:
        per_src = list(ex.map(lambda s: (s, _resources(s, str(tmp_path))), SOURCES))
    total = 0
    for src, kernels in per_src:
        kernels = [k for k in kernels if "kernel" in k["name"]]
        if os.path.basename(src) != "noalloc.hip":   # the library-owned workspace array only
            assert kernels, "no kernel remarks for %s" % src
        for k in kernels:
            total += 1
            assert k.get("scratch", -1) == 0, (os.path.basename(src), k)
            assert k.get("lds", 0) <= 160 * 1024, (os.path.basename(src), k)
            assert k.get("occupancy", 0) >= 1, (os.path.basename(src), k)
    print("kernel instantiations checked:", total)
    assert total >= 100
