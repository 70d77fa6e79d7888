"""The C-ABI library without a GPU: exported symbols, validation errors and the
planner (pure host integer code reached through conv_wgrad_get_plan)."""
import ctypes
import glob
import json
import os
import sys
import re
import subprocess

import numpy as np
import pytest

import implicit_gemm_amd as iga

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "conv_wgrad.h")
PROBES_HEADER = os.path.join(ROOT, "implicit_gemm_amd", "probes", "probes.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")


PUBLIC_FUNCTIONS = {"conv_wgrad", "conv_wgrad_ex", "conv_wgrad_get_plan", "conv_wgrad_timed",
                    "conv_wgrad_status_string", "conv_wgrad_workspace_size", "conv_wgrad_bias",
                    "conv_wgrad_bias_timed", "conv_wgrad_noalloc", "conv_wgrad2_workspace_size",
                    "conv_wgrad2_get_plan", "conv_wgrad2", "conv_wgrad2_timed", "conv_wgrad2_call_timed", "conv_igemm_get_plan",
                    "conv_igemm_workspace_size", "conv_fwd", "conv_dgrad", "conv_igemm_call_timed"}


def declared_functions(header=HEADER, prefix="conv_"):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(%s\w*)\s*\(" % prefix, text)))


def exported_symbols(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return set(re.findall(r"\s[TW]\s(\w+)$", out, flags=re.M))


def test_library_loads_and_exports_every_declared_symbol():
    lib = iga.load()
    headers = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
    assert headers == [HEADER]
    names = declared_functions()
    assert set(names) == PUBLIC_FUNCTIONS
    for n in names:
        assert hasattr(lib, n), n
    exported = exported_symbols(iga.LIB_PATH)
    assert set(names) <= exported
    # The measurement probes live in their own library, not in the product's ABI.
    assert not any("probe" in n or "peak" in n for n in exported if n.startswith("conv_"))


def test_probe_library_exports_its_declared_symbols():
    from implicit_gemm_amd import probes
    lib = probes.load()
    names = declared_functions(PROBES_HEADER, prefix="cwprobe")
    assert set(names) == {"cwprobe_read", "cwprobe_mfma", "cwprobe_mfma16", "cwprobe_lds"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= exported_symbols(probes.LIB_PATH)


def test_struct_sizes_match_header_layout():
    # 11 int64 + 2 int32; plan: see conv_wgrad_plan_t field order.
    assert ctypes.sizeof(iga.Desc) == 11 * 8 + 2 * 4
    assert ctypes.sizeof(iga.Plan) == 8 + 8 * 7 + 4 + 4 + 8 * 3 + 8 * 4 + 8
    # desc2: 14 int64 + 4 int32; plan2: plan + 2 int32
    assert ctypes.sizeof(iga.Desc2) == 14 * 8 + 4 * 4
    assert ctypes.sizeof(iga.Plan2) == ctypes.sizeof(iga.Plan) + 8


def test_peak_probe_argument_errors():
    # Validation happens before any launch, so no GPU is needed.
    from implicit_gemm_amd import probes
    lib = probes.load()
    fake = ctypes.c_void_p(0x10000)
    assert lib.cwprobe_read(None, 16, 1, fake, None, None, None) == 1          # NULL_ARG
    assert lib.cwprobe_read(fake, 16, 1, None, None, None, None) == 1
    for nbytes, blocks in ((0, 1), (-16, 1), (24, 1), (16, 0), (16, 65537)):
        assert lib.cwprobe_read(fake, nbytes, blocks, fake, None, None, None) == 2  # BAD_SHAPE
    assert lib.cwprobe_read(ctypes.c_void_p(0x10008), 16, 1, fake, None, None, None) == 6
    assert lib.cwprobe_mfma(0, 1, 1, None, None, None, None) == 1
    for dtype in (3, -1):
        assert lib.cwprobe_mfma(dtype, 1, 1, fake, None, None, None) == 3       # BAD_DTYPE
    for iters, blocks in ((0, 1), (1 << 31, 1), (1, 0), (1, 65537)):
        assert lib.cwprobe_mfma(0, iters, blocks, fake, None, None, None) == 2
        assert lib.cwprobe_mfma16(iters, blocks, fake, None, None, None) == 2
        assert lib.cwprobe_lds(0, iters, blocks, fake, None, None, None) == 2
    assert lib.cwprobe_mfma16(1, 1, None, None, None, None) == 1
    assert lib.cwprobe_lds(1, 1, 1, None, None, None, None) == 1
    for mode in (-1, 3):
        assert lib.cwprobe_lds(mode, 1, 1, fake, None, None, None) == 2


def test_status_strings():
    lib = iga.load()
    for code in range(9):
        s = lib.conv_wgrad_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.conv_wgrad_status_string(99).decode() == "unknown status"


def D(**kw):
    base = dict(N=2, C=8, H=8, W=8, K=4, R=3, S=3, pad=1, stride=1, dilation=1, groups=1,
                dtype=iga.F32, split_k=-1)
    base.update(kw)
    return iga.make_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), 2), (dict(C=0), 2), (dict(H=0), 2), (dict(W=-1), 2), (dict(K=0), 2),
    (dict(R=0), 2), (dict(S=0), 2), (dict(pad=-1), 2), (dict(stride=0), 2),
    (dict(dilation=0), 2), (dict(groups=0), 2), (dict(groups=3), 2), (dict(C=6, K=4, groups=3), 2),
    (dict(H=2, R=5, pad=0), 2), (dict(W=2, S=3, dilation=2, pad=0), 2),
    (dict(dtype=3), 3), (dict(dtype=-1), 3),
    (dict(split_k=0), 4), (dict(split_k=-2), 4), (dict(split_k=-100), 4),
    (dict(N=1 << 40, C=1 << 20, H=1 << 20, W=1 << 20), 2),
    (dict(H=1 << 16, W=1 << 16, C=1024), 5),
])
def test_invalid_desc_is_rejected_before_any_launch(kw, code):
    d = D(**kw)
    with pytest.raises(iga.ConvWgradError) as ei:
        iga.get_plan(d)
    assert ei.value.status == code
    with pytest.raises(iga.ConvWgradError) as ei:
        iga.workspace_size(d)
    assert ei.value.status == code
    lib = iga.load()
    # conv_wgrad itself validates before touching pointers or the GPU.
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, 16, 16, None) == code


def test_null_arguments():
    lib = iga.load()
    d = D()
    assert lib.conv_wgrad(None, 16, 16, 16, 16, None) == 1
    assert lib.conv_wgrad(ctypes.byref(d), None, 16, 16, 16, None) == 1
    assert lib.conv_wgrad(ctypes.byref(d), 16, None, 16, 16, None) == 1
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, None, 16, None) == 1
    assert lib.conv_wgrad_get_plan(ctypes.byref(d), None) == 1
    assert lib.conv_wgrad_workspace_size(ctypes.byref(d), None) == 1
    # A plan with several slices needs a workspace.
    d = D(N=8, H=32, W=32, split_k=4)
    assert iga.get_plan(d).ks_count > 1
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, 16, None, None) == 1
    # The bias entry point: db is required; the rest as conv_wgrad_ex.
    ws = iga.workspace_size(d)
    assert lib.conv_wgrad_bias(ctypes.byref(d), 16, 16, 16, None, 16, ws, None) == 1
    assert lib.conv_wgrad_bias(ctypes.byref(d), 16, 16, None, 16, 16, ws, None) == 1
    assert lib.conv_wgrad_bias(ctypes.byref(d), 16, 16, 16, 16, None, ws, None) == 1
    assert lib.conv_wgrad_bias_timed(ctypes.byref(d), 16, 16, 16, None, 16, ws, None, None, None) == 1
    assert lib.conv_wgrad_noalloc(ctypes.byref(d), None, 16, 16, None, None) == 1
    assert lib.conv_wgrad_noalloc(ctypes.byref(d), 16, 16, None, 16, None) == 1
    assert lib.conv_wgrad_noalloc(None, 16, 16, 16, None, None) == 1


def test_misaligned_and_small_workspace():
    lib = iga.load()
    d = D(N=8, H=32, W=32, split_k=4)
    ws = iga.workspace_size(d)
    assert ws > 0
    assert lib.conv_wgrad(ctypes.byref(d), 18, 16, 16, 16, None) == 6
    assert lib.conv_wgrad(ctypes.byref(d), 16, 20, 16, 16, None) == 6
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, 24, 16, None) == 6
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, 16, 8, None) == 6
    assert lib.conv_wgrad_ex(ctypes.byref(d), 16, 16, 16, 16, ws - 1, None) == 7
    assert lib.conv_wgrad_bias(ctypes.byref(d), 16, 16, 16, 40, 16, ws, None) == 6
    assert lib.conv_wgrad_bias(ctypes.byref(d), 16, 16, 16, 16, 16, ws - 1, None) == 7


def check_plan_invariants(d, p):
    """Every plan: exact ceil-division slices covering all units, no empty slice."""
    Ho = (d.H + 2 * d.pad - d.dilation * (d.R - 1) - 1) // d.stride + 1
    Wo = (d.W + 2 * d.pad - d.dilation * (d.S - 1) - 1) // d.stride + 1
    assert (p.Ho, p.Wo) == (Ho, Wo)
    assert p.L == d.N * Ho * Wo
    assert p.E == d.K * d.R * d.S * (d.C // d.groups)
    if p.path == iga.PATH_DENSE and p.variant == 3 and p.unit_rows > Wo:   # units of ru whole rows
        ru = p.unit_rows // Wo
        assert p.unit_rows == ru * Wo and ru >= 2 and ru * (Wo + min(d.S, 4) - 1) <= 64
        assert p.units == d.N * -(-Ho // ru)
    elif p.path == iga.PATH_DENSE and p.variant in (5, 6):   # all-taps kernel: ru whole rows, ru = 64 // (Wo + 2)
        ru = 64 // (Wo + 2)
        assert d.R == d.S == 3 and d.stride == d.dilation == 1 and ru >= 1
        assert p.unit_rows == ru * Wo and p.units == d.N * -(-Ho // ru)
    elif (p.path == iga.PATH_DENSE and p.variant == 1 and d.stride == d.dilation == 1 and Wo <= 14
          and Wo + min(d.S, 4) - 1 <= 16):
        # fp32 row kernel, packed rows: units of 4 whole output rows
        assert p.unit_rows == 4 * Wo and p.units == d.N * -(-Ho // 4)
    elif p.path == iga.PATH_DENSE and p.variant in (1, 3):   # row units: (n, ho, chunk of Wo)
        assert p.units == d.N * Ho * -(-Wo // p.unit_rows)
    elif p.variant in (12, 13):                       # depthwise, row-streaming grouped: one output row per unit
        assert p.units == d.N * Ho and p.unit_rows == Wo
    elif p.variant == 11:                             # units of ru rows x 32 pixels
        ru = p.unit_rows // 32
        assert p.units == d.N * -(-Ho // ru) * -(-Wo // 32)
    else:
        assert p.units == -(-p.L // p.unit_rows)
    ups, ks = p.units_per_slice, p.ks_count
    assert ks >= 1 and ups >= 1
    if p.variant == 12 and 2 <= ks <= 256:
        # depthwise slices balanced by staging steps: ups is the longest slice
        assert ks * ups >= p.units and ups >= -(-p.units // ks) and ks <= p.units
    else:
        assert (ks - 1) * ups < p.units <= ks * ups       # last slice non-empty, all covered
        assert ks == -(-p.units // ups)
    if d.split_k >= 1:
        assert ks <= d.split_k
        assert ups == -(-p.units // min(d.split_k, p.units))
    assert p.needs_reduce == (1 if ks > 1 else 0)
    if p.variant in (12, 13):   # one workgroup per (slice, 64-channel block)
        assert p.tiles == -(-d.C // 64)
    assert p.grid == p.tiles * ks
    # a slab: the dW partial, then the db partial from the next 16-byte boundary
    assert p.slab_stride % 64 == 0 and p.slab_stride >= -(-p.E // 4) * 4 + d.K
    assert p.ws_bytes == (ks * p.slab_stride * 4 if ks > 1 else 0)
    esz = 4 if d.dtype == iga.F32 else 2
    assert p.x_bytes == d.N * d.H * d.W * d.C * esz
    assert p.dy_bytes == d.N * Ho * Wo * d.K * esz
    assert p.windows_4g == -(-max(p.x_bytes, p.dy_bytes) // (1 << 32))


def test_planner_random_descs():
    rng = np.random.default_rng(7)
    for _ in range(3000):
        groups = int(rng.choice([1, 1, 2, 4, 8, 32]))
        C = groups * int(rng.integers(1, 12))
        K = groups * int(rng.integers(1, 12))
        H, W = int(rng.integers(1, 80)), int(rng.integers(1, 80))
        R, S = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        pad, stride, dil = int(rng.integers(0, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
        if (H + 2 * pad - dil * (R - 1) - 1) < 0 or (W + 2 * pad - dil * (S - 1) - 1) < 0:
            continue
        split = int(rng.choice([-1, 1, 2, 3, 7, 64, 1000]))
        d = iga.make_desc(int(rng.integers(1, 40)), C, H, W, K, R, S, pad, stride, dil, groups,
                          int(rng.integers(0, 3)), split)
        check_plan_invariants(d, iga.get_plan(d))


def test_planner_large_tensor_geometry_sweep():
    """The 1x1 96->64 conv on 512x512 images of the MIOpen ticket, N = 1..256, without allocation."""
    g = json.load(open(os.path.join(GOLDEN, "p1_ticket.json")))
    c = g["conv"]
    img_x = c["H"] * c["W"] * c["C"] * 4
    img_dy = c["H"] * c["W"] * c["K"] * 4
    for N in range(1, 257):
        d = iga.make_desc(N, c["C"], c["H"], c["W"], c["K"], 1, 1, split_k=-1)
        p = iga.get_plan(d)
        check_plan_invariants(d, p)
        assert p.x_bytes == N * img_x and p.dy_bytes == N * img_dy
        for split in (1, 5, 43, 1000):
            d2 = iga.make_desc(N, c["C"], c["H"], c["W"], c["K"], 1, 1, split_k=split)
            check_plan_invariants(d2, iga.get_plan(d2))
    lo, hi = g["sweep_range"]
    # Every sweep point past the first 4 GiB window; the ticket's dY is exactly 2^32 bytes.
    for N in g["sweep_points"]:
        assert lo <= N <= hi
        p = iga.get_plan(iga.make_desc(N, c["C"], c["H"], c["W"], c["K"], 1, 1))
        assert p.x_bytes > 1 << 32
        assert p.windows_4g == -(-(N * img_x) // (1 << 32))
        # A truncating quotient would claim one window fewer than the tensor spans.
        assert p.windows_4g == (N * img_x + (1 << 32) - 1) // (1 << 32)
        assert p.windows_4g > (N * img_x) // (1 << 32) or (N * img_x) % (1 << 32) == 0
    p = iga.get_plan(iga.make_desc(g["ticket_batch"], c["C"], c["H"], c["W"], c["K"], 1, 1))
    assert p.dy_bytes == 1 << 32
    assert p.windows_4g == 2
    assert p.x_bytes == g["ticket_batch"] * 96 * 512 * 512 * 4


def test_split_pinning_and_auto():
    d = D(N=32, C=64, H=56, W=56, K=64, split_k=1)
    p = iga.get_plan(d)
    assert p.ks_count == 1 and p.needs_reduce == 0 and p.ws_bytes == 0
    assert iga.workspace_size(d) == 0
    for ks in (2, 3, 7, 64):
        p = iga.get_plan(D(N=32, C=64, H=56, W=56, K=64, split_k=ks))
        assert p.ks_count == ks
    # More slices than units: every slice keeps at least one unit.
    p = iga.get_plan(D(N=1, H=2, W=2, R=1, S=1, pad=0, split_k=1000))
    assert p.ks_count == p.units
    # Auto: the row kernel's 256-lane form (two workgroups per CU) when the
    # split reaches 1.5 workgroups per CU, else the 512-lane form (one per CU);
    # rows of at most 14 pixels: packed rows, about 768 workgroups.
    pa = iga.get_plan(D(N=32, C=64, H=56, W=56, K=64, split_k=-1))
    assert pa.variant == 1 and 384 <= pa.grid <= 512
    pb = iga.get_plan(D(N=8, C=512, H=14, W=14, K=512, split_k=-1))
    assert pb.variant == 1 and pb.unit_rows == 4 * 14 and (pb.ks_count, pb.grid) == (4, 768)
    pc = iga.get_plan(D(N=8, C=512, H=16, W=16, K=512, split_k=-1))   # Wo = 16: one-row units
    assert pc.variant == 1 and pc.unit_rows == 16 and pc.grid <= 256
    # Launch-bound (2 * L * E <= 2^20 FLOP, automatic split): one launch on the
    # general kernel, no fold, no workspace; a pinned split is honoured.
    tiny = D(N=2, C=8, H=8, W=8, K=4, R=1, S=1, pad=0, split_k=-1)
    pt = iga.get_plan(tiny)
    assert (pt.variant, pt.ks_count, pt.needs_reduce, pt.ws_bytes, pt.grid) == (0, 1, 0, 0, 1)
    assert iga.get_plan(D(N=2, C=8, H=8, W=8, K=4, R=1, S=1, pad=0, split_k=4)).ks_count == 4
    # just past the bound: the automatic split is back
    big = iga.get_plan(D(N=8, C=64, H=8, W=8, K=64, R=3, S=3, pad=1, split_k=-1))
    assert 2 * big.L * big.E > (1 << 20) and big.variant == 1


def test_one_hip_runtime_when_the_library_loads_first():
    """Loading the library before torch must not leave two HIP runtimes in the process.

    torch's bundled runtime and ROCm's share a soname but torch asks for it by
    another name; if the library pulled in ROCm's copy first, torch would load a
    second one and its streams would be foreign to the library's launches.
    """
    import subprocess
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import implicit_gemm_amd as iga\n"
        "iga.load()\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read().split('\\n')\n"
        "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
        "print(len(paths), paths)\n" % ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.split()[0] == "1", out.stdout


def test_launch_lane_limits_are_rejected_before_launch():
    """A launch holds fewer than 2^32 lanes: a plan whose slab fold would need more
    (E = 12288 * 9 * 12288 dW elements folded by 256-lane workgroups of 64
    elements) is UNSUPPORTED, while the same problem with one slice (no fold) plans."""
    lib = iga.load()
    big = dict(N=1, C=12288, H=8, W=8, K=12288, R=3, S=3, pad=1)
    p = iga.get_plan(D(split_k=1, **big))
    assert p.ks_count == 1 and p.E == 12288 * 9 * 12288
    d = D(split_k=2, **big)
    assert (p.E // 64) * 256 >= 1 << 32
    plan = iga.Plan()
    assert lib.conv_wgrad_get_plan(ctypes.byref(d), ctypes.byref(plan)) == 5
    n = ctypes.c_size_t(0)
    assert lib.conv_wgrad_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 5
    assert lib.conv_wgrad(ctypes.byref(d), 16, 16, 16, 16, None) == 5


def test_row_kernel_lane_offsets_stay_32_bit():
    """The row-unit kernels address a unit's 64 dY pixels with 32-bit lane offsets:
    a channel count that would carry the last pixel's offset past 2^30 bytes must not
    reach them (the general kernel, 64-bit addressed, takes the shape instead)."""
    ok = iga.get_plan(D(N=1, C=4, H=1, W=1, K=4194300, R=1, S=1, pad=0))
    assert ok.variant == 1                     # 64 * K * 4 < 2^30: the row kernel
    over = iga.get_plan(D(N=1, C=4, H=1, W=1, K=4194308, R=1, S=1, pad=0))
    assert 64 * 4194308 * 4 > (1 << 30) - 1
    assert over.variant == 0                   # the general LDS kernel
    # 16-bit: X columns reach (W + 2 pad + S + 96) pixels of C channels (a pinned
    # split: with an automatic one this tiny problem runs unsplit on the general kernel)
    ok16 = iga.get_plan(D(N=1, C=8, H=1, W=1, K=8, R=1, S=1, pad=0, dtype=iga.BF16, split_k=1))
    assert ok16.variant == 3
    c_over = -(-((1 << 30)) // (2 * (1 + 1 + 96))) + 8
    c_over += (-c_over) % 8
    over16 = iga.get_plan(D(N=1, C=c_over, H=1, W=1, K=8, R=1, S=1, pad=0, dtype=iga.BF16, split_k=1))
    assert over16.variant != 3


def D2(**kw):
    base = dict(N=2, C=8, H=8, W=8, K=4, R=3, S=3, pad=1, stride=1, dilation=1, groups=1,
                dtype=iga.F32, split_k=-1, math="exact", fold_width=-1)
    base.update(kw)
    return iga.make_desc2(**base)


def _status2(d):
    plan = iga.Plan2()
    return iga.load().conv_wgrad2_get_plan(ctypes.byref(d), ctypes.byref(plan))


@pytest.mark.parametrize("kw,code", [
    (dict(pad=(-1, 0)), 2), (dict(pad=(0, -1)), 2), (dict(stride=(0, 1)), 2), (dict(stride=(1, 0)), 2),
    (dict(dilation=(1, 0)), 2), (dict(dilation=(0, 1)), 2),
    (dict(W=2, S=3, pad=(1, 0)), 2),                 # Wo < 1 from the column geometry
    (dict(H=2, R=3, pad=(0, 1)), 2),                 # Ho < 1 from the row geometry
    (dict(math=2), 3), (dict(math=-1), 3),
    (dict(fold_width=-2), 2),
    (dict(fold_width=2, S=3), 2),                    # 2 does not divide S
    (dict(fold_width=2, S=2, pad=0, stride=2, groups=2), 2),     # groups
    (dict(fold_width=2, S=2, pad=0, stride=2, dilation=(1, 2)), 2),  # column dilation
    (dict(fold_width=2, S=2, pad=(0, 1), stride=2), 2),  # 2 does not divide pad_w
    (dict(fold_width=2, S=2, pad=0, stride=2, W=7), 2),  # 2 does not divide W
    (dict(split_k=0), 4),
])
def test_desc2_invalid_is_rejected(kw, code):
    lib = iga.load()
    d = D2(**kw)
    assert _status2(d) == code
    n = ctypes.c_size_t(0)
    assert lib.conv_wgrad2_workspace_size(ctypes.byref(d), ctypes.byref(n)) == code
    assert lib.conv_wgrad2(ctypes.byref(d), 16, 16, 16, None, 16, 1 << 30, None) == code


def test_desc2_null_arguments():
    lib = iga.load()
    d = D2()
    ws = iga.get_plan2(d).base.ws_bytes
    assert lib.conv_wgrad2(None, 16, 16, 16, None, 16, ws, None) == 1
    assert lib.conv_wgrad2(ctypes.byref(d), None, 16, 16, None, 16, ws, None) == 1
    assert lib.conv_wgrad2(ctypes.byref(d), 16, None, 16, None, 16, ws, None) == 1
    assert lib.conv_wgrad2(ctypes.byref(d), 16, 16, None, None, 16, ws, None) == 1
    assert lib.conv_wgrad2_get_plan(ctypes.byref(d), None) == 1
    assert lib.conv_wgrad2_workspace_size(ctypes.byref(d), None) == 1


def test_desc2_equal_axes_plan_equals_plain_plan():
    """An extended descriptor with equal axes, exact math and the automatic fold
    plans exactly as the plain descriptor."""
    rng = np.random.default_rng(5)
    fields = [n for n, _ in iga.Plan._fields_]
    for _ in range(400):
        groups = int(rng.choice([1, 2, 4, 16]))
        C, K = groups * int(rng.integers(1, 9)), groups * int(rng.integers(1, 9))
        H, W = int(rng.integers(3, 40)), int(rng.integers(3, 40))
        R, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        pad, stride, dil = int(rng.integers(0, 2)), int(rng.integers(1, 3)), int(rng.integers(1, 3))
        if H + 2 * pad - dil * (R - 1) - 1 < 0 or W + 2 * pad - dil * (S - 1) - 1 < 0:
            continue
        dt, sk = int(rng.integers(0, 3)), int(rng.choice([-1, 1, 3]))
        N = int(rng.integers(1, 9))
        a = iga.get_plan(iga.make_desc(N, C, H, W, K, R, S, pad, stride, dil, groups, dt, sk))
        b = iga.get_plan2(iga.make_desc2(N, C, H, W, K, R, S, pad, stride, dil, groups, dt, sk))
        assert [getattr(a, f) for f in fields] == [getattr(b.base, f) for f in fields]


def test_per_axis_plans_route_to_per_axis_kernels():
    """Unequal axes reach only the kernels that take per-axis geometry (dense rows,
    16-bit dense rows, the general dense kernel, the element kernel), and the plan's
    extents follow the row and column geometry."""
    rng = np.random.default_rng(9)
    per_axis_variants = {0, 1, 3, 4, 5, 6, 10}
    seen = set()
    for _ in range(1500):
        groups = int(rng.choice([1, 1, 2, 8, 32]))
        C, K = groups * int(rng.integers(1, 9)), groups * int(rng.integers(1, 9))
        H, W = int(rng.integers(1, 60)), int(rng.integers(1, 60))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        ph, pw = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        sh, sw = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        dh, dw = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        Ho = (H + 2 * ph - dh * (R - 1) - 1)
        Wo = (W + 2 * pw - dw * (S - 1) - 1)
        if Ho < 0 or Wo < 0 or (ph == pw and sh == sw and dh == dw):
            continue
        d = iga.make_desc2(int(rng.integers(1, 9)), C, H, W, K, R, S, (ph, pw), (sh, sw), (dh, dw), groups,
                           int(rng.integers(0, 3)), int(rng.choice([-1, 2])), "exact", 0)
        p = iga.get_plan2(d)
        assert p.fold_width == 1
        assert p.base.variant in per_axis_variants, (d.pad_h, d.pad_w, p.base.variant)
        assert (p.base.Ho, p.base.Wo) == (Ho // sh + 1, Wo // sw + 1)
        seen.add(p.base.variant)
    assert {0, 1, 10} <= seen
    # per-axis padding alone keeps the 16-bit row kernel (and BF16x3 for fp32)
    p = iga.get_plan2(iga.make_desc2(4, 64, 20, 24, 64, 3, 5, (1, 2), 1, 1, 1, iga.BF16))
    assert p.base.variant == 3 and (p.base.Ho, p.base.Wo) == (20, 24)
    p = iga.get_plan2(iga.make_desc2(4, 64, 20, 24, 64, 3, 5, (1, 2), 1, 1, 1, iga.F32, -1, "bf16x3"))
    assert p.base.variant == iga.VARIANT_DENSE_BF16X3


def test_width_fold_plans():
    """The width fold: automatic for a 16x16 stride-16 patch embedding with C = 3
    (f = 16: 48 channels, one filter column), off on request, explicit f checked;
    the folded plan keeps the tensor sizes and dW elements of the original."""
    base = dict(N=2, C=3, H=224, W=224, K=768, R=16, S=16, pad=0, stride=16)
    auto = iga.get_plan2(D2(**base))
    off = iga.get_plan2(D2(fold_width=0, **base))
    f4 = iga.get_plan2(D2(fold_width=4, **base))
    assert auto.fold_width == 16 and off.fold_width == 1 and f4.fold_width == 4
    for p in (auto, off, f4):
        assert p.base.E == 768 * 16 * 16 * 3 and (p.base.Ho, p.base.Wo) == (14, 14)
        assert p.base.x_bytes == 2 * 224 * 224 * 3 * 4 and p.base.dy_bytes == 2 * 14 * 14 * 768 * 4
    # the general kernel both ways: scalar channel loads unfolded, 4-wide folded
    assert off.base.variant == 0 and auto.base.variant == 0
    # 2x2 stride 2, C = 6: f = 2 makes 12 channels
    p = iga.get_plan2(D2(N=2, C=6, H=32, W=32, K=16, R=2, S=2, pad=0, stride=2))
    assert p.fold_width == 2
    # channels already in quads: no automatic fold
    assert iga.get_plan2(D2(N=2, C=8, H=32, W=32, K=16, R=2, S=2, pad=0, stride=2)).fold_width == 1
    # per-axis padding divisible by f: 5x4 filter, stride (1, 4), pad (2, 4), W = 36
    p = iga.get_plan2(D2(N=1, C=3, H=10, W=36, K=8, R=5, S=4, pad=(2, 4), stride=(1, 4)))
    assert p.fold_width == 4 and p.base.Wo == (36 + 8 - 4) // 4 + 1


def test_bf16x3_plan_selection():
    """math = BF16X3 takes the BF16x3 kernel where the 16-bit row kernel covers the
    shape (fp32, stride 1, dilation 1, channels in eights) and the exact path
    elsewhere; it never applies to 16-bit inputs."""
    c2 = dict(N=32, C=64, H=56, W=56, K=64, R=3, S=3, pad=1)
    p = iga.get_plan2(D2(math="bf16x3", **c2))
    assert p.math == 1 and p.base.variant == iga.VARIANT_DENSE_BF16X3_TAPS
    assert iga.get_plan2(D2(**c2)).base.variant == 1 and iga.get_plan2(D2(**c2)).math == 0
    # 5x5: the row kernel's BF16x3 form
    p5 = iga.get_plan2(D2(math="bf16x3", **dict(c2, R=5, S=5, pad=2)))
    assert p5.math == 1 and p5.base.variant == iga.VARIANT_DENSE_BF16X3
    for kw in (dict(stride=2), dict(dilation=2), dict(C=60), dict(groups=32, C=64, K=64)):
        q = iga.get_plan2(D2(math="bf16x3", **dict(c2, **kw)))
        assert q.math == 0 and q.base.variant not in iga.VARIANTS_BF16X3, kw
    q = iga.get_plan2(D2(math="bf16x3", dtype=iga.BF16, **c2))
    assert q.math == 0 and q.base.variant == 3


def test_all_taps_plan_selection():
    """16-bit 3x3 stride-1 dense shapes with more than 64 input or output channels
    per group, whose padded output row fits 64 slots and whose unit's X rows fit
    192 slots (Wo + 2 <= 63), take the all-taps kernel, with units of
    64 // (Wo + 2) whole rows and tiles of 32 output x 64 input channels; longer
    rows, other filters, strides, dilations and groups of at most 64 x 64
    channels keep the row kernel.  BF16x3 takes it at any channel count, with
    64 output channels per tile."""
    def plan(**kw):
        base = dict(N=4, C=128, H=30, W=30, K=64, R=3, S=3, pad=1, dtype=iga.BF16, split_k=2)
        return iga.get_plan2(D2(**dict(base, **kw))).base
    for W, ru in ((14, 4), (28, 2), (30, 2), (31, 1), (56, 1), (61, 1)):
        p = plan(H=W, W=W)
        assert p.variant == iga.VARIANT_DENSE16_TAPS and p.unit_rows == ru * W, (W, p.variant)
        assert p.units == 4 * -(-W // ru) and p.tiles == 2 * 2
    assert plan(C=64).variant == 3 and plan(C=64, K=72).variant == iga.VARIANT_DENSE16_TAPS
    x3 = plan(C=64, dtype=iga.F32, math="bf16x3")
    assert x3.variant == iga.VARIANT_DENSE_BF16X3_TAPS and x3.tiles == 1
    assert plan(C=24, K=40, dtype=iga.F32, math="bf16x3").tiles == 1
    assert plan(H=62, W=62).variant == 3            # 64 + 2 * 64 + 2 X slots: over 192
    assert plan(R=5, S=5, pad=2).variant == 3
    assert plan(stride=2).variant != iga.VARIANT_DENSE16_TAPS
    assert plan(dilation=2).variant != iga.VARIANT_DENSE16_TAPS
    assert plan(dtype=iga.F16).variant == iga.VARIANT_DENSE16_TAPS
    assert plan(C=256, K=96, groups=2).tiles == 2 * 2 * 2   # per group: 48 output channels, 128 inputs
    assert plan(pad=(0, 2)).Wo == 32 and plan(pad=(0, 2)).variant == iga.VARIANT_DENSE16_TAPS
    assert plan(C=60).variant not in (iga.VARIANT_DENSE16_TAPS, 3)


def test_igemm_plans_and_errors():
    """Forward / data-gradient plans: output sizes, exact ceil-division slices, the
    refitted auto degree (split only grids under 1024 workgroups over a reduction
    of at least 512, the smallest power of two reaching 2048 workgroups, at most
    32, at least two reduction tiles per slice), and validation before any launch."""
    lib = iga.load()
    # A small-M layer: 1568 output pixels, reduction 4608.
    d = D2(N=8, C=512, H=14, W=14, K=512, R=3, S=3, pad=1)
    for direction in (iga.DIRECTION_FWD, iga.DIRECTION_DGRAD):
        p = iga.get_igemm_plan(d, direction).base
        assert p.variant == (20 if direction == iga.DIRECTION_FWD else 21)
        assert p.L == 8 * 14 * 14 and p.E == p.L * 512
        assert p.units == 4608 // 32 and p.tiles == 25 * 8
        assert p.ks_count == 16 and p.grid == 3200 and p.needs_reduce == 1   # 200 tiles x 16 >= 2048
        assert p.ws_bytes == 16 * (-(-p.E // 64) * 64) * 4
    # Large grids and shallow reductions are not split.
    assert iga.get_igemm_plan(D2(N=32, C=64, H=56, W=56, K=64, R=3, S=3, pad=1), 1).base.ks_count == 1
    assert iga.get_igemm_plan(D2(N=1, C=32, H=4, W=4, K=32, R=3, S=3, pad=1), 1).base.ks_count == 1
    # Degree caps: at most 32, at least two reduction tiles per slice.
    p = iga.get_igemm_plan(D2(N=1, C=2048, H=4, W=4, K=64, R=3, S=3, pad=1), 1).base
    assert p.ks_count == 32 and p.units_per_slice >= 2
    # Q = 576: 18 reduction tiles; degree 8 (18 / 16 < 2), i.e. 3 tiles per slice, 6 slices
    p = iga.get_igemm_plan(D2(N=1, C=64, H=4, W=4, K=64, R=3, S=3, pad=1), 1).base
    assert p.units_per_slice == 3 and p.ks_count == 6
    # Pinned degrees keep every slice non-empty.
    for sk in (1, 3, 7, 100):
        p = iga.get_igemm_plan(D2(N=2, C=64, H=9, W=9, K=32, R=3, S=3, pad=1, split_k=sk), 2).base
        assert p.ks_count <= sk and (p.ks_count - 1) * p.units_per_slice < p.units <= p.ks_count * p.units_per_slice
    # Width fold applies to these directions too.
    assert iga.get_igemm_plan(D2(N=2, C=3, H=64, W=64, K=96, R=16, S=16, pad=0, stride=16), 1).fold_width == 16
    # Errors before any launch.
    plan = iga.Plan2()
    assert lib.conv_igemm_get_plan(ctypes.byref(d), 3, ctypes.byref(plan)) == 3
    assert lib.conv_igemm_get_plan(ctypes.byref(D2(split_k=0)), 1, ctypes.byref(plan)) == 4
    ws = iga.get_igemm_plan(d, 1).base.ws_bytes
    assert lib.conv_fwd(ctypes.byref(d), None, 16, 16, 16, ws, None) == 1
    assert lib.conv_fwd(ctypes.byref(d), 16, 16, 16, None, ws, None) == 1
    assert lib.conv_fwd(ctypes.byref(d), 16, 16, 16, 16, ws - 1, None) == 7
    assert lib.conv_dgrad(ctypes.byref(d), 16, 24, 16, 16, ws, None) == 6
    assert lib.conv_dgrad(None, 16, 16, 16, 16, ws, None) == 1
    n = ctypes.c_size_t(0)
    assert lib.conv_igemm_workspace_size(ctypes.byref(d), 2, ctypes.byref(n)) == 0 and n.value == ws
