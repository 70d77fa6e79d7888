"""The fp32 row kernel's 256-lane forms on the GPU against the oracle, element
by element, across the k-index assignments it picks from the output width:
packed rows (Wo <= 14: four output rows per unit, one per lane group),
contiguous quarters of an output row per lane group (ceil(Wo / 4) odd, or 2 mod
4) and interleaved pixels (ceil(Wo / 4) a multiple of 4, or rows wider than
one unit), with 1 to 4 taps per tile, partial channel tiles and units, groups,
per-axis geometry, bias gradient and pinned and automatic splits."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_bias_against_oracle, log, to_device

pytestmark = pytest.mark.gpu

ROWS_VARIANT = 1   # plan variant of the dense row kernel


# (N, C, H, W, K, R, S, (pad_h, pad_w), groups, split_k, bias)
CASES = [
    (4, 64, 56, 56, 64, 3, 3, (1, 1), 1, 224, True),     # Wo = 56: Q = 14, pitch 72
    (8, 64, 28, 28, 64, 3, 3, (1, 1), 1, 224, False),    # Wo = 28: Q = 7, pitch 80
    (8, 64, 22, 22, 64, 3, 3, (1, 1), 1, 176, False),    # Wo = 22: Q = 6
    (2, 64, 64, 64, 64, 3, 3, (1, 1), 1, 128, True),     # Wo = 64: Q = 16, interleaved
    (4, 64, 80, 80, 64, 3, 3, (1, 1), 1, 128, False),    # Wo = 80: two units per row, interleaved
    (16, 64, 20, 41, 64, 2, 4, (0, 0), 1, 304, True),    # 4 taps per tile, Wo = 38: Q = 10
    (8, 64, 24, 28, 64, 3, 5, (1, 2), 1, 96, False),     # taps 0-3 and 4, Wo = 28
    (8, 72, 18, 18, 40, 3, 3, (1, 1), 1, 144, True),     # partial tiles: 64 + 8 in, 40 out; Q = 5
    (4, 128, 26, 26, 128, 3, 3, (1, 1), 2, 104, True),   # groups of 64; Q = 7
]

# Packed rows: (N, C, H, W, K, R, S, pad, stride, dilation, groups, split_k, bias);
# pad / stride / dilation are (h, w) pairs.  Units of 4 output rows; the last
# unit of an image is partial unless 4 divides Ho.
PACKED = [
    (8, 512, 14, 14, 512, 3, 3, (1, 1), (1, 1), (1, 1), 1, -1, True),   # Wo = 14: QA 14, QB 18; automatic split
    (16, 64, 14, 14, 64, 3, 3, (1, 1), (1, 1), (1, 1), 1, 3, False),    # 4 units per image, the last of 2 rows
    (32, 64, 7, 7, 64, 3, 3, (1, 1), (1, 1), (1, 1), 1, 5, True),       # Wo = 7: QA 10, QB 10
    (12, 64, 16, 16, 72, 2, 4, (0, 0), (1, 1), (1, 1), 1, 4, True),     # Wo = 13, 4 taps: QB 18
    (12, 64, 9, 16, 64, 1, 4, (0, 0), (1, 1), (1, 1), 1, 2, False),     # 1x4, Wo = 13: 16 X columns per row
    (12, 64, 9, 17, 64, 1, 4, (0, 0), (1, 1), (1, 1), 1, 2, False),     # Wo = 14, 4 taps: 17 X columns, not packed
    (64, 64, 3, 3, 64, 3, 3, (0, 0), (1, 1), (1, 1), 1, 7, True),       # Wo = 1, Ho = 1
    (16, 64, 9, 5, 64, 5, 5, (2, 2), (1, 1), (1, 1), 1, 3, False),      # taps 0-3 and 4, Wo = 5
    (8, 64, 14, 14, 64, 3, 3, (2, 1), (1, 1), (2, 1), 1, 4, True),      # row dilation 2, per-axis pad
    (8, 144, 10, 10, 144, 3, 3, (1, 1), (1, 1), (1, 1), 2, 2, True),    # groups of 72: 64 + 8 channel tiles
    (24, 64, 3, 12, 64, 3, 3, (1, 1), (1, 1), (1, 1), 1, -1, False),    # Ho = 3: one partial unit per image
    (8, 64, 14, 14, 64, 3, 3, (1, 1), (2, 1), (1, 1), 1, 4, False),     # row stride 2: not packed
]


def _inputs(N, C, H, W, K, R, S, pad, seed, stride=(1, 1), dil=(1, 1)):
    Ho = (H + 2 * pad[0] - dil[0] * (R - 1) - 1) // stride[0] + 1
    Wo = (W + 2 * pad[1] - dil[1] * (S - 1) - 1) // stride[1] + 1
    x = wd.draw_images(seed, wd.X_ID, 0, N, H, W, C, wd.Dist("normal", 1.0))
    dy = wd.draw_images(seed, wd.DY_ID, 0, N, Ho, Wo, K, wd.Dist("normal", 0.1))
    return x, dy


@pytest.mark.parametrize("case", range(len(CASES)))
def test_rows_kernel_256_lane_forms(case):
    import torch
    import implicit_gemm_amd as iga
    N, C, H, W, K, R, S, pad, groups, split_k, bias = CASES[case]
    log("rows 256-lane case", case, CASES[case])
    x, dy = _inputs(N, C, H, W, K, R, S, pad, seed=9300 + case)
    xd, dyd = to_device(x, "f32"), to_device(dy, "f32")
    plan = iga.get_plan2(iga.desc2_for(xd, dyd, R, S, pad, 1, 1, groups, split_k, "exact", -1))
    assert plan.base.variant == ROWS_VARIANT, plan.base.variant
    assert plan.base.grid >= 384, plan.base.grid          # the 256-lane form
    out = iga.wgrad(xd, dyd, R, S, pad, 1, 1, groups, split_k=split_k, bias=bias)
    torch.cuda.synchronize()
    got = (out[0] if bias else out).cpu().numpy().astype(np.float64)
    ref, den = oracle.wgrad_ref(x, dy, R, S, pad, 1, 1, groups)
    assert got.shape == ref.shape
    err = oracle.normalised_error(got, ref, den)
    log("  ks", plan.base.ks_count, "grid", plan.base.grid, "error %.3e" % err)
    assert err <= oracle.TOL["f32"], "normalised error %.3e" % err
    assert np.all(np.isfinite(got)) and np.count_nonzero(got == 0.0) == 0
    if bias:
        check_bias_against_oracle(dy, out[1].cpu().numpy(), "f32")


@pytest.mark.parametrize("case", range(len(PACKED)))
def test_rows_kernel_packed_rows(case):
    import torch
    import implicit_gemm_amd as iga
    N, C, H, W, K, R, S, pad, stride, dil, groups, split_k, bias = PACKED[case]
    log("rows packed case", case, PACKED[case])
    x, dy = _inputs(N, C, H, W, K, R, S, pad, 9400 + case, stride, dil)
    Ho, Wo = dy.shape[1], dy.shape[2]
    xd, dyd = to_device(x, "f32"), to_device(dy, "f32")
    plan = iga.get_plan2(iga.desc2_for(xd, dyd, R, S, pad, stride, dil, groups, split_k, "exact", -1))
    assert plan.base.variant == ROWS_VARIANT, plan.base.variant
    packed = stride[0] == 1 and dil[1] == 1 and Wo <= 14 and Wo + min(S, 4) - 1 <= 16
    if packed:
        assert plan.base.unit_rows == 4 * Wo and plan.base.units == N * -(-Ho // 4)
    else:
        assert plan.base.unit_rows != 4 * Wo
    out = iga.wgrad(xd, dyd, R, S, pad, stride, dil, groups, split_k=split_k, bias=bias)
    torch.cuda.synchronize()
    got = (out[0] if bias else out).cpu().numpy().astype(np.float64)
    ref, den = oracle.wgrad_ref(x, dy, R, S, pad, stride, dil, groups)
    assert got.shape == ref.shape
    err = oracle.normalised_error(got, ref, den)
    log("  ks", plan.base.ks_count, "grid", plan.base.grid, "error %.3e" % err)
    assert err <= oracle.TOL["f32"], "normalised error %.3e" % err
    assert np.all(np.isfinite(got)) and np.count_nonzero(got == 0.0) == 0
    if bias:
        check_bias_against_oracle(dy, out[1].cpu().numpy(), "f32")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_rows_kernel_packed_rows_16bit(dtype):
    """16-bit inputs whose channel counts the 16-bit kernels do not take (not
    multiples of 8) reach the row kernel, widened to fp32 at staging: packed
    rows against the oracle at the 16-bit bar."""
    import torch
    import implicit_gemm_amd as iga
    N, C, H, W, K = 16, 60, 14, 14, 44
    x, dy = _inputs(N, C, H, W, K, 3, 3, (1, 1), 9480)
    x, dy = wd.round_to(x, dtype), wd.round_to(dy, dtype)
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    plan = iga.get_plan2(iga.desc2_for(xd, dyd, 3, 3, 1, 1, 1, 1, -1, "exact", -1))
    assert plan.base.variant == ROWS_VARIANT and plan.base.unit_rows == 4 * 14
    out, db = iga.wgrad(xd, dyd, 3, 3, 1, 1, 1, 1, bias=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref, den = oracle.wgrad_ref(x, dy, 3, 3, 1, 1, 1, 1)
    err = oracle.normalised_error(got, ref, den)
    log("rows packed", dtype, "ks", plan.base.ks_count, "error %.3e" % err)
    assert err <= oracle.TOL[dtype]
    assert np.all(np.isfinite(got)) and np.count_nonzero(got == 0.0) == 0
    check_bias_against_oracle(dy, db.cpu().numpy(), dtype)


def _random_rows_case(rng):
    """A random fp32 problem the row kernel takes: channel counts in quads,
    unit strides (row stride 2 now and then), filters up to 5x5, per-axis
    padding, groups, output widths 1..14 (packed rows) half of the time and
    15..64 otherwise, a random pinned or automatic split."""
    groups = int(rng.choice([1, 1, 1, 2, 4]))
    C = groups * 4 * int(rng.integers(1, 20))
    K = groups * 4 * int(rng.integers(1, 20))
    R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    pad = (int(rng.integers(0, R)), int(rng.integers(0, S)))
    stride = (int(rng.choice([1, 1, 1, 2])), 1)
    Wo = int(rng.integers(1, 15)) if rng.integers(0, 2) else int(rng.integers(15, 65))
    W = Wo - 1 + S - 2 * pad[1]
    if W < 1:
        pad = (pad[0], 0)
        W = Wo - 1 + S
    H = int(rng.integers(max(1, R - 2 * pad[0]), 24))
    N = int(rng.integers(1, 17))
    split = int(rng.choice([-1, -1, 1, 2, 3, 5, 17, 64, 1000]))
    bias = bool(rng.integers(0, 2))
    return N, C, H, W, K, R, S, pad, stride, groups, split, bias


@pytest.mark.parametrize("seed", range(32))
def test_rows_kernel_random_shapes(seed):
    import torch
    import implicit_gemm_amd as iga
    rng = np.random.default_rng(9500 + seed)
    for _ in range(50):   # draw until the planner gives the row kernel
        N, C, H, W, K, R, S, pad, stride, groups, split, bias = _random_rows_case(rng)
        d = iga.make_desc2(N, C, H, W, K, R, S, pad, stride, (1, 1), groups, 0, split, "exact", -1)
        if iga.get_plan2(d).base.variant == ROWS_VARIANT:
            break
    else:
        pytest.skip("no row-kernel shape drawn")
    case = (N, C, H, W, K, R, S, pad, stride, groups, split, bias)
    log("rows random case", seed, case)
    x, dy = _inputs(N, C, H, W, K, R, S, pad, 9600 + seed, stride)
    xd, dyd = to_device(x, "f32"), to_device(dy, "f32")
    plan = iga.get_plan2(iga.desc2_for(xd, dyd, R, S, pad, stride, 1, groups, split, "exact", -1))
    out = iga.wgrad(xd, dyd, R, S, pad, stride, 1, groups, split_k=split, bias=bias)
    torch.cuda.synchronize()
    got = (out[0] if bias else out).cpu().numpy().astype(np.float64)
    ref, den = oracle.wgrad_ref(x, dy, R, S, pad, stride, 1, groups)
    err = oracle.normalised_error(got, ref, den)
    log("  unit rows", plan.base.unit_rows, "ks", plan.base.ks_count, "grid", plan.base.grid, "error %.3e" % err)
    assert err <= oracle.TOL["f32"], "normalised error %.3e" % err
    assert np.all(np.isfinite(got))
    if bias:
        check_bias_against_oracle(dy, out[1].cpu().numpy(), "f32")
