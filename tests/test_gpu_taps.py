"""The 16-bit all-taps dense kernel (3x3, stride 1, dilation 1, output rows up to
61 pixels, more than 64 input or output channels per group) and its BF16x3 form
on the GPU against the oracle, element by element:
units of one to 21 packed rows, the three X staging sizes, partial output- and
input-channel tiles, groups, per-axis and large padding, bias gradient, pinned
and automatic splits."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_bias_against_oracle, log, to_device

pytestmark = pytest.mark.gpu


def _inputs(N, C, H, W, K, pad, dtype, seed):
    Ho, Wo = H + 2 * pad[0] - 2, W + 2 * pad[1] - 2
    x = wd.draw_images(seed, wd.X_ID, 0, N, H, W, C, wd.Dist("normal", 1.0))
    dy = wd.draw_images(seed, wd.DY_ID, 0, N, Ho, Wo, K, wd.Dist("normal", 0.1))
    return wd.round_to(x, dtype), wd.round_to(dy, dtype)


def _run(x, dy, pad, groups, dtype, split_k, math, bias):
    import torch
    import implicit_gemm_amd as iga
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    plan = iga.get_plan2(iga.desc2_for(xd, dyd, 3, 3, pad, 1, 1, groups, split_k, math, -1))
    out = iga.wgrad(xd, dyd, 3, 3, pad, 1, 1, groups, split_k=split_k, math=math, bias=bias)
    torch.cuda.synchronize()
    if bias:
        return out[0].cpu().numpy().astype(np.float64), out[1].cpu().numpy(), plan
    return out.cpu().numpy().astype(np.float64), None, plan


# (N, C, H, W, K, (pad_h, pad_w), groups, dtype, split_k, bias, math)
CASES = [
    (2, 64, 56, 56, 96, (1, 1), 1, "bf16", -1, False, "exact"),    # one 56-pixel row per unit, 192 X slots
    (3, 64, 14, 14, 72, (1, 1), 1, "f16", -1, True, "exact"),      # 4 rows per unit, 128 X slots, tiles 32+32+8 out
    (2, 72, 28, 28, 40, (1, 1), 1, "bf16", 3, True, "exact"),      # 2 rows; partial tiles: 64 + 8 in, 32 + 8 out
    (1, 24, 31, 31, 80, (0, 0), 1, "bf16", 1, False, "exact"),     # Wo = 29: 2 rows of pitch 31, unsplit
    (2, 128, 20, 61, 64, (1, 1), 1, "f16", 2, False, "exact"),     # Wo = 61: pitch 63, the largest row
    (2, 256, 16, 16, 96, (2, 1), 2, "bf16", -1, True, "exact"),    # groups of 128 in / 48 out, per-axis pad
    (1, 16, 9, 40, 72, (0, 2), 1, "bf16", 5, True, "exact"),       # Wo = 42: 160 X slots; 7 one-row units in 4 slices
    (2, 80, 30, 3, 8, (0, 0), 1, "f16", 2, True, "exact"),         # Wo = 1: 21 rows per unit; 64 + 16 in
    (1, 16, 10, 10, 136, (3, 3), 1, "bf16", 2, False, "exact"),    # pad 3: unit X rows past the image
    (4, 256, 14, 14, 256, (1, 1), 1, "bf16", -1, True, "exact"),   # 8 x 4 channel tiles
    (2, 64, 56, 56, 64, (1, 1), 1, "f32", -1, True, "bf16x3"),     # BF16x3, 192 X slots in two planes
    (2, 24, 14, 14, 40, (1, 1), 1, "f32", 2, True, "bf16x3"),      # BF16x3, 4 rows per unit, a 40-channel tile
    (1, 64, 12, 45, 32, (1, 1), 1, "f32", 1, False, "bf16x3"),     # BF16x3, 160 X slots, unsplit
    (2, 128, 10, 12, 136, (1, 1), 1, "f32", 3, True, "bf16x3"),    # BF16x3, 64 + 64 + 8 out x 64 + 64 in tiles
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_all_taps_kernel(case):
    import implicit_gemm_amd as iga
    N, C, H, W, K, pad, groups, dtype, split_k, bias, math = CASES[case]
    log("all-taps case", case, CASES[case])
    x, dy = _inputs(N, C, H, W, K, pad, dtype, seed=9100 + case)
    got, db, plan = _run(x, dy, pad, groups, dtype, split_k, math, bias)
    want = iga.VARIANT_DENSE_BF16X3_TAPS if math == "bf16x3" else iga.VARIANT_DENSE16_TAPS
    assert plan.base.variant == want, plan.base.variant
    ref, den = oracle.wgrad_ref(x, dy, 3, 3, pad, 1, 1, groups)
    assert got.shape == ref.shape
    err = oracle.normalised_error(got, ref, den)
    tol = oracle.TOL[dtype]
    log("  ks", plan.base.ks_count, "grid", plan.base.grid, "error %.3e" % err)
    assert err <= tol, "normalised error %.3e > %.1e" % (err, tol)
    assert np.all(np.isfinite(got)) and np.count_nonzero(got == 0.0) == 0
    if db is not None:
        check_bias_against_oracle(dy, db, dtype)


def test_all_taps_bit_identical_and_split_independent():
    """Two calls at one split agree bit for bit; pinned splits 1, 6 and 21 (of 42
    two-row units) agree with the oracle to the 16-bit bar (only the summation
    order differs)."""
    N, C, H, W, K, pad = 3, 64, 28, 28, 96, (1, 1)
    x, dy = _inputs(N, C, H, W, K, pad, "bf16", seed=9177)
    a, _, _ = _run(x, dy, pad, 1, "bf16", 4, "exact", False)
    b, _, _ = _run(x, dy, pad, 1, "bf16", 4, "exact", False)
    assert np.array_equal(a, b)
    ref, den = oracle.wgrad_ref(x, dy, 3, 3, pad, 1, 1, 1)
    for sk in (1, 6, 21):
        got, _, plan = _run(x, dy, pad, 1, "bf16", sk, "exact", False)
        assert plan.base.ks_count == sk
        assert oracle.normalised_error(got, ref, den) <= oracle.TOL["bf16"]
