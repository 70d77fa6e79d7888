"""The fp32 row kernel's 256-lane form on the GPU against the oracle, element
by element, across the k-index assignments it picks from the output width:
contiguous quarters of an output row per lane group (ceil(Wo / 4) odd, or 2 mod
4: pixel pitches 112 and 88) and interleaved pixels (ceil(Wo / 4) a multiple
of 4, or rows wider than one unit), with 1 to 4 taps per tile, partial channel
tiles, groups, bias gradient and pinned splits."""
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
    (4, 64, 56, 56, 64, 3, 3, (1, 1), 1, 224, True),     # Wo = 56: Q = 14, pitch 88
    (8, 64, 28, 28, 64, 3, 3, (1, 1), 1, 224, False),    # Wo = 28: Q = 7, pitch 112
    (16, 64, 9, 9, 64, 3, 3, (1, 1), 1, 144, True),      # Wo = 9: Q = 3
    (8, 64, 22, 22, 64, 3, 3, (1, 1), 1, 176, False),    # Wo = 22: Q = 6
    (32, 64, 5, 5, 64, 3, 3, (1, 1), 1, 160, True),      # Wo = 5: Q = 2
    (192, 64, 3, 3, 64, 3, 3, (0, 0), 1, 192, False),    # Wo = 1: Q = 1
    (2, 64, 64, 64, 64, 3, 3, (1, 1), 1, 128, True),     # Wo = 64: Q = 16, interleaved
    (4, 64, 80, 80, 64, 3, 3, (1, 1), 1, 128, False),    # Wo = 80: two units per row, interleaved
    (16, 64, 20, 41, 64, 2, 4, (0, 0), 1, 304, True),    # 4 taps per tile, Wo = 38: Q = 10
    (8, 64, 24, 28, 64, 3, 5, (1, 2), 1, 96, False),     # taps 0-3 and 4, Wo = 28
    (8, 72, 18, 18, 40, 3, 3, (1, 1), 1, 144, True),     # partial tiles: 64 + 8 in, 40 out; Q = 5
    (4, 128, 26, 26, 128, 3, 3, (1, 1), 2, 104, True),   # groups of 64; Q = 7
    (48, 64, 10, 10, 64, 1, 2, (0, 0), 1, 480, False),   # 1x2 filter, two taps per tile; Q = 3
    (48, 64, 10, 10, 64, 3, 1, (1, 0), 1, 480, True),    # 3x1 filter, one tap per tile; Q = 3
]


def _inputs(N, C, H, W, K, R, S, pad, seed):
    Ho, Wo = H + 2 * pad[0] - R + 1, W + 2 * pad[1] - S + 1
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
