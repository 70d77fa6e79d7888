"""Extended descriptor on the GPU against the oracle: per-axis pad / stride /
dilation, the width fold, and BF16x3 for fp32 inputs (conv_wgrad2 through the
binding's wgrad)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_bias_against_oracle, log, to_device

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1, "f16": 2}


def _extent(n, k, pad, stride, dil):
    return (n + 2 * pad - dil * (k - 1) - 1) // stride + 1


def _inputs(N, C, H, W, K, R, S, pad, stride, dil, dtype, seed, x_dist=None, dy_dist=None):
    """Seeded inputs for per-axis geometry (dY shaped by the row and column extents)."""
    Ho = _extent(H, R, pad[0], stride[0], dil[0])
    Wo = _extent(W, S, pad[1], stride[1], dil[1])
    x_dist = x_dist or wd.Dist("normal", 1.0)
    dy_dist = dy_dist or wd.Dist("normal", 0.1)
    x = wd.draw_images(seed, wd.X_ID, 0, N, H, W, C, x_dist)
    dy = wd.draw_images(seed, wd.DY_ID, 0, N, Ho, Wo, K, dy_dist)
    return wd.round_to(x, dtype), wd.round_to(dy, dtype)


def _run(x, dy, R, S, pad, stride, dil, groups, dtype, split_k=-1, math="exact", fold_width=-1, bias=False):
    import torch
    import implicit_gemm_amd as iga
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    d = iga.desc2_for(xd, dyd, R, S, pad, stride, dil, groups, split_k, math, fold_width)
    plan = iga.get_plan2(d)
    out = iga.wgrad(xd, dyd, R, S, pad, stride, dil, groups, split_k=split_k, math=math,
                    fold_width=fold_width, bias=bias)
    torch.cuda.synchronize()
    if bias:
        return out[0].cpu().numpy().astype(np.float64), out[1].cpu().numpy(), plan
    return out.cpu().numpy().astype(np.float64), None, plan


def _check(x, dy, R, S, pad, stride, dil, groups, dtype, tol=None, **kw):
    got, db, plan = _run(x, dy, R, S, pad, stride, dil, groups, dtype, **kw)
    ref, den = oracle.wgrad_ref(x, dy, R, S, pad, stride, dil, groups)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = oracle.normalised_error(got, ref, den)
    tol = oracle.TOL[dtype] if tol is None else tol
    assert err <= tol, "normalised error %.3e > %.1e" % (err, tol)
    if db is not None:
        check_bias_against_oracle(dy, db, dtype)
    return err, plan


# (N, C, H, W, K, R, S, pad, stride, dilation, groups, dtype, split_k, bias, variant expected)
PER_AXIS_CASES = [
    (4, 64, 20, 24, 64, 3, 5, (1, 2), (1, 1), (1, 1), 1, "f32", -1, True, 1),     # dense rows, pad only
    (4, 64, 21, 30, 48, 3, 3, (1, 0), (1, 2), (1, 1), 1, "f32", 3, False, 1),     # column stride 2
    (2, 32, 18, 19, 32, 3, 3, (0, 2), (2, 1), (1, 2), 1, "f32", -1, True, 1),     # row stride, column dilation
    (3, 64, 14, 40, 64, 5, 3, (2, 1), (1, 1), (1, 1), 1, "bf16", 2, True, 3),     # 16-bit rows, pad only
    (3, 64, 17, 17, 72, 1, 5, (0, 2), (1, 1), (1, 1), 1, "f16", -1, False, 3),    # 1x5 filter
    (2, 64, 16, 26, 64, 3, 3, (1, 0), (2, 1), (1, 1), 1, "bf16", -1, False, 1),   # 16-bit on dense rows
    (2, 12, 11, 13, 10, 3, 2, (1, 0), (1, 3), (2, 1), 1, "f32", 2, True, 0),      # general kernel
    (2, 9, 10, 12, 6, 2, 3, (0, 1), (3, 1), (1, 1), 3, "bf16", -1, True, 10),     # 3 ch/group: element kernel
    (2, 32, 12, 15, 32, 5, 3, (2, 1), (1, 2), (1, 1), 32, "bf16", -1, True, 10),  # depthwise: element kernel
    (2, 32, 9, 14, 32, 3, 3, (0, 1), (2, 1), (1, 1), 8, "f16", 3, False, 10),     # 4 ch/group: element kernel
]


@pytest.mark.parametrize("idx", range(len(PER_AXIS_CASES)))
def test_per_axis_geometry(idx):
    N, C, H, W, K, R, S, pad, stride, dil, groups, dtype, sk, bias, variant = PER_AXIS_CASES[idx]
    x, dy = _inputs(N, C, H, W, K, R, S, pad, stride, dil, dtype, 600 + idx)
    err, plan = _check(x, dy, R, S, pad, stride, dil, groups, dtype, split_k=sk, bias=bias, fold_width=0)
    log("per-axis", PER_AXIS_CASES[idx], "variant", plan.base.variant, "ks", plan.base.ks_count,
        "error %.3e" % err)
    assert plan.base.variant == variant


def test_per_axis_random_sweep():
    rng = np.random.default_rng(77)
    worst = {}
    done = 0
    while done < 60:
        groups = int(rng.choice([1, 1, 1, 2, 4, 16]))
        cg = int(rng.choice([1, 3, 4, 8, 16])) if groups > 1 else int(rng.choice([4, 8, 12, 16, 24, 64]))
        kg = cg if groups > 1 and rng.random() < 0.7 else int(rng.choice([4, 8, 16, 64]))
        C, K = groups * cg, groups * kg
        H, W = int(rng.integers(4, 30)), int(rng.integers(4, 30))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        pad = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        stride = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        if _extent(H, R, pad[0], stride[0], dil[0]) < 1 or _extent(W, S, pad[1], stride[1], dil[1]) < 1:
            continue
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        sk = int(rng.choice([-1, -1, 1, 2, 5]))
        bias = bool(rng.random() < 0.4)
        x, dy = _inputs(int(rng.integers(1, 5)), C, H, W, K, R, S, pad, stride, dil, dtype, 6000 + done)
        err, plan = _check(x, dy, R, S, pad, stride, dil, groups, dtype, split_k=sk, bias=bias)
        v = int(plan.base.variant)
        worst[v] = max(worst.get(v, 0.0), err)
        done += 1
    log("per-axis sweep: worst normalised error per variant", worst)


# (N, C, H, W, K, R, S, pad, stride, dtype, fold expected under auto)
FOLD_CASES = [
    (4, 3, 64, 64, 96, 16, 16, (0, 0), (16, 16), "f32", 16),   # patch embedding 16x16 / 16
    (2, 3, 64, 64, 64, 16, 16, (0, 0), (16, 16), "bf16", 16),
    (2, 3, 48, 48, 32, 8, 8, (0, 0), (8, 8), "f16", 8),
    (3, 6, 32, 32, 16, 2, 2, (0, 0), (2, 2), "f32", 2),        # 2x2 stride-2 downsample
    (2, 3, 10, 36, 8, 5, 4, (2, 4), (1, 4), "f32", 4),         # per-axis padding divisible by f
]


@pytest.mark.parametrize("idx", range(len(FOLD_CASES)))
def test_width_fold(idx):
    """Folded (automatic and explicit) and unfolded runs all match the oracle of the
    original problem, and the folded plan is the one the shape allows."""
    N, C, H, W, K, R, S, pad, stride, dtype, f = FOLD_CASES[idx]
    dil = (1, 1)
    x, dy = _inputs(N, C, H, W, K, R, S, pad, stride, dil, dtype, 900 + idx)
    errs = {}
    for fw in (-1, 0, 2 if f % 2 == 0 else f):
        err, plan = _check(x, dy, R, S, pad, stride, dil, 1, dtype, fold_width=fw, bias=(fw == -1))
        errs[fw] = (err, int(plan.fold_width), int(plan.base.variant))
        if fw == -1:
            assert plan.fold_width == f
        if fw == 0:
            assert plan.fold_width == 1
    log("fold", FOLD_CASES[idx], errs)


def test_bf16x3_full_size_3x3():
    """BF16x3 on the 3x3 fp32 workload (N=32, C=K=64, 56x56) against the oracle,
    bit-identical run to run, bias gradient exact in fp32."""
    wl = wd.WORKLOADS["c2_3x3_f32"]
    s = wl.shape
    x, dy = wd.make_inputs(wl)
    got, db, plan = _run(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, "f32", math="bf16x3", bias=True)
    assert plan.base.variant == 6 and plan.math == 1   # the all-taps kernel's BF16x3 form
    ref, den = oracle.wgrad_ref(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
    err = oracle.normalised_error(got, ref, den)
    db_err = check_bias_against_oracle(dy, db, "f32")
    log("bf16x3 3x3 full size: normalised error %.3e (db %.3e), ks %d" % (err, db_err, plan.base.ks_count))
    assert err <= oracle.TOL["f32"]
    again, _, _ = _run(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, "f32", math="bf16x3")
    assert np.array_equal(again, got)
    exact, _, _ = _run(x, dy, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, "f32")
    log("exact fp32 path error %.3e" % oracle.normalised_error(exact, ref, den))


# (N, C, H, W, K, R, S, pad, split_k, bias)
X3_CASES = [
    (2, 64, 14, 14, 64, 3, 3, (1, 1), -1, True),     # short rows: units of several rows
    (3, 72, 9, 30, 40, 3, 3, (1, 0), 2, False),      # partial channel tiles, per-axis pad
    (2, 64, 12, 12, 136, 5, 5, (2, 2), 4, True),     # two tap blocks, three M tiles
    (4, 128, 10, 70, 40, 1, 1, (0, 0), 3, False),    # 1x1 with two 64-pixel chunks per row
    (2, 64, 16, 16, 64, 3, 3, (1, 1), 1, True),      # one slice (writes dw directly)
    (1, 8, 5, 9, 8, 3, 2, (0, 1), 2, True),          # 8 channels (pinned split: automatic would run it unsplit, exact)
    (2, 64, 6, 70, 64, 3, 3, (1, 1), 2, True),       # 3x3 with 70-pixel rows: the row kernel
]


@pytest.mark.parametrize("idx", range(len(X3_CASES)))
def test_bf16x3_shapes(idx):
    N, C, H, W, K, R, S, pad, sk, bias = X3_CASES[idx]
    x, dy = _inputs(N, C, H, W, K, R, S, pad, (1, 1), (1, 1), "f32", 950 + idx)
    err, plan = _check(x, dy, R, S, pad, 1, 1, 1, "f32", split_k=sk, math="bf16x3", bias=bias)
    log("bf16x3", X3_CASES[idx], "ks", plan.base.ks_count, "error %.3e" % err)
    # 3x3 rows of at most 61 pixels: the all-taps kernel; otherwise the row kernel
    assert plan.base.variant == (6 if (R, S) == (3, 3) and W + 2 * pad[1] - 2 <= 61 else 4)


def test_bf16x3_positive_inputs_and_fallback():
    """All-positive inputs (errors of one sign in the split residuals would add up)
    stay within the fp32 bar; a shape no BF16x3 kernel covers runs the exact path."""
    N, C, H, W, K = 4, 64, 24, 24, 64
    x, dy = _inputs(N, C, H, W, K, 3, 3, (1, 1), (1, 1), (1, 1), "f32", 990,
                    x_dist=wd.Dist("uniform"), dy_dist=wd.Dist("uniform"))
    x, dy = np.abs(x), np.abs(dy)
    err, plan = _check(x, dy, 3, 3, 1, 1, 1, 1, "f32", math="bf16x3")
    log("bf16x3 positive inputs: error %.3e" % err)
    assert plan.base.variant == 6
    x2, dy2 = _inputs(2, 64, 20, 20, 64, 3, 3, (1, 1), (2, 2), (1, 1), "f32", 991)
    err2, plan2 = _check(x2, dy2, 3, 3, 1, 2, 1, 1, "f32", math="bf16x3")
    assert plan2.math == 0 and plan2.base.variant not in (4, 6)
    log("bf16x3 request on stride 2: exact path, error %.3e" % err2)
    # A launch-bound problem with an automatic split runs unsplit on the exact general kernel.
    x3, dy3 = _inputs(1, 8, 5, 9, 8, 3, 2, (0, 1), (1, 1), (1, 1), "f32", 992)
    err3, plan3 = _check(x3, dy3, 3, 2, (0, 1), 1, 1, 1, "f32", math="bf16x3")
    assert plan3.math == 0 and plan3.base.variant == 0 and plan3.base.ks_count == 1
    log("bf16x3 request on a launch-bound problem: exact, one launch, error %.3e" % err3)
