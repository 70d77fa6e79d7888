"""Forward convolution and data gradient (conv_fwd / conv_dgrad) on the GPU
against the oracle: geometry, groups, dtypes, split degrees, the width fold,
run-to-run bit identity."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu


def _extent(n, k, pad, stride, dil):
    return (n + 2 * pad - dil * (k - 1) - 1) // stride + 1


def _pair(v):
    return tuple(v) if isinstance(v, (tuple, list)) else (v, v)


def _case_inputs(N, C, H, W, K, R, S, pad, stride, dil, groups, dtype, seed):
    (ph, pw), (sh, sw), (dh, dw) = _pair(pad), _pair(stride), _pair(dil)
    Ho, Wo = _extent(H, R, ph, sh, dh), _extent(W, S, pw, sw, dw)
    x = wd.round_to(wd.draw_images(seed, wd.X_ID, 0, N, H, W, C, wd.Dist("normal", 1.0)), dtype)
    dy = wd.round_to(wd.draw_images(seed, wd.DY_ID, 0, N, Ho, Wo, K, wd.Dist("normal", 0.1)), dtype)
    w = wd.draw_filter(seed, K, R, S, C // groups, wd.Dist("normal", 0.05), dtype)
    return x, dy, w


def run_fwd(x, w, pad, stride, dil, groups, dtype, split_k=-1, fold_width=-1):
    import torch
    import implicit_gemm_amd as iga
    y = iga.fwd(to_device(x, dtype), to_device(w, dtype), pad, stride, dil, groups, split_k, fold_width)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def run_dgrad(dy, w, H, W, pad, stride, dil, groups, dtype, split_k=-1, fold_width=-1):
    import torch
    import implicit_gemm_amd as iga
    dx = iga.dgrad(to_device(dy, dtype), to_device(w, dtype), H, W, pad, stride, dil, groups, split_k,
                   fold_width)
    torch.cuda.synchronize()
    return dx.cpu().numpy().astype(np.float64)


def check_both(N, C, H, W, K, R, S, pad, stride, dil, groups, dtype, split_k=-1, seed=0, fold_width=-1):
    import implicit_gemm_amd as iga
    x, dy, w = _case_inputs(N, C, H, W, K, R, S, pad, stride, dil, groups, dtype, seed)
    d = iga.make_desc2(N, C, H, W, K, R, S, pad, stride, dil, groups, {"f32": 0, "bf16": 1, "f16": 2}[dtype],
                       split_k, "exact", fold_width)
    pf = iga.get_igemm_plan(d, iga.DIRECTION_FWD)
    pd = iga.get_igemm_plan(d, iga.DIRECTION_DGRAD)
    y = run_fwd(x, w, pad, stride, dil, groups, dtype, split_k, fold_width)
    yr, yden = oracle.fwd_ref(x, w, pad, stride, dil, groups)
    ef = oracle.normalised_error(y, yr, yden)
    dx = run_dgrad(dy, w, H, W, pad, stride, dil, groups, dtype, split_k, fold_width)
    dxr, dden = oracle.dgrad_ref(dy, w, H, W, pad, stride, dil, groups)
    ed = oracle.normalised_error(dx, dxr, dden)
    tol = oracle.TOL[dtype]
    assert ef <= tol and ed <= tol, ("fwd %.3e dgrad %.3e" % (ef, ed))
    return ef, ed, pf, pd


# (N, C, H, W, K, R, S, pad, stride, dilation, groups, dtype, split_k)
CASES = [
    (4, 256, 14, 14, 256, 3, 3, 1, 1, 1, 1, "f32", -1),            # small-M layer, auto split
    (2, 64, 17, 15, 96, 3, 3, 1, 2, 1, 1, "f32", 3),               # stride 2 (dgrad holes)
    (2, 64, 13, 13, 64, 3, 3, 2, 1, 2, 1, "bf16", -1),             # dilation 2
    (3, 32, 9, 12, 48, 5, 3, (2, 1), (1, 2), (1, 1), 1, "f16", 5),  # per-axis
    (2, 3, 32, 32, 96, 16, 16, 0, 16, 1, 1, "f32", -1),            # patch embedding (folded)
    (2, 12, 10, 11, 20, 3, 2, (1, 0), 1, 1, 2, "f32", 2),          # groups, channels off quads
    (2, 9, 8, 8, 15, 2, 2, 0, 1, 1, 3, "bf16", -1),                # 3 channels per group: scalar loads
    (2, 64, 8, 8, 64, 3, 3, 1, 1, 1, 64, "bf16", -1),              # depthwise
    (1, 40, 7, 9, 72, 1, 1, 0, 1, 1, 1, "f16", 1),                 # 1x1, one slice
    (2, 128, 6, 6, 130, 3, 3, 1, 1, 1, 1, "f32", 40),              # pinned deep split, partial tiles
    (2, 136, 12, 12, 144, 3, 3, 1, 2, 1, 1, "f32", -1),            # dgrad at stride 2, partial tiles
    (2, 256, 10, 9, 256, 3, 3, (1, 0), 1, 1, 2, "bf16", 3),        # two groups of 128, per-axis pad
    (3, 132, 11, 13, 260, 3, 3, 1, 1, 1, 1, "f16", -1),            # partial tiles in M and N
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_fwd_dgrad_cases(idx):
    c = CASES[idx]
    ef, ed, pf, pd = check_both(*c, seed=1200 + idx)
    log("fwd/dgrad", c, "ks fwd %d dgrad %d fold %d" % (pf.base.ks_count, pd.base.ks_count, pf.fold_width),
        "errors %.3e %.3e" % (ef, ed))


def test_fwd_dgrad_random_sweep():
    rng = np.random.default_rng(1234)
    worst = [0.0, 0.0]
    done = 0
    while done < 40:
        groups = int(rng.choice([1, 1, 2, 4]))
        C, K = groups * int(rng.choice([3, 4, 8, 16, 24])), groups * int(rng.choice([4, 5, 16, 32]))
        H, W = int(rng.integers(3, 20)), int(rng.integers(3, 20))
        R, S = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        pad = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        stride = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        if _extent(H, R, pad[0], stride[0], dil[0]) < 1 or _extent(W, S, pad[1], stride[1], dil[1]) < 1:
            continue
        dtype = str(rng.choice(["f32", "bf16", "f16"]))
        sk = int(rng.choice([-1, 1, 2, 3, 7]))
        ef, ed, _, _ = check_both(int(rng.integers(1, 4)), C, H, W, K, R, S, pad, stride, dil, groups, dtype,
                                  sk, seed=7000 + done)
        worst = [max(worst[0], ef), max(worst[1], ed)]
        done += 1
    log("fwd/dgrad sweep: worst normalised errors", worst)


def test_fwd_dgrad_bits_repeat_with_nan_buffers():
    """At a fixed split the results are bit-identical run to run, whatever the
    output and the workspace held before (NaN fills)."""
    import torch
    import implicit_gemm_amd as iga
    N, C, H, W, K, R, S = 4, 128, 12, 12, 96, 3, 3
    x, dy, w = _case_inputs(N, C, H, W, K, R, S, 1, 1, 1, 1, "f32", 77)
    xd, dyd, wdv = to_device(x, "f32"), to_device(dy, "f32"), to_device(w, "f32")
    d = iga.make_desc2(N, C, H, W, K, R, S, 1, 1, 1, 1, 0, 6)
    for direction, src, shape in ((iga.DIRECTION_FWD, xd, (N, H, W, K)), (iga.DIRECTION_DGRAD, dyd, (N, H, W, C))):
        plan = iga.get_igemm_plan(d, direction).base
        assert plan.ks_count == 6
        outs = []
        for _ in range(2):
            out = torch.full(shape, float("nan"), device="cuda")
            ws = torch.full((int(plan.ws_bytes) // 4,), float("nan"), device="cuda")
            f = iga.conv_fwd if direction == iga.DIRECTION_FWD else iga.conv_dgrad
            f(d, src.data_ptr(), wdv.data_ptr(), out.data_ptr(), ws.data_ptr(), int(plan.ws_bytes),
              torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            outs.append(out)
        assert torch.equal(outs[0], outs[1]) and bool(torch.isfinite(outs[0]).all())
