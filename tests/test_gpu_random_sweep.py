"""Seeded random sweeps over every stage-1 path against the fp64 oracle.

Each sweep draws a few hundred small shapes aimed at one family of kernels
(dense rows fp32 with stride and dilation, the general dense kernel on odd
channel counts, 16-bit dense with short and long rows, row-streaming and
windowed grouped kernels at stride 1 and 2, depthwise, the element fallback,
the 1x1 streaming kernel), with random split degrees and, on some cases, the
fused bias gradient (db checked against the bias oracle).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_against_oracle, check_bias_against_oracle, log, to_device

DT = {"f32": 0, "bf16": 1, "f16": 2}


def _out(shp):
    Ho = (shp.H + 2 * shp.pad - shp.dilation * (shp.R - 1) - 1) // shp.stride + 1
    Wo = (shp.W + 2 * shp.pad - shp.dilation * (shp.S - 1) - 1) // shp.stride + 1
    return Ho, Wo


def _draw(kind, rng):
    N = int(rng.integers(1, 4))
    if kind == "dense16_short":
        R = int(rng.choice([1, 3, 5])); pad = int(rng.integers(0, R // 2 + 2)); g = int(rng.choice([1, 1, 2]))
        return wd.ConvShape(N, g * 8 * int(rng.integers(1, 10)), int(rng.integers(1, 20)), int(rng.integers(1, 31)),
                            g * 8 * int(rng.integers(1, 10)), R, R, pad=pad, groups=g), str(rng.choice(["bf16", "f16"]))
    if kind == "dense16_long":
        R = int(rng.integers(1, 6)); S = int(rng.integers(1, 6)); g = int(rng.choice([1, 2]))
        return wd.ConvShape(N, g * 8 * int(rng.integers(1, 12)), int(rng.integers(1, 12)), int(rng.integers(31, 130)),
                            g * 8 * int(rng.integers(1, 12)), R, S, pad=int(rng.integers(0, 3)), groups=g), \
            str(rng.choice(["bf16", "f16"]))
    if kind == "dense32":
        g = int(rng.choice([1, 1, 2, 4]))
        return wd.ConvShape(N, g * 4 * int(rng.integers(1, 40)), int(rng.integers(1, 40)), int(rng.integers(1, 70)),
                            g * 4 * int(rng.integers(1, 40)), int(rng.integers(1, 6)), int(rng.integers(1, 6)),
                            pad=int(rng.integers(0, 4)), stride=int(rng.choice([1, 1, 2, 3])),
                            dilation=int(rng.choice([1, 1, 2])), groups=g), "f32"
    if kind == "dense_odd":
        return wd.ConvShape(N, int(rng.integers(1, 70)), int(rng.integers(1, 20)), int(rng.integers(1, 20)),
                            int(rng.integers(1, 70)), int(rng.integers(1, 4)), int(rng.integers(1, 4)),
                            pad=int(rng.integers(0, 2)), stride=int(rng.choice([1, 2]))), \
            str(rng.choice(["f32", "bf16", "f16"]))
    if kind in ("grouped_s1", "grouped_s2"):
        R = int(rng.choice([1, 3, 5, 7])); cpg = int(rng.choice([1, 2, 4, 8, 16])); C = 16 * int(rng.integers(1, 9))
        return wd.ConvShape(N, C, int(rng.integers(1, 30)), int(rng.integers(1, 66)), C, R, R,
                            pad=int(rng.integers(0, R)), stride=1 if kind == "grouped_s1" else 2,
                            groups=C // cpg), str(rng.choice(["bf16", "f16"]))
    if kind == "grouped_other":
        cpg = int(rng.choice([2, 4, 8])); C = 16 * int(rng.integers(1, 6))
        return wd.ConvShape(N, C, int(rng.integers(1, 16)), int(rng.integers(1, 120)), C, int(rng.integers(1, 5)),
                            int(rng.integers(1, 5)), pad=int(rng.integers(0, 3)), dilation=int(rng.choice([1, 2])),
                            groups=C // cpg), str(rng.choice(["bf16", "f16"]))
    if kind == "depthwise":
        C = 16 * int(rng.integers(1, 13))
        return wd.ConvShape(N, C, int(rng.integers(1, 24)), int(rng.integers(1, 100)), C, int(rng.integers(1, 9)),
                            int(rng.integers(1, 9)), pad=int(rng.integers(0, 5)), stride=int(rng.choice([1, 1, 2])),
                            groups=C), str(rng.choice(["bf16", "f16"]))
    if kind == "elem":
        G = int(rng.integers(1, 9))
        return wd.ConvShape(N, int(rng.choice([1, 2, 3, 4, 8])) * G, int(rng.integers(1, 14)), int(rng.integers(1, 20)),
                            int(rng.choice([1, 2, 3, 4, 8])) * G, int(rng.integers(1, 5)), int(rng.integers(1, 5)),
                            pad=int(rng.integers(0, 3)), stride=int(rng.choice([1, 2, 3])), groups=G), \
            str(rng.choice(["f32", "bf16", "f16"]))
    # 1x1 streaming kernel
    return wd.ConvShape(int(rng.integers(1, 5)), 16 * int(rng.integers(1, 9)), int(rng.integers(1, 40)),
                        int(rng.integers(1, 40)), 64 * int(rng.integers(1, 3)), 1, 1), "f32"


KINDS = ["dense16_short", "dense16_long", "dense32", "dense_odd", "grouped_s1", "grouped_s2", "grouped_other",
         "depthwise", "elem", "1x1"]


@pytest.mark.gpu
@pytest.mark.parametrize("seed", [1, 2])
def test_random_sweep(seed):
    import torch
    import implicit_gemm_amd as iga
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < 30 * len(KINDS):
        kind = KINDS[len(cases) % len(KINDS)]
        shp, dt = _draw(kind, rng)
        Ho, Wo = _out(shp)
        if Ho < 1 or Wo < 1:
            continue
        cases.append((kind, shp, dt, int(rng.choice([-1, -1, 1, 2, 3, 7])), bool(rng.random() < 0.4)))
    worst = {}
    for i, (kind, shp, dt, sk, bias) in enumerate(cases):
        plan = iga.get_plan(iga.make_desc(shp.N, shp.C, shp.H, shp.W, shp.K, shp.R, shp.S, shp.pad, shp.stride,
                                          shp.dilation, shp.groups, DT[dt], sk))
        log("sweep", seed, i, kind, "variant", plan.variant, shp, dt, "split", sk, "bias", bias)
        x, dy = wd.random_inputs(shp, dt, seed=1000 * seed + i, x_dist=wd.Dist("normal", 1.0),
                                 dy_dist=wd.Dist("normal", 0.1))
        if bias:
            dw, db = iga.wgrad(to_device(x, dt), to_device(dy, dt), shp.R, shp.S, shp.pad, shp.stride,
                               shp.dilation, shp.groups, split_k=sk, bias=True)
            torch.cuda.synchronize()
            err = check_against_oracle(x, dy, shp, dt, split_k=sk, dw_gpu=dw.cpu().numpy().astype(np.float64))
            db_err = check_bias_against_oracle(dy, db.cpu().numpy(), dt)
            err = max(err, db_err)
        else:
            err = check_against_oracle(x, dy, shp, dt, split_k=sk)
        worst[kind] = max(worst.get(kind, 0.0), err)
    log("sweep", seed, len(cases), "cases; worst normalised error per kind:", worst)
