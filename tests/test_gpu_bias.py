"""Fused bias gradient (conv_wgrad_bias) on the GPU vs the oracle, through the C ABI.

For every stage-1 kernel variant and for one slice, several slices and more
than 256 slices (two fold passes):
  * db against the fp64 oracle db[k] = sum dY[..., k], normalised by
    max_k sum |dY[..., k]|, within the dtype's tolerance;
  * dW bit-identical to what conv_wgrad_ex writes for the same descriptor;
  * dW against the weight-gradient oracle;
  * two runs bit-identical, with dw, db and the workspace pre-filled with NaN.
"""
import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_against_oracle, log, to_device

pytestmark = pytest.mark.gpu

VARIANT = {0: "dense_lds", 1: "dense_rows", 2: "dense_1x1", 3: "dense16_rows", 5: "dense16_taps", 10: "direct_elem",
           11: "grouped16",
           12: "depthwise", 13: "grouped16_rows"}

BIAS_CASES = [
    (wd.ConvShape(4, 64, 56, 56, 64, 3, 3, pad=1), "f32", -1),                 # dense rows, 3x3
    (wd.ConvShape(4, 64, 56, 56, 64, 3, 3, pad=1), "f32", 1),                  # one slice: db written directly
    (wd.ConvShape(2, 64, 12, 12, 96, 3, 3, pad=1), "bf16", 3),                 # 16-bit all-taps (16x16x32 MFMA)
    (wd.ConvShape(2, 64, 12, 12, 64, 3, 3, pad=1), "bf16", 3),                 # 16-bit dense rows, 3x3
    (wd.ConvShape(3, 136, 9, 45, 72, 3, 3, pad=1), "f16", -1),                 # 16-bit all-taps, 3 M / 3 C tiles
    (wd.ConvShape(2, 64, 12, 12, 64, 5, 5, pad=2), "bf16", 3),                 # 16-bit dense rows, 5x5
    (wd.ConvShape(2, 72, 5, 70, 40, 3, 3, pad=1), "f16", 2),                   # 16-bit dense rows, 70-pixel rows
    (wd.ConvShape(2, 6, 9, 9, 10, 3, 3, pad=1), "f32", 3),                    # general dense (Kg % 4 != 0)
    (wd.ConvShape(2, 40, 11, 13, 70, 3, 2, pad=1, stride=2), "f16", 4),        # general dense, stride 2, 2 M tiles
    (wd.ConvShape(2, 40, 11, 13, 72, 3, 2, pad=1, stride=2), "bf16", 4),       # dense rows, stride 2
    (wd.ConvShape(2, 32, 16, 16, 64, 1, 1), "f32", -1),                        # 1x1 streamed
    (wd.ConvShape(2, 96, 20, 20, 128, 1, 1), "f32", 1),                        # 1x1, 2 output tiles, one slice
    (wd.ConvShape(3, 12, 7, 7, 24, 3, 3, pad=1, groups=3), "f32", 4),         # direct, Cg 4 / Kg 8
    (wd.ConvShape(3, 48, 7, 7, 48, 3, 3, pad=1, groups=48), "bf16", 5),        # depthwise
    (wd.ConvShape(3, 384, 14, 14, 384, 7, 7, pad=3, groups=384), "bf16", 3),  # depthwise, 6 channel blocks
    (wd.ConvShape(2, 96, 9, 33, 96, 5, 5, pad=2, groups=96), "f16", 2),        # depthwise, partial second quad
    (wd.ConvShape(2, 80, 6, 120, 80, 3, 3, pad=1, groups=80), "f16", 1),       # depthwise, 2 pixel passes
    (wd.ConvShape(2, 32, 14, 40, 32, 11, 11, pad=5, groups=32), "bf16", 3),    # depthwise, 3 x 3 filter blocks
    (wd.ConvShape(2, 48, 23, 100, 48, 7, 7, pad=3, stride=2, groups=48), "f16", 2),  # depthwise stride 2
    (wd.ConvShape(3, 64, 9, 32, 64, 3, 3, pad=1, groups=16), "f16", -1),       # grouped rows
    (wd.ConvShape(2, 48, 7, 13, 48, 3, 3, pad=0, groups=6), "bf16", 3),        # grouped rows, partial block
    (wd.ConvShape(3, 64, 10, 20, 64, 7, 7, pad=3, groups=16), "f16", 2),       # grouped rows 7x7
    (wd.ConvShape(2, 64, 13, 29, 64, 3, 3, pad=1, stride=2, groups=16), "bf16", 2),  # grouped rows stride 2
    (wd.ConvShape(2, 64, 9, 56, 64, 3, 3, pad=1, groups=16), "f16", 2),        # grouped rows, 64-pixel rows
    (wd.ConvShape(3, 64, 10, 37, 64, 3, 3, pad=1, groups=16), "f16", -1),      # grouped window kernel
    (wd.ConvShape(2, 48, 11, 12, 48, 3, 3, pad=2, dilation=2, groups=6), "bf16", 2),  # grouped generic
    (wd.ConvShape(8, 16, 40, 40, 16, 3, 3, pad=1), "f32", 320),                # > 256 slices: two fold passes
]


def _run(iga, torch, d, plan, xd, dyd, shape, bias):
    dw = torch.full((shape.K, shape.R, shape.S, shape.Cg), float("nan"), dtype=torch.float32,
                    device="cuda")
    db = torch.full((shape.K,), float("nan"), dtype=torch.float32, device="cuda")
    ws_bytes = int(plan.ws_bytes)
    ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    if bias:
        iga.conv_wgrad_bias(d, xd.data_ptr(), dyd.data_ptr(), dw.data_ptr(), db.data_ptr(),
                            ws.data_ptr() if ws_bytes else 0, ws_bytes, sp)
    else:
        iga.conv_wgrad_ex(d, xd.data_ptr(), dyd.data_ptr(), dw.data_ptr(),
                          ws.data_ptr() if ws_bytes else 0, ws_bytes, sp)
    torch.cuda.synchronize()
    return dw.cpu().numpy(), db.cpu().numpy()


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import implicit_gemm_amd as iga
    iga.load()


@pytest.mark.parametrize("idx", range(len(BIAS_CASES)))
def test_bias_gradient(idx):
    import torch
    import implicit_gemm_amd as iga
    shp, dtype, split_k = BIAS_CASES[idx]
    d = iga.make_desc(shp.N, shp.C, shp.H, shp.W, shp.K, shp.R, shp.S, shp.pad, shp.stride,
                      shp.dilation, shp.groups, {"f32": 0, "bf16": 1, "f16": 2}[dtype], split_k)
    plan = iga.get_plan(d)
    log("bias", idx, shp, dtype, "split", split_k, "variant", VARIANT[int(plan.variant)],
        "ks", plan.ks_count)
    if split_k == 320:
        assert plan.ks_count > 256
    x, dy = wd.random_inputs(shp, dtype, seed=900 + idx, x_dist=wd.Dist("normal", 1.0),
                             dy_dist=wd.Dist("normal", 0.1))
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    dw1, db1 = _run(iga, torch, d, plan, xd, dyd, shp, True)
    dw2, db2 = _run(iga, torch, d, plan, xd, dyd, shp, True)
    dw0, _ = _run(iga, torch, d, plan, xd, dyd, shp, False)
    assert np.all(np.isfinite(db1)) and np.all(np.isfinite(dw1))
    assert np.array_equal(db1.view(np.uint32), db2.view(np.uint32))
    assert np.array_equal(dw1.view(np.uint32), dw2.view(np.uint32))
    assert np.array_equal(dw1.view(np.uint32), dw0.view(np.uint32))
    ref, den = oracle.bgrad_ref(dy)
    err = oracle.normalised_error(db1.astype(np.float64), ref, den)
    log("  db err %.3e" % err)
    assert err <= oracle.TOL[dtype], (err, shp, dtype, split_k)
    check_against_oracle(x, dy, shp, dtype, split_k=split_k, dw_gpu=dw1.astype(np.float64))


@pytest.mark.parametrize("name", ["c2_3x3_f32", "c3_dw7x7_bf16", "c4a_grp3x3_cpg4_f16",
                                  "c4b_grp3x3_cpg8_f16"])
def test_bias_gradient_workloads(name):
    """The benchmark workloads at full size through the binding's wgrad(bias=True)."""
    import torch
    import implicit_gemm_amd as iga
    wl = wd.WORKLOADS[name]
    s = wl.shape
    log("bias workload", name, s)
    x, dy = wd.make_inputs(wl)
    xd, dyd = to_device(x, wl.dtype), to_device(dy, wl.dtype)
    dw, db = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, bias=True)
    dw_plain = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
    torch.cuda.synchronize()
    assert torch.equal(dw, dw_plain)
    ref, den = oracle.bgrad_ref(dy)
    err = oracle.normalised_error(db.cpu().numpy().astype(np.float64), ref, den)
    log("  db err %.3e" % err)
    assert err <= oracle.TOL[wl.dtype], err
    assert int((db == 0).sum()) == 0
