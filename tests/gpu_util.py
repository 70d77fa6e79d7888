"""Helpers for the GPU tests: move seeded inputs to the device and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import wgrad_data as wd

TORCH_DTYPE_NAME = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(a: np.ndarray, dtype: str):
    """Host float32 array (already rounded to dtype) -> contiguous device tensor of dtype."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    t = t.to(getattr(torch, TORCH_DTYPE_NAME[dtype]))
    return t.cuda()


def run_gpu(x, dy, shape: wd.ConvShape, dtype: str, split_k=-1):
    import torch
    import implicit_gemm_amd as iga
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    dw = iga.wgrad(xd, dyd, shape.R, shape.S, shape.pad, shape.stride, shape.dilation, shape.groups,
                   split_k=split_k)
    torch.cuda.synchronize()
    return dw.cpu().numpy().astype(np.float64)


def check_against_oracle(x, dy, shape: wd.ConvShape, dtype: str, split_k=-1, tol=None, dw_gpu=None):
    ref, den = oracle.wgrad_ref(x, dy, shape.R, shape.S, shape.pad, shape.stride, shape.dilation,
                                shape.groups)
    if dw_gpu is None:
        dw_gpu = run_gpu(x, dy, shape, dtype, split_k)
    err = oracle.normalised_error(dw_gpu, ref, den)
    tol = oracle.TOL[dtype] if tol is None else tol
    assert dw_gpu.shape == ref.shape, (dw_gpu.shape, ref.shape)
    assert err <= tol, "normalised error %.3e > %.1e for %s %s split_k=%s" % (err, tol, shape, dtype, split_k)
    return err


def check_bias_against_oracle(dy, db_gpu, dtype: str, tol=None):
    """Bias gradient db [K] from the GPU against the oracle's db = sum of dy per channel."""
    ref, den = oracle.bgrad_ref(dy)
    err = oracle.normalised_error(np.asarray(db_gpu, np.float64), ref, den)
    tol = oracle.TOL[dtype] if tol is None else tol
    assert err <= tol, "bias-gradient normalised error %.3e > %.1e (%s)" % (err, tol, dtype)
    return err
