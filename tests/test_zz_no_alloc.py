"""conv_wgrad_noalloc (the entry point for callers that cannot allocate) through the
C ABI, against conv_wgrad_bias / conv_wgrad_ex on the same inputs: two calls in a
row on the library-owned workspace, the second with a smaller input, each to the
parity bar (and, at the same split degree, bit for bit)."""
import ctypes

import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import log, to_device

pytestmark = pytest.mark.gpu

DT = {"f32": 0, "bf16": 1, "f16": 2}


def _lib():
    import implicit_gemm_amd as iga
    lib = iga.load()
    lib.conv_wgrad_noalloc.restype = ctypes.c_int
    lib.conv_wgrad_noalloc.argtypes = [ctypes.POINTER(iga.Desc), ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    return lib


def _run_pair(lib, shape, dtype, seed, with_db, split_k=-1):
    """Existing entry point (caller workspace) and conv_wgrad_noalloc on the same inputs."""
    import torch
    import implicit_gemm_amd as iga
    x, dy = wd.random_inputs(shape, dtype, seed, x_dist=wd.Dist("normal", 1.0), dy_dist=wd.Dist("normal", 0.1))
    xd, dyd = to_device(x, dtype), to_device(dy, dtype)
    d = iga.desc_for(xd, dyd, shape.R, shape.S, shape.pad, shape.stride, shape.dilation, shape.groups,
                     split_k)
    plan = iga.get_plan(d)
    log("noalloc", shape, dtype, "ks", plan.ks_count, "ws bytes", plan.ws_bytes, "db", with_db)
    assert 0 < plan.ws_bytes <= iga.NOALLOC_SCRATCH_BYTES
    ref_dw, ref_db = (iga.wgrad(xd, dyd, shape.R, shape.S, shape.pad, shape.stride, shape.dilation,
                                shape.groups, split_k=split_k, bias=True) if with_db else
                      (iga.wgrad(xd, dyd, shape.R, shape.S, shape.pad, shape.stride, shape.dilation,
                                 shape.groups, split_k=split_k), None))
    dw = torch.full_like(ref_dw, float("nan"))
    db = torch.full((shape.K,), float("nan"), dtype=torch.float32, device=xd.device) if with_db else None
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.conv_wgrad_noalloc(ctypes.byref(d), xd.data_ptr(), dyd.data_ptr(), dw.data_ptr(),
                                db.data_ptr() if with_db else None, stream)
    assert st == 0, iga.STATUS.get(st)
    torch.cuda.synchronize()
    assert torch.equal(dw, ref_dw)                    # same plan, same kernels: the same bits
    ref, den = oracle.wgrad_ref(x, dy, shape.R, shape.S, shape.pad, shape.stride, shape.dilation,
                                shape.groups)
    err = oracle.normalised_error(dw.cpu().numpy(), ref, den)
    assert err <= oracle.TOL[dtype], err
    if with_db:
        assert torch.equal(db, ref_db)
        rb, dden = oracle.bgrad_ref(dy)
        assert oracle.normalised_error(db.cpu().numpy(), rb, dden) <= oracle.TOL[dtype]
    return err


@pytest.mark.parametrize("first,second,split2,dtype", [
    (wd.ConvShape(8, 64, 28, 28, 64, 3, 3, pad=1), wd.ConvShape(4, 32, 20, 20, 48, 3, 3, pad=1), -1, "f32"),
    (wd.ConvShape(8, 128, 20, 20, 128, 7, 7, pad=3, groups=128),
     wd.ConvShape(2, 64, 9, 11, 64, 7, 7, pad=3, groups=64), 3, "bf16"),
    (wd.ConvShape(8, 256, 14, 14, 256, 3, 3, pad=1, groups=64),
     wd.ConvShape(3, 64, 7, 7, 64, 3, 3, pad=1, groups=16), 2, "f16"),
])
def test_noalloc_matches_existing_entry_point_twice(first, second, split2, dtype):
    lib = _lib()
    e1 = _run_pair(lib, first, dtype, 31, True)
    e2 = _run_pair(lib, second, dtype, 32, False, split2)   # smaller input, same shared workspace
    log("noalloc errors", e1, e2)


def test_noalloc_rejects_oversized_workspace_and_bad_args():
    import torch
    import implicit_gemm_amd as iga
    lib = _lib()
    # Pinned split degree whose slabs exceed the library's array: refused, nothing enqueued.
    d = iga.make_desc(64, 96, 512, 512, 64, 1, 1, split_k=4096)
    assert iga.get_plan(d).ws_bytes > iga.NOALLOC_SCRATCH_BYTES
    dw = torch.full((64, 1, 1, 96), 7.0, device="cuda")
    fake = 1 << 20
    assert lib.conv_wgrad_noalloc(ctypes.byref(d), fake, fake, dw.data_ptr(), None, None) == 7
    assert lib.conv_wgrad_noalloc(ctypes.byref(d), None, fake, dw.data_ptr(), None, None) == 1
    torch.cuda.synchronize()
    assert bool((dw == 7.0).all())
