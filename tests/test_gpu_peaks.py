"""The achievable-peak probes of libcwprobes.so (they compute nothing of the
gradient; these tests check that they run, stay in their buffers and time)."""
import ctypes

import numpy as np
import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from implicit_gemm_amd import probes
    probes.load()


def _events():
    hip = ctypes.CDLL("libamdhip64.so.7")
    evs = []
    for _ in range(2):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e)
    return hip, evs


def test_peak_read_leaves_sink_and_times():
    import torch
    from implicit_gemm_amd import probes
    hip, (e0, e1) = _events()
    buf = torch.ones(1 << 18, dtype=torch.float32, device="cuda")      # 1 MiB: every lane's XOR is 0
    sink = torch.full((64 + 1,), 7, dtype=torch.int32, device="cuda")   # one guard word past the blocks
    stream = torch.cuda.current_stream().cuda_stream
    for blocks in (1, 7, 64):
        probes.peak_read(buf.data_ptr(), buf.numel() * 4, blocks, sink.data_ptr(), stream, e0, e1)
        assert hip.hipEventSynchronize(e1) == 0
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1) == 0
        log("peak_read blocks", blocks, "ms", ms.value)
        assert ms.value > 0
    torch.cuda.synchronize()
    assert (sink.cpu().numpy() == 7).all()


@pytest.mark.parametrize("dtype", [0, 1, 2])
def test_peak_mfma_writes_finite_repeatable_sums(dtype):
    import torch
    from implicit_gemm_amd import probes
    blocks = 3
    sink = torch.full((blocks * 256 + 64,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    probes.peak_mfma(dtype, 5, blocks, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    a = sink.cpu().numpy().copy()
    probes.peak_mfma(dtype, 5, blocks, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    b = sink.cpu().numpy()
    assert np.isfinite(a[:blocks * 256]).all() and (a[:blocks * 256] > 0).all()
    assert (a == b).all()
    assert (a[blocks * 256:] == -1.0).all()   # nothing past blocks * 256 floats


def test_peak_mfma16_writes_finite_repeatable_sums():
    import torch
    from implicit_gemm_amd import probes
    blocks = 3
    sink = torch.full((blocks * 256 + 64,), -1.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    probes.peak_mfma16(5, blocks, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    a = sink.cpu().numpy().copy()
    probes.peak_mfma16(5, blocks, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    b = sink.cpu().numpy()
    assert np.isfinite(a[:blocks * 256]).all() and np.array_equal(a, b)
    assert (a[blocks * 256:] == -1.0).all()


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_peak_lds_stays_in_its_sink_and_times(mode):
    import torch
    from implicit_gemm_amd import probes
    hip, (e0, e1) = _events()
    blocks = 8
    sink = torch.full((blocks + 16,), 7, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    probes.peak_lds(mode, 50, blocks, sink.data_ptr(), stream, e0, e1)
    assert hip.hipEventSynchronize(e1) == 0
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1) == 0
    log("peak_lds mode", mode, "ms", ms.value)
    torch.cuda.synchronize()
    assert ms.value > 0 and (sink.cpu().numpy()[blocks:] == 7).all()
