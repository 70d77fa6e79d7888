"""ctypes binding of libcwprobes.so: achievable-peak probes of the chip (a streaming
read and an MFMA loop) used by the benchmark beside the published peaks.  They
compute nothing of the weight gradient and are not part of its C ABI."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcwprobes.so")
_lib = None


def load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libcwprobes.so is not built (%s); run `python -m implicit_gemm_amd.build`"
                          % LIB_PATH)
    import torch  # noqa: F401  (one HIP runtime in the process: torch's)
    lib = ctypes.CDLL(LIB_PATH)
    lib.cwprobe_read.restype = ctypes.c_int
    lib.cwprobe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.cwprobe_mfma.restype = ctypes.c_int
    lib.cwprobe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.cwprobe_mfma16.restype = ctypes.c_int
    lib.cwprobe_mfma16.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.cwprobe_lds.restype = ctypes.c_int
    lib.cwprobe_lds.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


def _check(st, what):
    if st != 0:
        from implicit_gemm_amd import ConvWgradError
        raise ConvWgradError(st, what)


def peak_read(src_ptr: int, nbytes: int, blocks: int, sink_ptr: int, stream: int, begin=None,
              end=None) -> None:
    """Streaming-read probe (cwprobe_read): device pointers as integers."""
    _check(load().cwprobe_read(src_ptr, nbytes, blocks, sink_ptr, stream or None, begin, end), "peak_read")


def peak_mfma(dtype: int, iters: int, blocks: int, sink_ptr: int, stream: int, begin=None,
              end=None) -> None:
    """MFMA-loop probe (cwprobe_mfma): sink holds blocks * 256 floats."""
    _check(load().cwprobe_mfma(dtype, iters, blocks, sink_ptr, stream or None, begin, end), "peak_mfma")


def peak_mfma16(iters: int, blocks: int, sink_ptr: int, stream: int, begin=None, end=None) -> None:
    """16x16x32 bf16 MFMA-loop probe (cwprobe_mfma16): sink holds blocks * 256 floats."""
    _check(load().cwprobe_mfma16(iters, blocks, sink_ptr, stream or None, begin, end), "peak_mfma16")


def peak_lds(mode: int, iters: int, blocks: int, sink_ptr: int, stream: int, begin=None, end=None) -> None:
    """LDS-read probe (cwprobe_lds): mode 0 transposed 8-byte, 1 plain 8-byte, 2 plain 16-byte reads."""
    _check(load().cwprobe_lds(mode, iters, blocks, sink_ptr, stream or None, begin, end), "peak_lds")
