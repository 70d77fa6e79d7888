"""Convolution weight-gradient oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library (``implicit_gemm_amd``)
never imports it, and the two share no code.

The arithmetic lives in ``wgrad_ref.c`` (plain C, OpenMP, fp64 accumulation):
the weight gradient of a 2-D convolution over NHWC tensors, written out as its
definition (rocm-libraries PR #11188, section Motivation: the ``weight.grad``
of ``nn.Conv2d``).  This module only compiles that file, marshals numpy arrays
into it and finishes the normalised-error metric.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wgrad_ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_wgrad.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH, strict: bool = True) -> str:
    """Compile the C oracle into a shared library with gcc (-O2, OpenMP)."""
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall"]
    cmd += ["-Werror"] if strict else []
    cmd += ["-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building if absent) the oracle library and declare its signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    with _lock:
        if path is None and _lib is not None:
            return _lib
        p = path or _LIB_PATH
        if path is None and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(_SRC)):
            build(force=True)
        lib = ctypes.CDLL(p)
        i64 = ctypes.c_int64
        lib.oracle_out_size.restype = i64
        lib.oracle_out_size.argtypes = [i64] * 5
        lib.oracle_wgrad_accumulate.restype = ctypes.c_int
        lib.oracle_wgrad_accumulate.argtypes = [i64] * 11 + [ctypes.c_void_p] * 4 + [ctypes.c_int]
        lib.oracle_wgrad2_accumulate.restype = ctypes.c_int
        lib.oracle_wgrad2_accumulate.argtypes = [i64] * 14 + [ctypes.c_void_p] * 4 + [ctypes.c_int]
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [i64] * 14 + [ctypes.c_void_p] * 4 + [ctypes.c_int]
        lib.oracle_dgrad.restype = ctypes.c_int
        lib.oracle_dgrad.argtypes = [i64] * 14 + [ctypes.c_void_p] * 4 + [ctypes.c_int]
        lib.oracle_bgrad_accumulate.restype = ctypes.c_int
        lib.oracle_bgrad_accumulate.argtypes = [i64] * 4 + [ctypes.c_void_p] * 3
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        if path is None:
            _lib = lib
        return lib


def default_threads() -> int:
    return max(1, len(os.sched_getaffinity(0)))


def out_size(n_in: int, k: int, pad: int, stride: int, dil: int, lib=None) -> int:
    """Output extent along one axis, from the C oracle."""
    return int((lib or load()).oracle_out_size(n_in, k, pad, stride, dil))


def pair(v):
    """(row, column) value of a geometry argument given as one int or an (h, w) pair."""
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise ValueError("expected an int or an (h, w) pair, got %r" % (v,))
        return int(v[0]), int(v[1])
    return int(v), int(v)


class WgradAccumulator:
    """Streams images through the oracle: dW and the |dY||X| sums in fp64.

    ``pad``, ``stride`` and ``dilation`` are one int (both axes) or an (h, w)
    pair.  ``add(x, dy)`` adds the contribution of a chunk of images; ``dw``
    and ``den`` give the fp64 result [K, R, S, Cg] and max of the |dY|*|X| sums.
    """

    def __init__(self, C, H, W, K, R, S, pad=0, stride=1, dilation=1, groups=1,
                 nthreads=None, lib=None):
        self.lib = lib or load()
        self.C, self.H, self.W, self.K = C, H, W, K
        self.R, self.S = R, S
        self.pad, self.stride, self.dilation, self.groups = pair(pad), pair(stride), pair(dilation), groups
        if C % groups or K % groups:
            raise ValueError("C and K must be divisible by groups")
        self.Cg = C // groups
        self.Ho = out_size(H, R, self.pad[0], self.stride[0], self.dilation[0], self.lib)
        self.Wo = out_size(W, S, self.pad[1], self.stride[1], self.dilation[1], self.lib)
        if self.Ho < 1 or self.Wo < 1:
            raise ValueError("empty output")
        self.nthreads = nthreads or default_threads()
        self._dw = np.zeros((K, R, S, self.Cg), np.float64)
        self._abs = np.zeros((K, R, S, self.Cg), np.float64)
        self.images = 0

    def add(self, x: np.ndarray, dy: np.ndarray) -> None:
        x = np.ascontiguousarray(x, dtype=np.float32)
        dy = np.ascontiguousarray(dy, dtype=np.float32)
        nc = x.shape[0]
        if x.shape != (nc, self.H, self.W, self.C):
            raise ValueError("x shape %r" % (x.shape,))
        if dy.shape != (nc, self.Ho, self.Wo, self.K):
            raise ValueError("dy shape %r, expected %r" % (dy.shape, (nc, self.Ho, self.Wo, self.K)))
        rc = self.lib.oracle_wgrad2_accumulate(
            nc, self.C, self.H, self.W, self.K, self.R, self.S, self.pad[0], self.pad[1],
            self.stride[0], self.stride[1], self.dilation[0], self.dilation[1], self.groups,
            x.ctypes.data, dy.ctypes.data, self._dw.ctypes.data, self._abs.ctypes.data, self.nthreads)
        if rc != 0:
            raise RuntimeError("oracle_wgrad2_accumulate failed: %d" % rc)
        self.images += nc

    @property
    def dw(self) -> np.ndarray:
        return self._dw.copy()

    @property
    def abs_sum(self) -> np.ndarray:
        return self._abs.copy()

    @property
    def den(self) -> float:
        return float(self._abs.max()) if self._abs.size else 0.0


def wgrad_ref(x, dy, R, S, pad=0, stride=1, dilation=1, groups=1, nthreads=None, lib=None):
    """dW (fp64, [K, R, S, C/groups]) and the error denominator for NHWC x, dy.

    pad, stride and dilation: one int for both axes or an (h, w) pair."""
    x = np.asarray(x)
    dy = np.asarray(dy)
    _, H, W, C = x.shape
    K = dy.shape[3]
    acc = WgradAccumulator(C, H, W, K, R, S, pad, stride, dilation, groups, nthreads, lib)
    acc.add(x, dy)
    return acc.dw, acc.den


def bgrad_ref(dy, lib=None):
    """Bias gradient db (fp64, [K]) of NHWC dy, and its error denominator max_k sum |dy[..., k]|."""
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    if dy.ndim != 4:
        raise ValueError("dy must be [N, Ho, Wo, K]")
    n, ho, wo, k = dy.shape
    db = np.zeros(k, np.float64)
    ab = np.zeros(k, np.float64)
    rc = (lib or load()).oracle_bgrad_accumulate(n, ho, wo, k, dy.ctypes.data, db.ctypes.data,
                                                 ab.ctypes.data)
    if rc != 0:
        raise RuntimeError("oracle_bgrad_accumulate failed: %d" % rc)
    return db, float(ab.max()) if ab.size else 0.0


def fwd_ref(x, w, pad=0, stride=1, dilation=1, groups=1, nthreads=None, lib=None):
    """Forward convolution Y (fp64, [N, Ho, Wo, K]) of NHWC x [N,H,W,C] and the
    filter w [K,R,S,C/groups], and its error denominator max over Y of sum |X||W|.
    pad, stride and dilation: one int or an (h, w) pair."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, H, W, C = x.shape
    K, R, S, Cg = w.shape
    (ph, pw), (sh, sw), (dh, dw) = pair(pad), pair(stride), pair(dilation)
    if Cg * groups != C:
        raise ValueError("filter has %d channels per group, expected %d" % (Cg, C // groups))
    lib = lib or load()
    Ho, Wo = out_size(H, R, ph, sh, dh, lib), out_size(W, S, pw, sw, dw, lib)
    if Ho < 1 or Wo < 1:
        raise ValueError("empty output")
    y = np.empty((N, Ho, Wo, K), np.float64)
    a = np.empty((N, Ho, Wo, K), np.float64)
    rc = lib.oracle_fwd(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, x.ctypes.data, w.ctypes.data,
                        y.ctypes.data, a.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_fwd failed: %d" % rc)
    return y, float(a.max())


def dgrad_ref(dy, w, H, W, pad=0, stride=1, dilation=1, groups=1, nthreads=None, lib=None):
    """Data gradient dX (fp64, [N, H, W, C]) of NHWC dy [N,Ho,Wo,K] and the filter
    w [K,R,S,C/groups] for H x W images, and its error denominator max over dX of
    sum |dY||W|.  pad, stride and dilation: one int or an (h, w) pair."""
    dy = np.ascontiguousarray(dy, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, Ho, Wo, K = dy.shape
    Kw, R, S, Cg = w.shape
    if Kw != K:
        raise ValueError("filter has %d output channels, dy has %d" % (Kw, K))
    (ph, pw), (sh, sw), (dh, dw) = pair(pad), pair(stride), pair(dilation)
    lib = lib or load()
    if (out_size(H, R, ph, sh, dh, lib), out_size(W, S, pw, sw, dw, lib)) != (Ho, Wo):
        raise ValueError("dy extents do not match the geometry")
    C = Cg * groups
    dx = np.empty((N, H, W, C), np.float64)
    a = np.empty((N, H, W, C), np.float64)
    rc = lib.oracle_dgrad(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, dy.ctypes.data, w.ctypes.data,
                          dx.ctypes.data, a.ctypes.data, nthreads or default_threads())
    if rc != 0:
        raise RuntimeError("oracle_dgrad failed: %d" % rc)
    return dx, float(a.max())


def normalised_error(dw_test, dw_ref, den) -> float:
    """max |dW - dW_ref| / max(sum |X||dY|); inf when dw_test has NaN/Inf."""
    dw_test = np.asarray(dw_test, dtype=np.float64)
    if not np.all(np.isfinite(dw_test)):
        return float("inf")
    diff = float(np.max(np.abs(dw_test - dw_ref))) if dw_ref.size else 0.0
    if den == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return diff / den


# Acceptance bars of the normalised error: fp32 inputs, and bf16/fp16 inputs.
TOL = {"f32": 1e-5, "bf16": 4e-3, "f16": 4e-3}
