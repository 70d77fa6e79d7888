"""MI355X (gfx950) convolution weight gradient: thin Python binding of libconvwgrad.so.

Every step of the computation runs in the library's HIP kernels; this module
only marshals arguments (descriptor, device pointers, the current HIP stream)
through ctypes.  PyTorch is used for device memory and streams.  There is no
fallback: if the library is missing or a call fails, an exception is raised.

    dw = wgrad(x, dy, R=3, S=3, pad=1)          # x [N,H,W,C], dy [N,Ho,Wo,K] -> dw [K,R,S,C/groups] fp32
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libconvwgrad.so")

F32, BF16, F16 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 64 << 20   # CONV_WGRAD_NOALLOC_SCRATCH_BYTES
PATH_DENSE, PATH_DIRECT = 0, 1

STATUS = {
    0: "OK", 1: "ERR_NULL_ARG", 2: "ERR_BAD_SHAPE", 3: "ERR_BAD_DTYPE", 4: "ERR_BAD_SPLIT",
    5: "ERR_UNSUPPORTED", 6: "ERR_MISALIGNED", 7: "ERR_WORKSPACE", 8: "ERR_HIP",
}


class Desc(ctypes.Structure):
    """conv_wgrad_desc_t."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("N", "C", "H", "W", "K", "R", "S", "pad", "stride", "dilation", "groups")] + \
               [("dtype", ctypes.c_int32), ("split_k", ctypes.c_int32)]


class Plan(ctypes.Structure):
    """conv_wgrad_plan_t."""
    _fields_ = [("path", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("Ho", ctypes.c_int64), ("Wo", ctypes.c_int64), ("L", ctypes.c_int64),
                ("E", ctypes.c_int64), ("unit_rows", ctypes.c_int64), ("units", ctypes.c_int64),
                ("units_per_slice", ctypes.c_int64), ("ks_count", ctypes.c_int32),
                ("needs_reduce", ctypes.c_int32), ("tiles", ctypes.c_int64), ("grid", ctypes.c_int64),
                ("slab_stride", ctypes.c_int64), ("ws_bytes", ctypes.c_uint64),
                ("x_bytes", ctypes.c_uint64), ("dy_bytes", ctypes.c_uint64),
                ("dw_bytes", ctypes.c_uint64), ("windows_4g", ctypes.c_int64)]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class Desc2(ctypes.Structure):
    """conv_wgrad_desc2_t: per-axis geometry, math mode and width fold."""
    _fields_ = [(n, ctypes.c_int64) for n in
                ("N", "C", "H", "W", "K", "R", "S", "pad_h", "pad_w", "stride_h", "stride_w",
                 "dil_h", "dil_w", "groups")] + \
               [(n, ctypes.c_int32) for n in ("dtype", "split_k", "math", "fold_width")]


class Plan2(ctypes.Structure):
    """conv_wgrad_plan2_t."""
    _fields_ = [("base", Plan), ("math", ctypes.c_int32), ("fold_width", ctypes.c_int32)]


MATH = {"exact": 0, "bf16x3": 1}
DIRECTION_WGRAD, DIRECTION_FWD, DIRECTION_DGRAD = 0, 1, 2
VARIANT_FWD, VARIANT_DGRAD = 20, 21
VARIANT_DENSE_BF16X3 = 4
VARIANT_DENSE16_TAPS, VARIANT_DENSE_BF16X3_TAPS = 5, 6
VARIANTS_BF16X3 = (VARIANT_DENSE_BF16X3, VARIANT_DENSE_BF16X3_TAPS)


class ConvWgradError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = STATUS.get(status, "UNKNOWN")
        msg = "%s (%d)" % (self.name, status)
        try:
            msg += ": " + load().conv_wgrad_status_string(status).decode()
        except Exception:  # library itself unavailable
            pass
        super().__init__(msg + (" [%s]" % what if what else ""))


_lib = None


def load():
    """Load libconvwgrad.so (built in-tree by implicit_gemm_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libconvwgrad.so is not built (%s); run `python -m implicit_gemm_amd.build`"
                          % LIB_PATH)
    # torch ships its own HIP runtime under the same soname as ROCm's but asks
    # for it by another name; loaded after this library it would be a second
    # runtime in the process, to which torch's streams belong and this
    # library's launches do not.  Loading torch first makes the library bind
    # to torch's runtime: one runtime, shared streams.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    lib.conv_wgrad_status_string.restype = ctypes.c_char_p
    lib.conv_wgrad_status_string.argtypes = [ctypes.c_int]
    lib.conv_wgrad_workspace_size.restype = ctypes.c_int
    lib.conv_wgrad_workspace_size.argtypes = [P(Desc), P(ctypes.c_size_t)]
    lib.conv_wgrad_get_plan.restype = ctypes.c_int
    lib.conv_wgrad_get_plan.argtypes = [P(Desc), P(Plan)]
    lib.conv_wgrad.restype = ctypes.c_int
    lib.conv_wgrad.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_void_p, ctypes.c_void_p]
    lib.conv_wgrad_ex.restype = ctypes.c_int
    lib.conv_wgrad_ex.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.conv_wgrad_timed.restype = ctypes.c_int
    lib.conv_wgrad_timed.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.conv_wgrad_bias.restype = ctypes.c_int
    lib.conv_wgrad_bias.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.conv_wgrad_bias_timed.restype = ctypes.c_int
    lib.conv_wgrad_bias_timed.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.conv_wgrad2_workspace_size.restype = ctypes.c_int
    lib.conv_wgrad2_workspace_size.argtypes = [P(Desc2), P(ctypes.c_size_t)]
    lib.conv_wgrad2_get_plan.restype = ctypes.c_int
    lib.conv_wgrad2_get_plan.argtypes = [P(Desc2), P(Plan2)]
    lib.conv_wgrad2.restype = ctypes.c_int
    lib.conv_wgrad2.argtypes = [P(Desc2), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.conv_wgrad2_timed.restype = ctypes.c_int
    lib.conv_wgrad2_timed.argtypes = [P(Desc2), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p]
    lib.conv_igemm_get_plan.restype = ctypes.c_int
    lib.conv_igemm_get_plan.argtypes = [P(Desc2), ctypes.c_int32, P(Plan2)]
    lib.conv_igemm_workspace_size.restype = ctypes.c_int
    lib.conv_igemm_workspace_size.argtypes = [P(Desc2), ctypes.c_int32, P(ctypes.c_size_t)]
    for name in ("conv_fwd", "conv_dgrad"):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [P(Desc2), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                      ctypes.c_size_t, ctypes.c_void_p]
    lib.conv_wgrad2_call_timed.restype = ctypes.c_int
    lib.conv_wgrad2_call_timed.argtypes = lib.conv_wgrad2_timed.argtypes
    lib.conv_igemm_call_timed.restype = ctypes.c_int
    lib.conv_igemm_call_timed.argtypes = [P(Desc2), ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.conv_wgrad_noalloc.restype = ctypes.c_int
    lib.conv_wgrad_noalloc.argtypes = [P(Desc), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


def make_desc(N, C, H, W, K, R, S, pad=0, stride=1, dilation=1, groups=1, dtype=F32,
              split_k=-1) -> Desc:
    return Desc(N, C, H, W, K, R, S, pad, stride, dilation, groups, dtype, split_k)


def _pair(v):
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise ValueError("expected an int or an (h, w) pair, got %r" % (v,))
        return int(v[0]), int(v[1])
    return int(v), int(v)


def make_desc2(N, C, H, W, K, R, S, pad=0, stride=1, dilation=1, groups=1, dtype=F32, split_k=-1,
               math="exact", fold_width=-1) -> Desc2:
    """Extended descriptor; pad, stride and dilation are one int or an (h, w) pair."""
    (ph, pw), (sh, sw), (dh, dw) = _pair(pad), _pair(stride), _pair(dilation)
    m = MATH[math] if isinstance(math, str) else int(math)
    return Desc2(N, C, H, W, K, R, S, ph, pw, sh, sw, dh, dw, groups, dtype, split_k, m, fold_width)


def get_plan2(desc: Desc2) -> Plan2:
    p = Plan2()
    st = load().conv_wgrad2_get_plan(ctypes.byref(desc), ctypes.byref(p))
    if st != 0:
        raise ConvWgradError(st, "get_plan2")
    return p


def conv_wgrad2(desc: Desc2, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, ws_ptr: int, ws_bytes: int,
                stream: int) -> None:
    """Raw extended call (db_ptr 0 for the weight gradient only)."""
    st = load().conv_wgrad2(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None, ws_ptr or None,
                            ws_bytes, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad2")


def conv_wgrad2_timed(desc: Desc2, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, ws_ptr: int,
                      ws_bytes: int, stream: int, ev_begin: int, ev_end: int) -> None:
    """conv_wgrad2 whose stage-1 dispatch stamps its start and end into two HIP events."""
    st = load().conv_wgrad2_timed(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None, ws_ptr or None,
                                  ws_bytes, stream or None, ev_begin or None, ev_end or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad2_timed")


def conv_wgrad2_call_timed(desc: Desc2, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, ws_ptr: int,
                           ws_bytes: int, stream: int, ev_begin: int, ev_end: int) -> None:
    """conv_wgrad2 whose first kernel stamps its start and last kernel its end into two HIP events."""
    st = load().conv_wgrad2_call_timed(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None,
                                       ws_ptr or None, ws_bytes, stream or None, ev_begin or None, ev_end or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad2_call_timed")


def get_plan(desc: Desc) -> Plan:
    p = Plan()
    st = load().conv_wgrad_get_plan(ctypes.byref(desc), ctypes.byref(p))
    if st != 0:
        raise ConvWgradError(st, "get_plan")
    return p


def workspace_size(desc: Desc) -> int:
    n = ctypes.c_size_t(0)
    st = load().conv_wgrad_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    if st != 0:
        raise ConvWgradError(st, "workspace_size")
    return int(n.value)


def conv_wgrad(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, ws_ptr: int, stream: int) -> None:
    """Raw call: device pointers as integers; raises on a non-OK status."""
    st = load().conv_wgrad(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, ws_ptr or None, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad")


def conv_wgrad_ex(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, ws_ptr: int, ws_bytes: int,
                  stream: int) -> None:
    st = load().conv_wgrad_ex(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, ws_ptr or None, ws_bytes,
                              stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad_ex")


def conv_wgrad_timed(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, ws_ptr: int, ws_bytes: int,
                     stream: int, ev_begin: int, ev_end: int) -> None:
    """conv_wgrad whose stage-1 dispatch stamps its start and end into two HIP events."""
    st = load().conv_wgrad_timed(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, ws_ptr or None, ws_bytes,
                                 stream or None, ev_begin or None, ev_end or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad_timed")


def conv_wgrad_bias(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, ws_ptr: int,
                    ws_bytes: int, stream: int) -> None:
    """Weight gradient into dw and bias gradient (sum of dy per channel) into db."""
    st = load().conv_wgrad_bias(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None,
                                ws_ptr or None, ws_bytes, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad_bias")


def conv_wgrad_bias_timed(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, ws_ptr: int,
                          ws_bytes: int, stream: int, ev_begin: int, ev_end: int) -> None:
    """conv_wgrad_bias whose stage-1 dispatch stamps its start and end into two HIP events."""
    st = load().conv_wgrad_bias_timed(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None,
                                      ws_ptr or None, ws_bytes, stream or None, ev_begin or None,
                                      ev_end or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad_bias_timed")


def conv_wgrad_noalloc(desc: Desc, x_ptr: int, dy_ptr: int, dw_ptr: int, db_ptr: int, stream: int) -> None:
    """Weight gradient (and the bias gradient when db_ptr is non-zero) with the
    library-owned workspace of NOALLOC_SCRATCH_BYTES per GPU: no allocation."""
    st = load().conv_wgrad_noalloc(ctypes.byref(desc), x_ptr, dy_ptr, dw_ptr, db_ptr or None, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_wgrad_noalloc")


def get_igemm_plan(desc: Desc2, direction: int) -> Plan2:
    """Plan of the forward (DIRECTION_FWD) or data-gradient (DIRECTION_DGRAD) implicit GEMM."""
    p = Plan2()
    st = load().conv_igemm_get_plan(ctypes.byref(desc), direction, ctypes.byref(p))
    if st != 0:
        raise ConvWgradError(st, "conv_igemm_get_plan")
    return p


def conv_fwd(desc: Desc2, x_ptr: int, w_ptr: int, y_ptr: int, ws_ptr: int, ws_bytes: int, stream: int) -> None:
    st = load().conv_fwd(ctypes.byref(desc), x_ptr, w_ptr, y_ptr, ws_ptr or None, ws_bytes, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_fwd")


def conv_dgrad(desc: Desc2, dy_ptr: int, w_ptr: int, dx_ptr: int, ws_ptr: int, ws_bytes: int,
               stream: int) -> None:
    st = load().conv_dgrad(ctypes.byref(desc), dy_ptr, w_ptr, dx_ptr, ws_ptr or None, ws_bytes, stream or None)
    if st != 0:
        raise ConvWgradError(st, "conv_dgrad")


def conv_igemm_call_timed(desc: Desc2, direction: int, src_ptr: int, w_ptr: int, out_ptr: int, ws_ptr: int,
                          ws_bytes: int, stream: int, ev_begin: int, ev_end: int) -> None:
    """conv_fwd / conv_dgrad with the whole call's GPU time in two hipEvent_t handles."""
    st = load().conv_igemm_call_timed(ctypes.byref(desc), direction, src_ptr, w_ptr, out_ptr, ws_ptr or None,
                                      ws_bytes, stream or None, ev_begin or None, ev_end or None)
    if st != 0:
        raise ConvWgradError(st, "conv_igemm_call_timed")


def _igemm_call(direction, src, w, out_shape, desc, split_k, stream, out):
    import torch
    plan = get_igemm_plan(desc, direction).base
    if stream is None:
        stream = torch.cuda.current_stream(src.device)
    with torch.cuda.stream(stream):
        if out is None:
            out = torch.empty(out_shape, dtype=torch.float32, device=src.device)
        ws = torch.empty(max(int(plan.ws_bytes), 16), dtype=torch.uint8, device=src.device)
    if tuple(out.shape) != tuple(out_shape) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("output must be a contiguous float32 tensor of shape %s" % (tuple(out_shape),))
    f = conv_fwd if direction == DIRECTION_FWD else conv_dgrad
    f(desc, src.data_ptr(), w.data_ptr(), out.data_ptr(), ws.data_ptr() if plan.ws_bytes else 0,
      int(plan.ws_bytes), stream.cuda_stream)
    return out


def fwd(x, w, pad=0, stride=1, dilation=1, groups=1, split_k=-1, fold_width=-1, y=None, stream=None):
    """Forward convolution y [N, Ho, Wo, K] (fp32) of NHWC x [N,H,W,C] and the filter
    w [K,R,S,C/groups] (same dtype as x)."""
    if x.dim() != 4 or w.dim() != 4 or x.dtype != w.dtype or x.device != w.device:
        raise ValueError("x [N,H,W,C] and w [K,R,S,Cg] must be 4-D, same dtype and device")
    if not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous")
    N, H, W, C = x.shape
    K, R, S, Cg = w.shape
    if Cg * groups != C:
        raise ValueError("w has %d channels per group, expected %d" % (Cg, C // groups))
    d = make_desc2(N, C, H, W, K, R, S, pad, stride, dilation, groups, _dtype_code(x), split_k, "exact",
                   fold_width)
    plan = get_igemm_plan(d, DIRECTION_FWD).base
    return _igemm_call(DIRECTION_FWD, x, w, (N, plan.Ho, plan.Wo, K), d, split_k, stream, y)


def dgrad(dy, w, H, W, pad=0, stride=1, dilation=1, groups=1, split_k=-1, fold_width=-1, dx=None,
          stream=None):
    """Data gradient dx [N, H, W, C] (fp32) of NHWC dy [N,Ho,Wo,K] and the filter
    w [K,R,S,C/groups] (same dtype as dy) for H x W input images."""
    if dy.dim() != 4 or w.dim() != 4 or dy.dtype != w.dtype or dy.device != w.device:
        raise ValueError("dy [N,Ho,Wo,K] and w [K,R,S,Cg] must be 4-D, same dtype and device")
    if not (dy.is_contiguous() and w.is_contiguous()):
        raise ValueError("dy and w must be contiguous")
    N, Ho, Wo, K = dy.shape
    Kw, R, S, Cg = w.shape
    if Kw != K:
        raise ValueError("w has %d output channels, dy has %d" % (Kw, K))
    C = Cg * groups
    d = make_desc2(N, C, H, W, K, R, S, pad, stride, dilation, groups, _dtype_code(dy), split_k, "exact",
                   fold_width)
    plan = get_igemm_plan(d, DIRECTION_DGRAD).base
    if (plan.Ho, plan.Wo) != (Ho, Wo):
        raise ValueError("dy extents %s do not match the geometry (%d, %d)" % ((Ho, Wo), plan.Ho, plan.Wo))
    return _igemm_call(DIRECTION_DGRAD, dy, w, (N, H, W, C), d, split_k, stream, dx)


def _dtype_code(t):
    import torch
    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in codes:
        raise TypeError("x / dy must be float32, bfloat16 or float16, got %s" % t.dtype)
    return codes[t.dtype]


def desc_for(x, dy, R, S, pad=0, stride=1, dilation=1, groups=1, split_k=-1) -> Desc:
    """Descriptor for NHWC torch tensors x [N,H,W,C] and dy [N,Ho,Wo,K]."""
    if x.dim() != 4 or dy.dim() != 4:
        raise ValueError("x and dy must be 4-D NHWC tensors")
    if x.dtype != dy.dtype:
        raise TypeError("x and dy must have the same dtype")
    N, H, W, C = x.shape
    K = dy.shape[3]
    return make_desc(N, C, H, W, K, R, S, pad, stride, dilation, groups, _dtype_code(x), split_k)


def desc2_for(x, dy, R, S, pad=0, stride=1, dilation=1, groups=1, split_k=-1, math="exact",
              fold_width=-1) -> Desc2:
    """Extended descriptor for NHWC torch tensors x [N,H,W,C] and dy [N,Ho,Wo,K]."""
    if x.dim() != 4 or dy.dim() != 4:
        raise ValueError("x and dy must be 4-D NHWC tensors")
    if x.dtype != dy.dtype:
        raise TypeError("x and dy must have the same dtype")
    N, H, W, C = x.shape
    K = dy.shape[3]
    return make_desc2(N, C, H, W, K, R, S, pad, stride, dilation, groups, _dtype_code(x), split_k, math,
                      fold_width)


def wgrad(x, dy, R, S, pad=0, stride=1, dilation=1, groups=1, split_k=-1, dw=None, workspace=None,
          stream=None, bias=False, db=None, math="exact", fold_width=-1):
    """Weight gradient dW [K, R, S, C/groups] (fp32) of NHWC x and dy on the current HIP stream.

    pad, stride and dilation are one int or an (h, w) pair.  math="bf16x3"
    allows BF16x3 emulation for fp32 inputs where a kernel covers the shape;
    fold_width is the width fold (-1 automatic, 0/1 off, f >= 2 fold by f).
    With bias=True, returns (dW, db) where db [K] (fp32) is the bias gradient,
    the sum of dy over its N, Ho, Wo axes, from the same pass over dy.
    """
    import torch
    d = desc2_for(x, dy, R, S, pad, stride, dilation, groups, split_k, math, fold_width)
    plan = get_plan2(d).base
    if tuple(dy.shape) != (d.N, plan.Ho, plan.Wo, d.K):
        raise ValueError("dy shape %s does not match [N, Ho, Wo, K] = %s"
                         % (tuple(dy.shape), (d.N, plan.Ho, plan.Wo, d.K)))
    if not (x.is_cuda and dy.is_cuda) or x.device != dy.device:
        raise ValueError("x and dy must be on the same GPU")
    if not (x.is_contiguous() and dy.is_contiguous()):
        raise ValueError("x and dy must be contiguous NHWC")
    shape = (d.K, d.R, d.S, d.C // d.groups)   # the unfolded layout (a fold keeps the bytes)
    if dw is not None and (tuple(dw.shape) != shape or dw.dtype != torch.float32 or not dw.is_contiguous()):
        raise ValueError("dw must be a contiguous float32 tensor of shape %s" % (shape,))
    if bias and db is not None and (tuple(db.shape) != (d.K,) or db.dtype != torch.float32
                                    or not db.is_contiguous()):
        raise ValueError("db must be a contiguous float32 tensor of shape (%d,)" % d.K)
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    ws_bytes = plan.ws_bytes
    # Buffers allocated here belong to the stream the work is enqueued on, so
    # the caching allocator does not hand the workspace (dropped on return,
    # while the kernels may still be queued) to another stream's allocation.
    with torch.cuda.stream(stream):
        if dw is None:
            dw = torch.empty(shape, dtype=torch.float32, device=x.device)
        if bias and db is None:
            db = torch.empty((d.K,), dtype=torch.float32, device=x.device)
        if ws_bytes and workspace is None:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    ws_ptr = workspace.data_ptr() if ws_bytes else 0
    ws_len = workspace.numel() * workspace.element_size() if ws_bytes else 0
    conv_wgrad2(d, x.data_ptr(), dy.data_ptr(), dw.data_ptr(), db.data_ptr() if bias else 0, ws_ptr, ws_len,
                stream.cuda_stream)
    return (dw, db) if bias else dw
