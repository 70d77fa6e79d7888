"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no weight-gradient arithmetic: it only draws random tensors
and rounds them to the input dtype.  Both the GPU path and the oracle receive
exactly the arrays produced here.

Recipe: one numpy PCG64 stream per (seed, tensor, image), seeded with
``SeedSequence([seed, tensor_id, n])`` (tensor_id 0 for X, 1 for dY, 2 for a
filter W, whose "images" are its output channels), filled
in NHWC order in float32.  Uniform draws are ``2*U[0,1) - 1``; normal draws are
``sigma * standard_normal``.  For 16-bit configurations the float32 draw is
rounded to bf16 / fp16 with round-to-nearest-even, and the rounded values are
what both sides see.  Per-image streams make batches prefix-consistent: the
first 43 images of a 64-image batch equal the 43-image batch.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

X_ID, DY_ID, W_ID = 0, 1, 2


def _extent(n_in, k, pad, stride, dil):
    # Output size along one axis (needed only to shape dY).
    span = n_in + 2 * pad - dil * (k - 1) - 1
    return span // stride + 1 if span >= 0 else 0


@dataclass(frozen=True)
class ConvShape:
    N: int
    C: int
    H: int
    W: int
    K: int
    R: int
    S: int
    pad: int = 0
    stride: int = 1
    dilation: int = 1
    groups: int = 1

    @property
    def Ho(self):
        return _extent(self.H, self.R, self.pad, self.stride, self.dilation)

    @property
    def Wo(self):
        return _extent(self.W, self.S, self.pad, self.stride, self.dilation)

    @property
    def Cg(self):
        return self.C // self.groups

    def with_n(self, n):
        return ConvShape(n, self.C, self.H, self.W, self.K, self.R, self.S, self.pad,
                         self.stride, self.dilation, self.groups)

    def flops(self):
        """Useful multiply-adds x 2 (group-sparse)."""
        return 2 * self.N * self.Ho * self.Wo * self.K * self.Cg * self.R * self.S

    def algorithmic_bytes(self, in_bytes):
        x = self.N * self.H * self.W * self.C * in_bytes
        dy = self.N * self.Ho * self.Wo * self.K * in_bytes
        dw = self.K * self.R * self.S * self.Cg * 4
        return x + dy + dw


@dataclass(frozen=True)
class Dist:
    kind: str  # "uniform" (U[-1,1]) or "normal"
    sigma: float = 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ConvShape
    dtype: str  # "f32", "bf16", "f16": element type of X and dY
    x_dist: Dist
    dy_dist: Dist
    seed: int
    note: str = ""
    n_sweep: tuple = field(default_factory=tuple)


def _fill_image(seed, tensor_id, n, flat, dist: Dist):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, n])))
    if dist.kind == "uniform":
        rng.random(out=flat, dtype=np.float32)
        flat *= np.float32(2.0)
        flat -= np.float32(1.0)
    elif dist.kind == "normal":
        rng.standard_normal(out=flat, dtype=np.float32)
        flat *= np.float32(dist.sigma)
    else:
        raise ValueError(dist.kind)


def draw_images(seed, tensor_id, n0, count, h, w, c, dist: Dist, out=None, threads=None) -> np.ndarray:
    """float32 [count, h, w, c] for images n0 .. n0+count-1 of one tensor.

    Images are independent streams, so they are drawn on a thread pool; the
    values do not depend on the number of threads.
    """
    if out is None:
        out = np.empty((count, h, w, c), np.float32)
    assert out.shape == (count, h, w, c) and out.dtype == np.float32 and out.flags.c_contiguous
    flat = out.reshape(count, -1)
    threads = threads or min(16, max(1, len(os.sched_getaffinity(0))))
    if count <= 1 or threads == 1 or h * w * c < (1 << 16):
        for i in range(count):
            _fill_image(seed, tensor_id, n0 + i, flat[i], dist)
    else:
        with ThreadPoolExecutor(min(threads, count)) as ex:
            list(ex.map(lambda i: _fill_image(seed, tensor_id, n0 + i, flat[i], dist), range(count)))
    return out


def draw_filter(seed, K, R, S, Cg, dist: Dist, dtype="f32") -> np.ndarray:
    """float32 [K, R, S, Cg] filter (one stream per output channel, tensor id 2),
    rounded to dtype like the activations."""
    return round_to(draw_images(seed, W_ID, 0, K, R, S, Cg, dist), dtype)


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to bf16 / fp16 (RNE); returns the rounded values as float32."""
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(dtype)


def make_inputs(wl: Workload, n0=0, count=None):
    """(x, dy) float32 arrays holding the (rounded) values of images n0 .. n0+count-1."""
    s = wl.shape
    count = s.N - n0 if count is None else count
    x = draw_images(wl.seed, X_ID, n0, count, s.H, s.W, s.C, wl.x_dist)
    dy = draw_images(wl.seed, DY_ID, n0, count, s.Ho, s.Wo, s.K, wl.dy_dist)
    return round_to(x, wl.dtype), round_to(dy, wl.dtype)


def random_inputs(shape: ConvShape, dtype: str, seed: int, x_dist=Dist("uniform"),
                  dy_dist=Dist("uniform")):
    wl = Workload("random", shape, dtype, x_dist, dy_dist, seed)
    return make_inputs(wl)


# The five workloads of the weight-gradient study.  "sigma" is the standard
# deviation of the normal draws.
WORKLOADS = {
    "c1_1x1_tiny_f32": Workload(
        "c1_1x1_tiny_f32", ConvShape(2, 8, 8, 8, 4, 1, 1), "f32",
        Dist("uniform"), Dist("uniform"), seed=1,
        note="1x1 fp32, N=2 C=8 K=4 H=W=8"),
    "c2_3x3_f32": Workload(
        "c2_3x3_f32", ConvShape(32, 64, 56, 56, 64, 3, 3, pad=1), "f32",
        Dist("normal", 1.0), Dist("normal", 0.1), seed=2,
        note="3x3 fp32, N=32 C=K=64 H=W=56 pad 1"),
    "c3_dw7x7_bf16": Workload(
        "c3_dw7x7_bf16", ConvShape(64, 384, 56, 56, 384, 7, 7, pad=3, groups=384), "bf16",
        Dist("normal", 1.0), Dist("normal", 0.1), seed=3,
        note="depthwise 7x7 bf16, N=64 C=K=groups=384 H=W=56 pad 3"),
    "c4a_grp3x3_cpg4_f16": Workload(
        "c4a_grp3x3_cpg4_f16", ConvShape(64, 256, 28, 28, 256, 3, 3, pad=1, groups=64), "f16",
        Dist("normal", 1.0), Dist("normal", 0.1), seed=41,
        note="grouped 3x3 fp16, 4 ch/group, N=64 C=K=256 H=W=28 pad 1"),
    "c4b_grp3x3_cpg8_f16": Workload(
        "c4b_grp3x3_cpg8_f16", ConvShape(64, 256, 28, 28, 256, 3, 3, pad=1, groups=32), "f16",
        Dist("normal", 1.0), Dist("normal", 0.1), seed=42,
        note="grouped 3x3 fp16, 8 ch/group, N=64 C=K=256 H=W=28 pad 1"),
    "c5_1x1_big_f32": Workload(
        "c5_1x1_big_f32", ConvShape(192, 96, 512, 512, 64, 1, 1), "f32",
        Dist("uniform"), Dist("normal", 0.01), seed=5,
        note="1x1 fp32, C=96 K=64 H=W=512, N swept", n_sweep=(43, 64, 96, 128, 192)),
}

# Geometry variants of the same operation (stride, dilation, larger depthwise
# and grouped filters, 16-bit dense), measured beside the five workloads.
def _geo(name, shape, dtype, seed, note):
    return Workload(name, shape, dtype, Dist("normal", 1.0), Dist("normal", 0.1), seed=seed, note=note)


GEOMETRY = {w.name: w for w in [
    _geo("g_dw3x3_bf16", ConvShape(64, 384, 56, 56, 384, 3, 3, pad=1, groups=384), "bf16", 101,
         "depthwise 3x3 bf16, N=64 C=384 56x56 pad 1"),
    _geo("g_dw5x5_bf16", ConvShape(64, 384, 56, 56, 384, 5, 5, pad=2, groups=384), "bf16", 102,
         "depthwise 5x5 bf16, N=64 C=384 56x56 pad 2"),
    _geo("g_dw11x11_bf16", ConvShape(64, 384, 56, 56, 384, 11, 11, pad=5, groups=384), "bf16", 103,
         "depthwise 11x11 bf16, N=64 C=384 56x56 pad 5"),
    _geo("g_dw7x7_s2_bf16", ConvShape(16, 384, 112, 112, 384, 7, 7, pad=3, stride=2, groups=384), "bf16", 104,
         "depthwise 7x7 stride 2 bf16, N=16 C=384 112x112 pad 3"),
    _geo("g_3x3_s2_f32", ConvShape(32, 64, 112, 112, 64, 3, 3, pad=1, stride=2), "f32", 105,
         "3x3 stride 2 fp32, N=32 C=K=64 112x112 pad 1"),
    _geo("g_3x3_d2_f32", ConvShape(32, 64, 56, 56, 64, 3, 3, pad=2, dilation=2), "f32", 106,
         "3x3 dilation 2 fp32, N=32 C=K=64 56x56 pad 2"),
    _geo("g_3x3_bf16", ConvShape(32, 64, 56, 56, 64, 3, 3, pad=1), "bf16", 107,
         "3x3 bf16, N=32 C=K=64 56x56 pad 1"),
    _geo("g_3x3_c256_bf16", ConvShape(64, 256, 14, 14, 256, 3, 3, pad=1), "bf16", 108,
         "3x3 bf16, N=64 C=K=256 14x14 pad 1"),
    _geo("g_grp5x5_cpg4_f16", ConvShape(64, 256, 28, 28, 256, 5, 5, pad=2, groups=64), "f16", 109,
         "grouped 5x5 fp16, 4 ch/group, N=64 C=K=256 28x28 pad 2"),
    _geo("g_grp3x3_cpg4_56_f16", ConvShape(32, 256, 56, 56, 256, 3, 3, pad=1, groups=64), "f16", 110,
         "grouped 3x3 fp16, 4 ch/group, N=32 C=K=256 56x56 pad 1"),
    _geo("g_grp3x3_s2_f16", ConvShape(64, 256, 56, 56, 256, 3, 3, pad=1, stride=2, groups=64), "f16", 111,
         "grouped 3x3 stride 2 fp16, 4 ch/group, N=64 C=K=256 56x56 pad 1"),
    _geo("g_patch16_f32", ConvShape(64, 3, 224, 224, 768, 16, 16, stride=16), "f32", 112,
         "patch embedding 16x16 stride 16 fp32, N=64 C=3 K=768 224x224"),
    _geo("l_3x3_c512_f32", ConvShape(8, 512, 14, 14, 512, 3, 3, pad=1), "f32", 113,
         "small-M 3x3 fp32 layer, N=8 C=K=512 14x14 pad 1 (1568 output pixels, reduction 4608)"),
    _geo("l_3x3_c512_bf16", ConvShape(8, 512, 14, 14, 512, 3, 3, pad=1), "bf16", 114,
         "small-M 3x3 bf16 layer, N=8 C=K=512 14x14 pad 1"),
]}


def workload(name: str) -> Workload:
    """A workload of the study or a geometry variant, by name."""
    if name in WORKLOADS:
        return WORKLOADS[name]
    return GEOMETRY[name]


IN_BYTES = {"f32": 4, "bf16": 2, "f16": 2}
