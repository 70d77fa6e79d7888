"""Pins of the oracle against facts that do not come from the oracle itself.

Each ``pin_*`` function takes an oracle library handle (so the same pins can
be run against deliberately broken copies of the oracle) and raises
AssertionError when the oracle disagrees with:

* hand-worked examples (``tests/golden/hand_examples.json``);
* finite differences of a forward convolution written independently here
  with numpy padding and strided slicing;
* torch's CPU fp64 convolution and its autograd (a library routine);
* the 1x1 closed form dW = dY^T X on the reshaped [N*H*W, .] matrices
  (the "F.linear on the reshaped tensor" equivalence of rocm-libraries
  PR #11188, section Motivation);
* the X == 1 special cases (the bias gradient db = sum dY for 1x1, and a box
  sum of dY for padded filters);
* depthwise as a per-channel 2-D cross-correlation (scipy.signal);
* bilinearity, batch-split and thread-count invariance (exact for
  integer-valued inputs, whose fp64 sums are exact).
"""
from __future__ import annotations

import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _ref(lib, x, dy, R, S, pad=0, stride=1, dil=1, groups=1, nthreads=4):
    return oracle.wgrad_ref(x, dy, R, S, pad, stride, dil, groups, nthreads=nthreads, lib=lib)


def _extent(n, k, pad, stride, dil):
    span = n + 2 * pad - dil * (k - 1) - 1
    return span // stride + 1 if span >= 0 else 0


def _pair(v):
    return (int(v[0]), int(v[1])) if isinstance(v, (tuple, list)) else (int(v), int(v))


def forward_conv_numpy(x, w, pad, stride, dil, groups):
    """Forward convolution, NHWC x [N,H,W,C], KRSC w [K,R,S,Cg] -> [N,Ho,Wo,K] (fp64).

    pad, stride, dil: one int or an (h, w) pair.  Built from np.pad and strided
    slices: every filter tap (r, s) selects the strided window of the padded
    input that it multiplies.
    """
    N, H, W, C = x.shape
    K, R, S, Cg = w.shape
    Kg = K // groups
    (ph, pw), (sh, sw), (dh, dw) = _pair(pad), _pair(stride), _pair(dil)
    Ho, Wo = _extent(H, R, ph, sh, dh), _extent(W, S, pw, sw, dw)
    xp = np.pad(x.astype(np.float64), ((0, 0), (ph, ph), (pw, pw), (0, 0)))
    y = np.zeros((N, Ho, Wo, K), np.float64)
    for r in range(R):
        for s in range(S):
            win = xp[:, r * dh: r * dh + (Ho - 1) * sh + 1: sh,
                     s * dw: s * dw + (Wo - 1) * sw + 1: sw, :]
            for g in range(groups):
                xs = win[..., g * Cg:(g + 1) * Cg].reshape(-1, Cg)
                ws = w[g * Kg:(g + 1) * Kg, r, s, :].astype(np.float64)
                y[..., g * Kg:(g + 1) * Kg] += (xs @ ws.T).reshape(N, Ho, Wo, Kg)
    return y


def fd_wgrad(x, dy, R, S, pad, stride, dil, groups, rng):
    """dW by central differences of L(W) = <dY, conv(X, W)> around a random W0, step 1.

    L is linear in W, so the difference quotient is exact up to fp64 rounding.
    """
    K = dy.shape[3]
    Cg = x.shape[3] // groups
    w0 = rng.standard_normal((K, R, S, Cg))
    out = np.zeros((K, R, S, Cg))
    dyd = dy.astype(np.float64)
    for idx in np.ndindex(K, R, S, Cg):
        wp = w0.copy()
        wp[idx] += 1.0
        wm = w0.copy()
        wm[idx] -= 1.0
        lp = np.sum(forward_conv_numpy(x, wp, pad, stride, dil, groups) * dyd)
        lm = np.sum(forward_conv_numpy(x, wm, pad, stride, dil, groups) * dyd)
        out[idx] = (lp - lm) / 2.0
    return out


def tiny_shapes(rng, count):
    """Random tiny shapes over the exhaustive grid, each with Ho, Wo >= 1."""
    shapes = []
    while len(shapes) < count:
        N = int(rng.integers(1, 3))
        groups = int(rng.choice([1, 1, 2, 3, 4]))
        Cg = int(rng.integers(1, 4 if groups > 1 else 5))
        Kg = int(rng.integers(1, 4 if groups > 1 else 5))
        C, K = Cg * groups, Kg * groups
        if C > 8 or K > 8:
            continue
        H, W = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        R, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        pad, stride, dil = int(rng.integers(0, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
        if _extent(H, R, pad, stride, dil) < 1 or _extent(W, S, pad, stride, dil) < 1:
            continue
        shapes.append((N, C, H, W, K, R, S, pad, stride, dil, groups))
    return shapes


def _int_inputs(rng, shape, lo=-8, hi=9):
    N, C, H, W, K, R, S, pad, stride, dil, groups = shape
    Ho, Wo = _extent(H, R, pad, stride, dil), _extent(W, S, pad, stride, dil)
    x = rng.integers(lo, hi, (N, H, W, C)).astype(np.float32)
    dy = rng.integers(lo, hi, (N, Ho, Wo, K)).astype(np.float32)
    return x, dy


def pin_hand_examples(lib):
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array(c["x"], np.float32)
        dy = np.array(c["dy"], np.float32)
        want = np.array(c["dw"], np.float64)
        got, _ = _ref(lib, x, dy, c["R"], c["S"], c["pad"], c["stride"], c["dilation"], c["groups"])
        assert got.shape == want.shape, (c["name"], got.shape, want.shape)
        assert np.array_equal(got, want), (c["name"], got, want)


def pin_finite_differences(lib, count=60, seed=11):
    rng = np.random.default_rng(seed)
    for shape in tiny_shapes(rng, count):
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad, stride, dil), _extent(W, S, pad, stride, dil)
        x = rng.uniform(-1, 1, (N, H, W, C)).astype(np.float32)
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        got, den = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        want = fd_wgrad(x, dy, R, S, pad, stride, dil, groups, rng)
        scale = max(den, 1e-30)
        err = np.max(np.abs(got - want)) / scale
        assert err <= 1e-12, (shape, err)


def pin_torch_autograd(lib, count=40, seed=12):
    import torch
    rng = np.random.default_rng(seed)
    for shape in tiny_shapes(rng, count) + [(2, 8, 9, 7, 6, 3, 2, 1, 2, 1, 2),
                                             (1, 6, 10, 10, 6, 5, 5, 2, 1, 1, 6),
                                             (2, 4, 8, 8, 8, 3, 3, 2, 1, 2, 1)]:
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad, stride, dil), _extent(W, S, pad, stride, dil)
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        dy = rng.standard_normal((N, Ho, Wo, K)).astype(np.float32)
        xt = torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2)
        wt = torch.zeros((K, C // groups, R, S), dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(xt, wt, None, stride, pad, dil, groups)
        assert tuple(y.shape) == (N, K, Ho, Wo), (shape, tuple(y.shape))
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        want = wt.grad.permute(0, 2, 3, 1).numpy()
        got, den = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        err = np.max(np.abs(got - want)) / max(den, 1e-30)
        assert err <= 1e-12, (shape, err)


def pin_closed_form_1x1(lib, seed=13):
    rng = np.random.default_rng(seed)
    for (N, C, H, W, K, stride) in [(2, 8, 8, 8, 4, 1), (3, 5, 7, 9, 6, 1), (2, 6, 9, 8, 3, 2),
                                    (1, 16, 11, 5, 12, 3)]:
        Ho, Wo = _extent(H, 1, 0, stride, 1), _extent(W, 1, 0, stride, 1)
        x = rng.uniform(-1, 1, (N, H, W, C)).astype(np.float32)
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        got, den = _ref(lib, x, dy, 1, 1, 0, stride, 1, 1)
        xs = x[:, ::stride, ::stride, :][:, :Ho, :Wo, :].reshape(-1, C).astype(np.float64)
        want = dy.reshape(-1, K).astype(np.float64).T @ xs
        err = np.max(np.abs(got[:, 0, 0, :] - want)) / den
        assert err <= 1e-13, ((N, C, H, W, K, stride), err)


def pin_bias_gradient(lib, seed=14):
    """X == 1 and a 1x1 filter: every dW[k, 0, 0, c] equals db[k] = sum dY[..., k]."""
    rng = np.random.default_rng(seed)
    N, C, H, W, K = 2, 5, 6, 7, 4
    x = np.ones((N, H, W, C), np.float32)
    dy = rng.uniform(-1, 1, (N, H, W, K)).astype(np.float32)
    got, _ = _ref(lib, x, dy, 1, 1)
    db = dy.astype(np.float64).sum(axis=(0, 1, 2))
    for c in range(C):
        assert np.allclose(got[:, 0, 0, c], db, rtol=0, atol=1e-12), (c, got[:, 0, 0, c], db)


def _bgrad(lib, dy):
    return oracle.bgrad_ref(dy, lib=lib)


def pin_bgrad(lib, seed=21):
    """The bias-gradient oracle db[k] = sum dY[..., k] against: integer hand values
    (exact), the weight-gradient oracle at X == 1 with a 1x1 filter (another code
    path), numpy's float64 sum and torch's conv2d bias gradient (library routines),
    and its denominator against numpy's sum of |dY|."""
    # Hand-worked: pixel values 1..6 and 10..60 in two channels -> 21 and 210.
    dy = np.array([[[[1, 10], [2, 20], [3, 30]], [[4, 40], [5, 50], [6, 60]]]], np.float32)
    db, den = _bgrad(lib, dy)
    assert np.array_equal(db, [21.0, 210.0]), db
    assert den == 210.0, den
    dy = -dy
    db, den = _bgrad(lib, dy)
    assert np.array_equal(db, [-21.0, -210.0]) and den == 210.0, (db, den)
    rng = np.random.default_rng(seed)
    import torch
    for (N, Ho, Wo, K) in [(2, 5, 7, 3), (1, 1, 1, 4), (3, 4, 2, 9)]:
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        db, den = _bgrad(lib, dy)
        assert db.shape == (K,)
        want = dy.astype(np.float64).sum(axis=(0, 1, 2))
        assert np.max(np.abs(db - want)) <= 1e-13 * den, (N, Ho, Wo, K)
        assert abs(den - np.abs(dy.astype(np.float64)).sum(axis=(0, 1, 2)).max()) <= 1e-13 * den
        # X == 1, 1x1, stride 1, pad 0: every dW[k, 0, 0, c] is db[k].
        dw, _ = _ref(lib, np.ones((N, Ho, Wo, 3), np.float32), dy, 1, 1)
        for c in range(3):
            assert np.max(np.abs(dw[:, 0, 0, c] - db)) <= 1e-13 * den, c
        # torch: the gradient of a conv2d bias is the sum of the output gradient.
        xt = torch.zeros((N, 2, Ho + 2, Wo + 2), dtype=torch.float64)
        wt = torch.zeros((K, 2, 3, 3), dtype=torch.float64)
        bt = torch.zeros((K,), dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(xt, wt, bt)
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        assert np.max(np.abs(db - bt.grad.numpy())) <= 1e-13 * den, (N, Ho, Wo, K)


def pin_box_sum(lib, seed=15):
    """X == 1, stride 1: dW[k,r,s,c] = sum of dY over the output window where the tap is inside."""
    rng = np.random.default_rng(seed)
    for (N, C, H, W, K, R, S, pad, dil) in [(2, 3, 6, 5, 4, 3, 3, 1, 1), (1, 2, 7, 7, 3, 3, 2, 2, 2),
                                            (1, 1, 5, 6, 2, 5, 5, 2, 1)]:
        Ho, Wo = _extent(H, R, pad, 1, dil), _extent(W, S, pad, 1, dil)
        x = np.ones((N, H, W, C), np.float32)
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        got, _ = _ref(lib, x, dy, R, S, pad, 1, dil, 1)
        for r in range(R):
            h_lo, h_hi = max(0, pad - r * dil), min(Ho, H + pad - r * dil)
            for s in range(S):
                w_lo, w_hi = max(0, pad - s * dil), min(Wo, W + pad - s * dil)
                box = dy[:, h_lo:max(h_lo, h_hi), w_lo:max(w_lo, w_hi), :].astype(np.float64).sum(axis=(0, 1, 2))
                for c in range(C):
                    assert np.allclose(got[:, r, s, c], box, rtol=0, atol=1e-12), (r, s, c)


def pin_depthwise_correlate(lib, seed=16):
    """Depthwise, stride 1, dilation 1: dW[c,:,:,0] = sum_n correlate2d(Xpad[n,:,:,c], dY[n,:,:,c], 'valid')."""
    from scipy.signal import correlate2d
    rng = np.random.default_rng(seed)
    for (N, C, H, W, R, pad) in [(2, 3, 9, 8, 7, 3), (1, 4, 6, 6, 3, 1), (2, 2, 5, 7, 3, 0)]:
        Ho, Wo = _extent(H, R, pad, 1, 1), _extent(W, R, pad, 1, 1)
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        dy = rng.standard_normal((N, Ho, Wo, C)).astype(np.float32)
        got, den = _ref(lib, x, dy, R, R, pad, 1, 1, C)
        want = np.zeros((C, R, R))
        for n in range(N):
            for c in range(C):
                xp = np.pad(x[n, :, :, c].astype(np.float64), pad)
                want[c] += correlate2d(xp, dy[n, :, :, c].astype(np.float64), mode="valid")
        err = np.max(np.abs(got[..., 0] - want)) / den
        assert err <= 1e-13, ((N, C, H, W, R, pad), err)


def pin_grouped_is_dense_per_group(lib, seed=17):
    rng = np.random.default_rng(seed)
    N, H, W, R, S, pad, stride, dil = 2, 7, 6, 3, 3, 1, 1, 1
    for groups, Cg, Kg in [(2, 3, 2), (4, 4, 4), (3, 1, 2)]:
        C, K = groups * Cg, groups * Kg
        x, dy = _int_inputs(rng, (N, C, H, W, K, R, S, pad, stride, dil, groups))
        got, _ = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        for g in range(groups):
            sub, _ = _ref(lib, np.ascontiguousarray(x[..., g * Cg:(g + 1) * Cg]),
                          np.ascontiguousarray(dy[..., g * Kg:(g + 1) * Kg]), R, S, pad, stride, dil, 1)
            assert np.array_equal(got[g * Kg:(g + 1) * Kg], sub), (groups, g)


def pin_bilinear(lib, seed=18):
    """Integer inputs and small integer coefficients: every sum is exact, so equality is exact."""
    rng = np.random.default_rng(seed)
    shape = (2, 4, 7, 6, 6, 3, 3, 1, 2, 1, 2)
    N, C, H, W, K, R, S, pad, stride, dil, groups = shape
    x1, dy1 = _int_inputs(rng, shape)
    x2, dy2 = _int_inputs(rng, shape)
    a, b = 3.0, -2.0
    args = (R, S, pad, stride, dil, groups)
    lhs, _ = _ref(lib, (a * x1 + b * x2).astype(np.float32), dy1, *args)
    rhs = a * _ref(lib, x1, dy1, *args)[0] + b * _ref(lib, x2, dy1, *args)[0]
    assert np.array_equal(lhs, rhs)
    lhs, _ = _ref(lib, x1, (a * dy1 + b * dy2).astype(np.float32), *args)
    rhs = a * _ref(lib, x1, dy1, *args)[0] + b * _ref(lib, x1, dy2, *args)[0]
    assert np.array_equal(lhs, rhs)


def pin_split_invariance(lib, seed=19):
    """Partitions of the batch and of the (n, ho) rows over threads give the same fp64 sum."""
    rng = np.random.default_rng(seed)
    shape = (7, 4, 6, 5, 3, 3, 2, 1, 1, 2, 1)
    N, C, H, W, K, R, S, pad, stride, dil, groups = shape
    x, dy = _int_inputs(rng, shape)
    whole, den = _ref(lib, x, dy, R, S, pad, stride, dil, groups, nthreads=1)
    for nt in (2, 3, 7, 64):
        got, _ = _ref(lib, x, dy, R, S, pad, stride, dil, groups, nthreads=nt)
        assert np.array_equal(got, whole), nt
    for parts in ([3, 4], [1, 1, 5], [2, 2, 2, 1]):
        acc = oracle.WgradAccumulator(C, H, W, K, R, S, pad, stride, dil, groups, nthreads=3, lib=lib)
        n0 = 0
        for p in parts:
            acc.add(x[n0:n0 + p], dy[n0:n0 + p])
            n0 += p
        assert np.array_equal(acc.dw, whole), parts
        assert acc.den == den


def pin_denominator(lib, seed=20):
    """With non-negative inputs the |dY||X| sums equal dW itself; with mixed signs they bound |dW|."""
    rng = np.random.default_rng(seed)
    shape = (2, 4, 6, 6, 4, 3, 3, 1, 1, 1, 2)
    N, C, H, W, K, R, S, pad, stride, dil, groups = shape
    x, dy = _int_inputs(rng, shape, 0, 5)
    acc = oracle.WgradAccumulator(C, H, W, K, R, S, pad, stride, dil, groups, nthreads=2, lib=lib)
    acc.add(x, dy)
    assert np.array_equal(acc.abs_sum, acc.dw)
    assert acc.den == acc.dw.max()
    x, dy = _int_inputs(rng, shape)
    acc = oracle.WgradAccumulator(C, H, W, K, R, S, pad, stride, dil, groups, nthreads=2, lib=lib)
    acc.add(x, dy)
    acc2 = oracle.WgradAccumulator(C, H, W, K, R, S, pad, stride, dil, groups, nthreads=2, lib=lib)
    acc2.add(np.abs(x), np.abs(dy))
    assert np.array_equal(acc.abs_sum, acc2.dw)
    assert np.all(np.abs(acc.dw) <= acc.abs_sum)


def _per_axis_shapes(rng, count):
    """Tiny shapes whose row and column geometry differ."""
    shapes = []
    while len(shapes) < count:
        N = int(rng.integers(1, 3))
        groups = int(rng.choice([1, 1, 2]))
        C, K = groups * int(rng.integers(1, 4)), groups * int(rng.integers(1, 4))
        H, W = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        R, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        pad = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        stride = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dil = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        if pad[0] == pad[1] and stride[0] == stride[1] and dil[0] == dil[1]:
            continue
        if _extent(H, R, pad[0], stride[0], dil[0]) < 1 or _extent(W, S, pad[1], stride[1], dil[1]) < 1:
            continue
        shapes.append((N, C, H, W, K, R, S, pad, stride, dil, groups))
    return shapes


def pin_per_axis_finite_differences(lib, count=40, seed=22):
    """Per-axis pad / stride / dilation: every dW element against central
    differences of the independent numpy forward convolution."""
    rng = np.random.default_rng(seed)
    for shape in _per_axis_shapes(rng, count):
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad[0], stride[0], dil[0]), _extent(W, S, pad[1], stride[1], dil[1])
        x = rng.uniform(-1, 1, (N, H, W, C)).astype(np.float32)
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        got, den = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        want = fd_wgrad(x, dy, R, S, pad, stride, dil, groups, rng)
        err = np.max(np.abs(got - want)) / max(den, 1e-30)
        assert err <= 1e-12, (shape, err)


def pin_per_axis_torch(lib, count=30, seed=23):
    """Per-axis geometry against torch's fp64 conv2d autograd with padding=(ph, pw),
    stride=(sh, sw), dilation=(dh, dw) (a library routine)."""
    import torch
    rng = np.random.default_rng(seed)
    for shape in _per_axis_shapes(rng, count) + [(2, 6, 9, 14, 4, 3, 5, (1, 2), (2, 1), (1, 2), 2),
                                                  (1, 4, 16, 12, 8, 7, 1, (3, 0), (1, 1), (1, 1), 1)]:
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad[0], stride[0], dil[0]), _extent(W, S, pad[1], stride[1], dil[1])
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        dy = rng.standard_normal((N, Ho, Wo, K)).astype(np.float32)
        xt = torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2)
        wt = torch.zeros((K, C // groups, R, S), dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(xt, wt, None, stride, pad, dil, groups)
        assert tuple(y.shape) == (N, K, Ho, Wo), (shape, tuple(y.shape))
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        want = wt.grad.permute(0, 2, 3, 1).numpy()
        got, den = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        err = np.max(np.abs(got - want)) / max(den, 1e-30)
        assert err <= 1e-12, (shape, err)


def pin_axis_swap(lib, seed=24):
    """Transposing the images (H <-> W) with the row and column geometry swapped
    transposes the filter taps: dW'[k, s, r, c] = dW[k, r, s, c], exactly
    (integer inputs, exact sums)."""
    rng = np.random.default_rng(seed)
    for (N, C, H, W, K, R, S, pad, stride, dil, groups) in [(2, 3, 7, 5, 2, 3, 2, (1, 0), (2, 1), (1, 2), 1),
                                                            (1, 4, 6, 9, 4, 2, 3, (0, 2), (1, 3), (2, 1), 2)]:
        x, dy = _int_inputs(rng, (N, C, H, W, K, R, S, 0, 1, 1, groups), lo=-4, hi=5)
        Ho, Wo = _extent(H, R, pad[0], stride[0], dil[0]), _extent(W, S, pad[1], stride[1], dil[1])
        dy = rng.integers(-4, 5, (N, Ho, Wo, K)).astype(np.float32)
        a, _ = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        b, _ = _ref(lib, np.ascontiguousarray(x.transpose(0, 2, 1, 3)), np.ascontiguousarray(dy.transpose(0, 2, 1, 3)),
                    S, R, pad[::-1], stride[::-1], dil[::-1], groups)
        assert np.array_equal(b, a.transpose(0, 2, 1, 3)), (N, C, H, W, K, R, S)


def _fwd(lib, x, w, pad, stride, dil, groups):
    return oracle.fwd_ref(x, w, pad, stride, dil, groups, nthreads=3, lib=lib)


def _dgrad(lib, dy, w, H, W, pad, stride, dil, groups):
    return oracle.dgrad_ref(dy, w, H, W, pad, stride, dil, groups, nthreads=3, lib=lib)


def _mixed_shapes(rng, count):
    """Tiny shapes with equal or per-axis geometry (forward / data-gradient pins)."""
    out = []
    for sh in tiny_shapes(rng, count // 2):
        N, C, H, W, K, R, S, pad, stride, dil, groups = sh
        out.append((N, C, H, W, K, R, S, (pad, pad), (stride, stride), (dil, dil), groups))
    return out + _per_axis_shapes(rng, count - len(out))


def pin_fwd_hand(lib):
    """Forward on the hand-worked cases: 2x2 filter [[1, 0], [0, 2]] over X = 1..9 (3x3),
    no padding: Y[ho, wo] = X[ho, wo] + 2 X[ho+1, wo+1] = [[11, 14], [20, 23]];
    and with pad (1, 0), stride (1, 2) on X = [[1, 2, 3, 4], [5, 6, 7, 8]] and a
    2x1 filter [3, -1]: Y[ho, wo] = 3 Xpad[ho-1, 2wo] - Xpad[ho, 2wo]
    = [[-1, -3], [3 - 5, 9 - 7], [15, 21]] = [[-1, -3], [-2, 2], [15, 21]]."""
    x = np.arange(1, 10, dtype=np.float32).reshape(1, 3, 3, 1)
    w = np.array([1, 0, 0, 2], np.float32).reshape(1, 2, 2, 1)
    y, _ = _fwd(lib, x, w, 0, 1, 1, 1)
    assert np.array_equal(y[0, :, :, 0], [[11, 14], [20, 23]]), y[0, :, :, 0]
    x = np.arange(1, 9, dtype=np.float32).reshape(1, 2, 4, 1)
    w = np.array([3, -1], np.float32).reshape(1, 2, 1, 1)
    y, _ = _fwd(lib, x, w, (1, 0), (1, 2), 1, 1)
    assert np.array_equal(y[0, :, :, 0], [[-1, -3], [-2, 2], [15, 21]]), y[0, :, :, 0]


def pin_fwd_library_routines(lib, count=40, seed=30):
    """Forward against torch's fp64 conv2d and the numpy strided-slice forward."""
    import torch
    rng = np.random.default_rng(seed)
    for shape in _mixed_shapes(rng, count):
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        w = rng.standard_normal((K, R, S, C // groups)).astype(np.float32)
        got, den = _fwd(lib, x, w, pad, stride, dil, groups)
        want = torch.nn.functional.conv2d(torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2),
                                          torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2),
                                          None, stride, pad, dil, groups).permute(0, 2, 3, 1).numpy()
        assert got.shape == want.shape, (shape, got.shape, want.shape)
        assert np.max(np.abs(got - want)) <= 1e-12 * max(den, 1e-30), shape
        want2 = forward_conv_numpy(x, w, pad, stride, dil, groups)
        assert np.max(np.abs(got - want2)) <= 1e-12 * max(den, 1e-30), shape


def pin_fwd_closed_form_1x1(lib, seed=31):
    """1x1 stride 1 forward per group: Y = X W^T on the [N*H*W, .] matrices."""
    rng = np.random.default_rng(seed)
    for (N, C, H, W, K, groups) in [(2, 6, 5, 7, 4, 1), (1, 8, 3, 4, 6, 2)]:
        x = rng.uniform(-1, 1, (N, H, W, C)).astype(np.float32)
        w = rng.uniform(-1, 1, (K, 1, 1, C // groups)).astype(np.float32)
        got, den = _fwd(lib, x, w, 0, 1, 1, groups)
        Cg, Kg = C // groups, K // groups
        for g in range(groups):
            xs = x[..., g * Cg:(g + 1) * Cg].reshape(-1, Cg).astype(np.float64)
            ws = w[g * Kg:(g + 1) * Kg, 0, 0, :].astype(np.float64)
            want = (xs @ ws.T).reshape(N, H, W, Kg)
            assert np.max(np.abs(got[..., g * Kg:(g + 1) * Kg] - want)) <= 1e-13 * den, g


def pin_dgrad_library_routines(lib, count=40, seed=32):
    """Data gradient against torch's fp64 conv2d autograd (the input gradient)."""
    import torch
    rng = np.random.default_rng(seed)
    for shape in _mixed_shapes(rng, count):
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad[0], stride[0], dil[0]), _extent(W, S, pad[1], stride[1], dil[1])
        dy = rng.standard_normal((N, Ho, Wo, K)).astype(np.float32)
        w = rng.standard_normal((K, R, S, C // groups)).astype(np.float32)
        xt = torch.zeros((N, C, H, W), dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(xt, torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2),
                                       None, stride, pad, dil, groups)
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        want = xt.grad.permute(0, 2, 3, 1).numpy()
        got, den = _dgrad(lib, dy, w, H, W, pad, stride, dil, groups)
        assert got.shape == want.shape, shape
        assert np.max(np.abs(got - want)) <= 1e-12 * max(den, 1e-30), shape


def pin_dgrad_finite_differences(lib, count=16, seed=33):
    """Every dX element against central differences (step 1, exact for the linear
    loss <dY, conv(X, W)>) of the independent numpy forward."""
    rng = np.random.default_rng(seed)
    for shape in _mixed_shapes(rng, count):
        N, C, H, W, K, R, S, pad, stride, dil, groups = shape
        Ho, Wo = _extent(H, R, pad[0], stride[0], dil[0]), _extent(W, S, pad[1], stride[1], dil[1])
        dy = rng.uniform(-1, 1, (N, Ho, Wo, K)).astype(np.float32)
        w = rng.uniform(-1, 1, (K, R, S, C // groups)).astype(np.float32)
        x0 = rng.standard_normal((N, H, W, C))
        want = np.zeros((N, H, W, C))
        dyd = dy.astype(np.float64)
        for idx in np.ndindex(N, H, W, C):
            xp, xm = x0.copy(), x0.copy()
            xp[idx] += 1.0
            xm[idx] -= 1.0
            want[idx] = (np.sum(forward_conv_numpy(xp, w, pad, stride, dil, groups) * dyd)
                         - np.sum(forward_conv_numpy(xm, w, pad, stride, dil, groups) * dyd)) / 2.0
        got, den = _dgrad(lib, dy, w, H, W, pad, stride, dil, groups)
        assert np.max(np.abs(got - want)) <= 1e-11 * max(den, 1e-30), shape


def pin_adjoint_identity(lib, seed=34):
    """<dY, fwd(X, W)> = <dgrad(dY, W), X> = <wgrad(X, dY), W>, exactly on integer
    inputs (every sum is exact in fp64): the three oracles are one bilinear form."""
    rng = np.random.default_rng(seed)
    for (N, C, H, W, K, R, S, pad, stride, dil, groups) in [
            (2, 4, 7, 6, 6, 3, 2, (1, 0), (2, 1), (1, 2), 2), (1, 3, 9, 8, 2, 3, 3, 1, 1, 1, 1),
            (2, 8, 6, 9, 8, 2, 4, (0, 2), (1, 3), (2, 1), 8)]:
        (ph, pw), (sh, sw), (dh, dw) = P_pair(pad), P_pair(stride), P_pair(dil)
        Ho, Wo = _extent(H, R, ph, sh, dh), _extent(W, S, pw, sw, dw)
        x = rng.integers(-5, 6, (N, H, W, C)).astype(np.float32)
        dy = rng.integers(-5, 6, (N, Ho, Wo, K)).astype(np.float32)
        w = rng.integers(-5, 6, (K, R, S, C // groups)).astype(np.float32)
        y, _ = _fwd(lib, x, w, pad, stride, dil, groups)
        dx, _ = _dgrad(lib, dy, w, H, W, pad, stride, dil, groups)
        dw_, _ = _ref(lib, x, dy, R, S, pad, stride, dil, groups)
        a = float(np.sum(y * dy.astype(np.float64)))
        b = float(np.sum(dx * x.astype(np.float64)))
        c = float(np.sum(dw_ * w.astype(np.float64)))
        assert a == b == c, (a, b, c)


def pin_fwd_dgrad_denominators(lib, seed=35):
    """With non-negative inputs the |.| sums equal the results; with mixed signs
    they bound them."""
    rng = np.random.default_rng(seed)
    N, C, H, W, K, R, S, pad, stride, dil, groups = 2, 4, 6, 7, 6, 3, 2, (1, 0), (1, 2), 1, 2
    Ho, Wo = _extent(H, R, 1, 1, 1), _extent(W, S, 0, 2, 1)
    x = rng.integers(0, 4, (N, H, W, C)).astype(np.float32)
    w = rng.integers(0, 4, (K, R, S, C // groups)).astype(np.float32)
    dy = rng.integers(0, 4, (N, Ho, Wo, K)).astype(np.float32)
    y, den = _fwd(lib, x, w, pad, stride, dil, groups)
    assert den == y.max()
    dx, den = _dgrad(lib, dy, w, H, W, pad, stride, dil, groups)
    assert den == dx.max()
    # mixed signs: the denominators are the results of |X|, |W| (and |dY|), which bound |Y| and |dX|
    xm, wm, dym = x - 2, w - 2, dy - 2
    y, den = _fwd(lib, xm, wm, pad, stride, dil, groups)
    ya, _ = _fwd(lib, np.abs(xm), np.abs(wm), pad, stride, dil, groups)
    assert den == ya.max() and np.abs(y).max() <= den, (den, ya.max())
    dx, den = _dgrad(lib, dym, wm, H, W, pad, stride, dil, groups)
    dxa, _ = _dgrad(lib, np.abs(dym), np.abs(wm), H, W, pad, stride, dil, groups)
    assert den == dxa.max() and np.abs(dx).max() <= den, (den, dxa.max())


def P_pair(v):
    return _pair(v)


ALL_PINS = [pin_hand_examples, pin_finite_differences, pin_torch_autograd, pin_closed_form_1x1,
            pin_bias_gradient, pin_box_sum, pin_depthwise_correlate, pin_grouped_is_dense_per_group,
            pin_bilinear, pin_split_invariance, pin_denominator, pin_bgrad,
            pin_per_axis_finite_differences, pin_per_axis_torch, pin_axis_swap,
            pin_fwd_hand, pin_fwd_library_routines, pin_fwd_closed_form_1x1, pin_dgrad_library_routines,
            pin_dgrad_finite_differences, pin_adjoint_identity, pin_fwd_dgrad_denominators]
