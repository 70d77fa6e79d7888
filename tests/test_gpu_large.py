"""1x1 conv wgrad past 4 GB: C=96, K=64, H=W=512, N swept over {43, 64, 96, 128, 192}.

The MIOpen ticket shape (rocm-libraries PR #11188, Motivation / Test Plan)
returned an all-zero weight gradient once the batch pushed X past ~4 GB.  The
inputs are generated once for N=192 (per-image seeded streams, so every
smaller N is a prefix) and stay on the GPU; each N is one call on a prefix.

The oracle streams every image through its fp64 loops (one image per worker
thread, the per-image partials added in image order) and computes the whole
[64, 96] result, so every dW element is compared with it at every N.  No
element may be exactly zero or non-finite.
"""
import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import log

pytestmark = pytest.mark.gpu

CHUNK = 16


def _image_terms(X, Y):
    """fp64 oracle contribution of one image: dW [K, C] and the |dY||X| sums [K, C]."""
    acc = oracle.WgradAccumulator(X.shape[-1], X.shape[0], X.shape[1], Y.shape[-1], 1, 1, nthreads=1)
    acc.add(X[None], Y[None])
    return acc.dw[:, 0, 0, :], acc.abs_sum[:, 0, 0, :]


@pytest.mark.timeout(900)
def test_large_1x1_sweep_past_4gb():
    import os
    from concurrent.futures import ThreadPoolExecutor
    import torch
    import implicit_gemm_amd as iga
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = wd.WORKLOADS["c5_1x1_big_f32"]
    s = wl.shape
    sweep = list(wl.n_sweep)
    n_max = max(sweep)
    free, _ = torch.cuda.mem_get_info()
    need = n_max * s.H * s.W * (s.C + s.K) * 4
    if free < need + (4 << 30):
        pytest.skip("needs %.1f GB free on the GPU" % (need / 1e9))
    log("large sweep: allocating %.1f GB" % (need / 1e9))
    x = torch.empty((n_max, s.H, s.W, s.C), dtype=torch.float32, device="cuda")
    dy = torch.empty((n_max, s.H, s.W, s.K), dtype=torch.float32, device="cuda")
    xh = torch.empty((CHUNK, s.H, s.W, s.C), dtype=torch.float32, pin_memory=True)
    dyh = torch.empty((CHUNK, s.H, s.W, s.K), dtype=torch.float32, pin_memory=True)
    xa_all, dya_all = xh.numpy(), dyh.numpy()

    def work(i, n):
        wd.draw_images(wl.seed, wd.X_ID, n, 1, s.H, s.W, s.C, wl.x_dist, out=xa_all[i:i + 1], threads=1)
        wd.draw_images(wl.seed, wd.DY_ID, n, 1, s.H, s.W, s.K, wl.dy_dist, out=dya_all[i:i + 1], threads=1)
        return _image_terms(xa_all[i], dya_all[i])

    totals = None
    snap = {}
    done = 0
    threads = min(16, max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(threads) as ex:
        while done < n_max:
            next_point = min(n for n in sweep if n > done)
            cnt = min(CHUNK, next_point - done)  # every sweep point ends a chunk
            terms = list(ex.map(lambda i: work(i, done + i), range(cnt)))
            x[done:done + cnt].copy_(xh[:cnt], non_blocking=True)
            dy[done:done + cnt].copy_(dyh[:cnt], non_blocking=True)
            for t in terms:  # image order: a fixed fp64 summation order
                totals = [a.copy() for a in t] if totals is None else [a + b for a, b in zip(totals, t)]
            torch.cuda.synchronize()  # the staging buffers are refilled by the next chunk
            done += cnt
            if done in sweep:
                snap[done] = [a.copy() for a in totals]
            log("  generated %d / %d images" % (done, n_max))

    for N in sweep:
        d = iga.make_desc(N, s.C, s.H, s.W, s.K, 1, 1)
        plan = iga.get_plan(d)
        log("N=%d x_bytes=%d dy_bytes=%d ks=%d windows=%d" % (N, plan.x_bytes, plan.dy_bytes,
                                                             plan.ks_count, plan.windows_4g))
        dw = iga.wgrad(x[:N], dy[:N], 1, 1)
        torch.cuda.synchronize()
        g = dw.cpu().numpy()[:, 0, 0, :].astype(np.float64)
        assert np.all(np.isfinite(g)), N
        assert int((g == 0).sum()) == 0, "exact zeros at N=%d" % N
        ref, ref_abs = snap[N]
        err = oracle.normalised_error(g, ref, float(ref_abs.max()))
        log("  full dW [%d x %d] normalised error %.3e (max |diff| %.3e, den %.3e)"
            % (g.shape[0], g.shape[1], err, float(np.max(np.abs(g - ref))), float(ref_abs.max())))
        assert err <= oracle.TOL["f32"], (N, err)


@pytest.mark.parametrize("N", [1, 3])
def test_big_image_1x1_full_parity(N):
    """Full element-wise parity on the large-image 1x1 geometry at small N."""
    from gpu_util import check_against_oracle
    wl = wd.WORKLOADS["c5_1x1_big_f32"]
    s = wl.shape.with_n(N)
    log("big-image 1x1 parity N=%d" % N)
    x, dy = wd.make_inputs(wd.Workload(wl.name, s, wl.dtype, wl.x_dist, wl.dy_dist, wl.seed))
    check_against_oracle(x, dy, s, "f32")
