"""GPU path vs the oracle, element by element, through the C ABI."""
import numpy as np
import pytest

import oracle
import wgrad_data as wd
from gpu_util import check_against_oracle, check_bias_against_oracle, log, run_gpu, to_device

pytestmark = pytest.mark.gpu

SMALL_CONFIGS = ["c1_1x1_tiny_f32", "c2_3x3_f32", "c3_dw7x7_bf16", "c4a_grp3x3_cpg4_f16",
                 "c4b_grp3x3_cpg8_f16"]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import implicit_gemm_amd as iga
    iga.load()


@pytest.mark.parametrize("name", SMALL_CONFIGS)
def test_workload_parity(name):
    wl = wd.WORKLOADS[name]
    log("parity", name, wl.shape, wl.dtype)
    x, dy = wd.make_inputs(wl)
    err = check_against_oracle(x, dy, wl.shape, wl.dtype)
    log("  err %.3e" % err)


def test_hand_examples_on_gpu():
    import json, os
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))["cases"]
    for c in cases:
        shape = wd.ConvShape(c["N"], c["C"], c["H"], c["W"], c["K"], c["R"], c["S"], c["pad"],
                             c["stride"], c["dilation"], c["groups"])
        log("hand", c["name"])
        x = np.array(c["x"], np.float32)
        dy = np.array(c["dy"], np.float32)
        got = run_gpu(x, dy, shape, "f32")
        assert np.array_equal(got, np.array(c["dw"], np.float64)), c["name"]


def _random_shapes(seed, count):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        kind = rng.integers(0, 4)
        if kind == 0:      # dense, mixed channel counts (vector and scalar loads)
            groups = 1
            C, K = int(rng.integers(1, 100)), int(rng.integers(1, 150))
        elif kind == 1:    # grouped with large groups (dense per group)
            groups = int(rng.choice([2, 3, 4]))
            C, K = groups * int(rng.integers(9, 40)), groups * int(rng.integers(9, 40))
        elif kind == 2:    # depthwise
            C = int(rng.integers(1, 80))
            groups, K = C, C
        else:              # small groups (<= 8 channels per group)
            groups = int(rng.integers(2, 12))
            C, K = groups * int(rng.integers(1, 9)), groups * int(rng.integers(1, 9))
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        pad, stride, dil = int(rng.integers(0, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 3))
        N = int(rng.integers(1, 5))
        shp = wd.ConvShape(N, C, H, W, K, R, S, pad, stride, dil, groups)
        if shp.Ho < 1 or shp.Wo < 1:
            continue
        out.append((shp, ["f32", "bf16", "f16"][int(rng.integers(0, 3))]))
    return out


@pytest.mark.parametrize("idx", range(40))
def test_random_shapes(idx):
    shp, dtype = _random_shapes(1234, 40)[idx]
    log("random", idx, shp, dtype)
    x, dy = wd.random_inputs(shp, dtype, seed=1000 + idx)
    check_against_oracle(x, dy, shp, dtype)


EDGE = [
    (wd.ConvShape(1, 1, 1, 1, 1, 1, 1), "f32"),                       # single element
    (wd.ConvShape(1, 3, 1, 1, 5, 3, 3, pad=1), "f32"),                 # 1x1 image, 3x3 filter
    (wd.ConvShape(2, 4, 5, 5, 4, 7, 7, pad=3), "bf16"),                # filter larger than image
    (wd.ConvShape(1, 64, 9, 9, 64, 9, 9, pad=0), "f32"),               # Ho = Wo = 1
    (wd.ConvShape(3, 130, 7, 5, 70, 1, 1), "f32"),                     # ragged tiles in both M and N
    (wd.ConvShape(2, 96, 17, 13, 200, 2, 3, pad=1, stride=2), "f16"),  # R != S, stride 2
    (wd.ConvShape(1, 8, 40, 3, 8, 3, 3, pad=2, dilation=2, groups=8), "bf16"),
    (wd.ConvShape(5, 12, 11, 11, 24, 3, 3, pad=1, stride=3, groups=3), "f32"),  # Cg=4, Kg=8 direct
    (wd.ConvShape(2, 16, 9, 9, 16, 5, 5, pad=0, stride=1, groups=2), "bf16"),   # Cg=8 dense? (Kg=8) direct
    (wd.ConvShape(1, 2, 300, 3, 2, 1, 1, groups=2), "f16"),            # long reduction, tiny output
]


@pytest.mark.parametrize("idx", range(len(EDGE)))
def test_edge_cases(idx):
    shp, dtype = EDGE[idx]
    log("edge", idx, shp, dtype)
    x, dy = wd.random_inputs(shp, dtype, seed=77 + idx)
    check_against_oracle(x, dy, shp, dtype)


@pytest.mark.parametrize("name", ["c2_3x3_f32", "c4b_grp3x3_cpg8_f16", "c1_1x1_tiny_f32"])
@pytest.mark.parametrize("split_k", [1, 2, 3, 7, 64, -1])
def test_split_invariance(name, split_k):
    wl = wd.WORKLOADS[name]
    if name == "c2_3x3_f32":  # a smaller batch keeps the oracle quick
        wl = wd.Workload(wl.name, wl.shape.with_n(4), wl.dtype, wl.x_dist, wl.dy_dist, wl.seed)
    log("split", name, split_k)
    x, dy = wd.make_inputs(wl)
    check_against_oracle(x, dy, wl.shape, wl.dtype, split_k=split_k)


@pytest.mark.parametrize("name,split_k", [("c2_3x3_f32", 5), ("c3_dw7x7_bf16", -1),
                                          ("c4a_grp3x3_cpg4_f16", 3), ("c1_1x1_tiny_f32", 1)])
def test_bitwise_determinism_and_full_overwrite(name, split_k):
    """Three runs at a fixed split degree agree bit for bit; dw and the workspace start as NaN."""
    import torch
    import implicit_gemm_amd as iga
    wl = wd.WORKLOADS[name]
    s = wl.shape
    log("determinism", name, split_k)
    x, dy = wd.make_inputs(wl)
    xd, dyd = to_device(x, wl.dtype), to_device(dy, wl.dtype)
    d = iga.desc_for(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, split_k)
    plan = iga.get_plan(d)
    ws_bytes = plan.ws_bytes
    results = []
    for _ in range(3):
        dw = torch.full((s.K, s.R, s.S, s.Cg), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.full((max(ws_bytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
        iga.conv_wgrad(d, xd.data_ptr(), dyd.data_ptr(), dw.data_ptr(), ws.data_ptr() if ws_bytes else 0,
                       torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        results.append(dw.cpu().numpy())
    assert np.all(np.isfinite(results[0]))
    for r in results[1:]:
        assert np.array_equal(r.view(np.uint32), results[0].view(np.uint32))
    check_against_oracle(x, dy, s, wl.dtype, dw_gpu=results[0].astype(np.float64))


def test_device_pointer_errors():
    import torch
    import implicit_gemm_amd as iga
    x = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    d = iga.make_desc(1, 4, 4, 4, 4, 1, 1, split_k=1)  # one slice: no workspace needed
    with pytest.raises(iga.ConvWgradError) as ei:
        iga.conv_wgrad(d, x.data_ptr() + 4, x.data_ptr(), x.data_ptr(), 0, 0)
    assert ei.value.name == "ERR_MISALIGNED"
    with pytest.raises(iga.ConvWgradError) as ei:
        iga.conv_wgrad(iga.make_desc(1, 4, 4, 4, 4, 1, 1, split_k=0), x.data_ptr(), x.data_ptr(),
                       x.data_ptr(), 0, 0)
    assert ei.value.name == "ERR_BAD_SPLIT"


def test_nonzero_result_stream_and_default_stream():
    """Runs on a non-default stream give the same bits as on the current stream."""
    import torch
    import implicit_gemm_amd as iga
    wl = wd.WORKLOADS["c4b_grp3x3_cpg8_f16"]
    s = wl.shape
    x, dy = wd.make_inputs(wl)
    xd, dyd = to_device(x, wl.dtype), to_device(dy, wl.dtype)
    a = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        b = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert int((a == 0).sum()) == 0


def test_explicit_stream_argument_keeps_workspace():
    """wgrad(stream=st) with st not the current stream: the workspace it allocates is
    dropped on return while the work is still queued on st (behind a sleep), and
    allocations on the current stream made meanwhile must not take its memory."""
    import torch
    import implicit_gemm_amd as iga
    wl = wd.WORKLOADS["c4a_grp3x3_cpg4_f16"]
    s = wl.shape
    x, dy = wd.make_inputs(wl)
    xd, dyd = to_device(x, wl.dtype), to_device(dy, wl.dtype)
    ref = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
    ws_bytes = int(iga.get_plan(iga.desc_for(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation,
                                             s.groups)).ws_bytes)
    assert ws_bytes > 0
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    for _ in range(3):
        with torch.cuda.stream(st):
            torch.cuda._sleep(20_000_000)   # keeps st busy well past the host's next steps
        got = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, stream=st)
        junk = [torch.full((ws_bytes // 4 + 64,), float("nan"), device=xd.device) for _ in range(4)]
        st.synchronize()
        torch.cuda.synchronize()
        del junk
        assert torch.equal(got, ref)


def test_timed_entry_point_events_and_bits():
    """conv_wgrad_timed gives conv_wgrad's bits, and its events bracket a stage-1 dispatch."""
    import ctypes
    import torch
    import implicit_gemm_amd as iga
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    for name in ("c2_3x3_f32", "c4a_grp3x3_cpg4_f16"):
        wl = wd.WORKLOADS[name]
        s = wl.shape
        log("timed entry point", name)
        x, dy = wd.make_inputs(wl)
        xd, dyd = to_device(x, wl.dtype), to_device(dy, wl.dtype)
        ref = iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
        d = iga.desc_for(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups, -1)
        plan = iga.get_plan(d)
        dw = torch.full_like(ref, float("nan"))
        ws = torch.empty(max(int(plan.ws_bytes), 16), dtype=torch.uint8, device=xd.device)
        evs = [ctypes.c_void_p(), ctypes.c_void_p()]
        for e in evs:
            assert hip.hipEventCreate(ctypes.byref(e)) == 0
        sp = torch.cuda.current_stream().cuda_stream
        iga.conv_wgrad_timed(d, xd.data_ptr(), dyd.data_ptr(), dw.data_ptr(), ws.data_ptr(),
                             int(plan.ws_bytes), sp, evs[0].value, evs[1].value)
        assert hip.hipEventSynchronize(evs[1]) == 0
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[0], evs[1]) == 0
        torch.cuda.synchronize()
        for e in evs:
            hip.hipEventDestroy(e)
        assert torch.equal(dw, ref)
        assert 0.0 < ms.value < 1000.0
        # A later launch on the thread does not record into the events again.
        iga.wgrad(xd, dyd, s.R, s.S, s.pad, s.stride, s.dilation, s.groups)
        torch.cuda.synchronize()


SMALL_GROUP_CASES = [
    # depthwise on the 4x4x4 kernel: filter sizes 1..8, pads, widths, ragged rows
    (wd.ConvShape(2, 16, 9, 11, 16, 7, 7, pad=3, groups=16), "bf16", -1),
    (wd.ConvShape(1, 32, 12, 120, 32, 5, 3, pad=2, groups=32), "f16", -1),
    (wd.ConvShape(3, 48, 7, 7, 48, 3, 3, pad=1, groups=48), "bf16", 5),
    (wd.ConvShape(2, 16, 10, 13, 16, 8, 8, pad=4, groups=16), "f16", 3),
    (wd.ConvShape(2, 16, 6, 30, 16, 1, 1, pad=0, groups=16), "bf16", -1),
    (wd.ConvShape(2, 32, 15, 17, 32, 2, 6, pad=0, groups=32), "bf16", 7),
    (wd.ConvShape(4, 16, 5, 6, 16, 7, 7, pad=3, groups=16), "f16", 1),
    (wd.ConvShape(2, 16, 9, 9, 16, 7, 7, pad=0, groups=16), "bf16", -1),      # Ho = Wo = 3
    (wd.ConvShape(2, 80, 6, 120, 80, 3, 3, pad=1, groups=80), "bf16", -1),    # two pixel passes, 5 groups
    (wd.ConvShape(1, 16, 5, 1, 16, 3, 3, pad=1, groups=16), "f16", -1),       # one column
    (wd.ConvShape(2, 32, 7, 20, 32, 3, 3, pad=4, groups=32), "bf16", 2),      # Ho > H, Wo > W
    (wd.ConvShape(2, 64, 8, 64, 64, 5, 5, pad=2, groups=64), "bf16", -1),     # even pad, 72-column rows
    (wd.ConvShape(3, 16, 4, 33, 16, 6, 2, pad=1, groups=16), "f16", 4),       # odd Wo
    (wd.ConvShape(3, 384, 14, 14, 384, 7, 7, pad=3, groups=384), "bf16", 5),  # slices across images
    (wd.ConvShape(2, 16, 6, 10, 16, 3, 3, pad=12, groups=16), "f16", 3),      # pad 12: zero X rows > R - 1
    # depthwise, two channel quads (a partial one), slices across images, stride 2
    (wd.ConvShape(2, 96, 9, 33, 96, 5, 5, pad=2, groups=96), "f16", -1),      # partial second quad
    (wd.ConvShape(3, 128, 12, 56, 128, 7, 7, pad=3, groups=128), "bf16", 5),  # slices across images
    (wd.ConvShape(2, 128, 20, 40, 128, 5, 5, pad=2, stride=2, groups=128), "bf16", 2),  # stride 2
    # depthwise stride 2 (dY rows staged upsampled; X rows advance two per output row)
    (wd.ConvShape(2, 16, 9, 11, 16, 3, 3, pad=1, stride=2, groups=16), "bf16", 2),
    (wd.ConvShape(2, 32, 20, 40, 32, 5, 5, pad=2, stride=2, groups=32), "f16", -1),
    (wd.ConvShape(3, 16, 15, 17, 16, 8, 8, pad=4, stride=2, groups=16), "bf16", 1),   # R = 8: ring guard
    (wd.ConvShape(2, 48, 23, 100, 48, 7, 7, pad=3, stride=2, groups=48), "bf16", 3),  # two pixel passes
    (wd.ConvShape(2, 16, 12, 13, 16, 4, 2, pad=0, stride=2, groups=16), "f16", -1),   # even R, pad 0, odd W
    (wd.ConvShape(4, 64, 7, 7, 64, 3, 3, pad=1, stride=2, groups=64), "bf16", 3),     # slices across images
    # depthwise with 3 x 3 blocks of filter rows / columns (R or S above 8)
    (wd.ConvShape(2, 16, 12, 20, 16, 9, 9, pad=4, groups=16), "bf16", 3),
    (wd.ConvShape(2, 32, 14, 40, 32, 11, 11, pad=5, groups=32), "f16", -1),
    (wd.ConvShape(3, 16, 9, 11, 16, 12, 12, pad=6, groups=16), "bf16", 2),
    (wd.ConvShape(2, 16, 9, 30, 16, 11, 3, pad=5, groups=16), "f16", 2),     # R > 8 only
    (wd.ConvShape(2, 16, 9, 30, 16, 3, 11, pad=5, groups=16), "bf16", -1),   # S > 8 only
    (wd.ConvShape(2, 16, 6, 8, 16, 10, 10, pad=12, groups=16), "f16", 1),    # Ho, Wo > H, W
    (wd.ConvShape(2, 48, 12, 12, 48, 9, 9, pad=0, groups=48), "bf16", -1),   # Ho = Wo = 4, 3 blocks of 16
    (wd.ConvShape(3, 64, 20, 50, 64, 11, 11, pad=5, groups=64), "bf16", 4),  # 56-column rows
    # grouped 16-bit, row-streaming path (stride 1, 1x1 / 3x3, Wo <= 32)
    (wd.ConvShape(3, 64, 9, 32, 64, 3, 3, pad=1, groups=16), "f16", -1),      # Wo = 32, cpg4
    (wd.ConvShape(2, 48, 7, 13, 48, 3, 3, pad=0, groups=6), "bf16", 3),       # cpg8, pad 0, partial block
    (wd.ConvShape(4, 128, 5, 1, 128, 3, 3, pad=1, groups=128), "f16", 5),     # cpg1, one column
    (wd.ConvShape(2, 64, 6, 20, 64, 1, 1, pad=0, groups=4), "bf16", -1),      # cpg16, 1x1
    (wd.ConvShape(5, 32, 3, 7, 32, 3, 3, pad=1, groups=16), "bf16", 4),       # cpg2, slices across images
    (wd.ConvShape(3, 64, 12, 28, 64, 5, 5, pad=2, groups=16), "f16", -1),     # 5x5 cpg4
    (wd.ConvShape(3, 32, 1, 24, 32, 3, 3, pad=1, groups=8), "f16", -1),       # Ho = 1: second half idle
    (wd.ConvShape(4, 64, 2, 17, 64, 3, 3, pad=1, groups=16), "bf16", 3),      # Ho = 2, slices across images
    # grouped row kernel with two 32-pixel k-steps per row (32 < Wo <= 64)
    (wd.ConvShape(2, 64, 9, 56, 64, 3, 3, pad=1, groups=16), "f16", -1),      # Wo = 56
    (wd.ConvShape(3, 128, 7, 64, 128, 3, 3, pad=1, groups=16), "bf16", 3),    # Wo = 64, cpg8
    (wd.ConvShape(2, 48, 8, 33, 48, 1, 1, pad=0, groups=12), "f16", 2),       # Wo = 33, 1x1, partial block
    (wd.ConvShape(2, 64, 10, 45, 64, 7, 7, pad=3, groups=16), "bf16", -1),    # 7x7, Wo = 45
    (wd.ConvShape(3, 32, 6, 40, 32, 5, 5, pad=1, groups=32), "f16", 4),       # 5x5 cpg1, pad < R - 1
    # grouped, stride 2 (X rows staged de-interleaved, two X rows per dY row)
    (wd.ConvShape(2, 64, 13, 29, 64, 3, 3, pad=1, stride=2, groups=16), "f16", 2),     # cpg4
    (wd.ConvShape(3, 128, 16, 64, 128, 3, 3, pad=1, stride=2, groups=16), "bf16", -1), # cpg8, Wo = 32
    (wd.ConvShape(2, 48, 11, 21, 48, 1, 1, pad=0, stride=2, groups=12), "bf16", 3),    # 1x1, partial block
    (wd.ConvShape(2, 64, 14, 30, 64, 5, 5, pad=2, stride=2, groups=64), "f16", -1),    # 5x5 cpg1
    (wd.ConvShape(3, 32, 9, 17, 32, 7, 7, pad=3, stride=2, groups=8), "bf16", 2),      # 7x7 cpg4
    (wd.ConvShape(4, 64, 6, 10, 64, 3, 3, pad=0, stride=2, groups=16), "f16", 3),      # pad 0, slices across images
    (wd.ConvShape(2, 128, 9, 32, 128, 5, 5, pad=4, groups=16), "bf16", 3),    # 5x5 cpg8, pad R - 1
    (wd.ConvShape(3, 64, 10, 20, 64, 7, 7, pad=3, groups=4), "bf16", 2),      # 7x7 cpg16
    (wd.ConvShape(2, 48, 7, 13, 48, 7, 7, pad=0, groups=12), "f16", -1),      # 7x7 cpg4, pad 0, partial block
    # grouped 16-bit: windowed 3x3 / 1x1 paths and the generic path (dilation, 2x2)
    (wd.ConvShape(3, 64, 10, 37, 64, 3, 3, pad=1, groups=16), "f16", -1),
    (wd.ConvShape(2, 128, 9, 9, 128, 1, 1, pad=0, groups=16), "bf16", 3),
    (wd.ConvShape(2, 48, 11, 12, 48, 3, 3, pad=2, dilation=2, groups=6), "bf16", -1),
    (wd.ConvShape(2, 32, 8, 8, 32, 2, 2, pad=1, groups=4), "f16", -1),
    (wd.ConvShape(2, 80, 6, 70, 80, 3, 3, pad=1, groups=10), "bf16", -1),     # two 32-pixel chunks + ragged
]


@pytest.mark.parametrize("idx", range(len(SMALL_GROUP_CASES)))
def test_small_group_kernels(idx):
    import implicit_gemm_amd as iga
    shp, dtype, split_k = SMALL_GROUP_CASES[idx]
    d = iga.make_desc(shp.N, shp.C, shp.H, shp.W, shp.K, shp.R, shp.S, shp.pad, shp.stride,
                      shp.dilation, shp.groups, {"f32": 0, "bf16": 1, "f16": 2}[dtype], split_k)
    plan = iga.get_plan(d)
    log("small-group", idx, shp, dtype, "split", split_k, "variant", plan.variant, "ks", plan.ks_count)
    x, dy = wd.random_inputs(shp, dtype, seed=500 + idx, x_dist=wd.Dist("normal", 1.0),
                             dy_dist=wd.Dist("normal", 0.1))
    check_against_oracle(x, dy, shp, dtype, split_k=split_k)


# Grouped row kernel with slices of one to three output rows, so that segments
# start at every row of the top padding band and below it: the dY rows that
# pair with padding rows above the image enter before the first step (only
# those inside the segment), and the bias gradient counts each dY row once.
GROUPED_SHORT_SLICE_CASES = [
    (wd.ConvShape(1, 64, 9, 20, 64, 7, 7, pad=3, groups=16), "bf16", 9),     # one row per slice
    (wd.ConvShape(2, 64, 8, 24, 64, 5, 5, pad=2, groups=16), "f16", 8),      # two rows per slice
    (wd.ConvShape(1, 32, 11, 17, 32, 7, 7, pad=2, groups=8), "f16", 4),      # three rows, pad < R / 2
    (wd.ConvShape(2, 64, 7, 40, 64, 5, 5, pad=4, groups=16), "bf16", 11),    # pad R - 1, Wo = 44
]


@pytest.mark.parametrize("idx", range(len(GROUPED_SHORT_SLICE_CASES)))
def test_grouped_rows_short_slices(idx):
    import torch
    import implicit_gemm_amd as iga
    shp, dtype, split_k = GROUPED_SHORT_SLICE_CASES[idx]
    d = iga.make_desc(shp.N, shp.C, shp.H, shp.W, shp.K, shp.R, shp.S, shp.pad, shp.stride,
                      shp.dilation, shp.groups, {"f32": 0, "bf16": 1, "f16": 2}[dtype], split_k)
    plan = iga.get_plan(d)
    log("grouped short slices", idx, shp, dtype, "split", split_k, "variant", plan.variant,
        "rows per slice", plan.units_per_slice, "ks", plan.ks_count)
    assert plan.variant == 13 and plan.units_per_slice <= 3
    x, dy = wd.random_inputs(shp, dtype, seed=800 + idx, x_dist=wd.Dist("normal", 1.0),
                             dy_dist=wd.Dist("normal", 0.1))
    dw, db = iga.wgrad(to_device(x, dtype), to_device(dy, dtype), shp.R, shp.S, shp.pad, shp.stride,
                       shp.dilation, shp.groups, split_k=split_k, bias=True)
    torch.cuda.synchronize()
    check_against_oracle(x, dy, shp, dtype, split_k=split_k, dw_gpu=dw.cpu().numpy().astype(np.float64))
    check_bias_against_oracle(dy, db.cpu().numpy(), dtype)


# 16-bit dense kernels with units of several short output rows (the row kernel for
# Wo + SB - 1 <= 32, the all-taps kernel for 3x3 filters): row pitch inside the
# 64-slot unit, Ho not a multiple of the rows per unit, padding 0..3, two tap
# blocks (S = 5, 7), partial channel tiles, slices.
DENSE16_ROW_CASES = [
    (wd.ConvShape(3, 64, 14, 14, 64, 3, 3, pad=1), "bf16", -1),       # 4 rows per unit, last unit 2 rows
    (wd.ConvShape(2, 72, 7, 7, 40, 3, 3, pad=1), "f16", 2),           # 7 rows per unit, partial tiles
    (wd.ConvShape(2, 64, 30, 30, 64, 3, 3, pad=0), "bf16", 3),        # Wo = 28, 2 rows per unit
    (wd.ConvShape(2, 64, 30, 30, 64, 3, 3, pad=1), "f16", -1),        # Wo = 30, pitch 32
    (wd.ConvShape(3, 32, 9, 1, 32, 1, 1), "bf16", 2),                 # Wo = 1: 64 rows per unit
    (wd.ConvShape(2, 64, 12, 12, 136, 5, 5, pad=2), "f16", 4),        # S = 5: two tap blocks, 3 M tiles
    (wd.ConvShape(4, 128, 10, 13, 64, 3, 3, pad=2), "bf16", -1),      # pad 2: Ho, Wo > H - 2
    (wd.ConvShape(2, 64, 16, 16, 64, 3, 3, pad=1, groups=2), "f16", 3),  # two groups of 32 channels
    (wd.ConvShape(3, 64, 14, 14, 64, 5, 5, pad=2), "bf16", -1),       # 5x5, 3 rows of pitch 17 per unit
    (wd.ConvShape(2, 40, 12, 12, 48, 7, 7, pad=3), "f16", 3),         # 7x7: two tap blocks, 4 rows per unit
]


@pytest.mark.parametrize("idx", range(len(DENSE16_ROW_CASES)))
def test_dense16_multirow_units(idx):
    import implicit_gemm_amd as iga
    shp, dtype, split_k = DENSE16_ROW_CASES[idx]
    d = iga.make_desc(shp.N, shp.C, shp.H, shp.W, shp.K, shp.R, shp.S, shp.pad, shp.stride,
                      shp.dilation, shp.groups, {"f32": 0, "bf16": 1, "f16": 2}[dtype], split_k)
    plan = iga.get_plan(d)
    log("dense16 rows", idx, shp, dtype, "split", split_k, "variant", plan.variant,
        "unit_rows", plan.unit_rows, "ks", plan.ks_count)
    # several rows per unit: the row kernel, or the all-taps kernel for 3x3
    # filters with more than 64 input or output channels per group
    taps = (shp.R, shp.S) == (3, 3) and max(shp.C, shp.K) // shp.groups > 64
    assert plan.variant == (5 if taps else 3) and plan.unit_rows > plan.Wo
    x, dy = wd.random_inputs(shp, dtype, seed=700 + idx, x_dist=wd.Dist("normal", 1.0),
                             dy_dist=wd.Dist("normal", 0.1))
    check_against_oracle(x, dy, shp, dtype, split_k=split_k)


# Depthwise slices balanced by the X rows each stages (2..256 slices), or
# uniform (one slice, or more than 256): (N, C, H, W, R, pad, stride, split_k, bias)
DW_BALANCED_CASES = [
    (5, 64, 13, 13, 7, 3, 1, 2, True),      # two slices across five images
    (5, 64, 13, 13, 7, 3, 1, 7, False),     # slices straddling image boundaries
    (5, 64, 13, 13, 7, 3, 1, 13, True),
    (3, 128, 20, 20, 5, 2, 1, 29, False),
    (4, 64, 17, 17, 3, 1, 1, 64, True),     # one row per slice in places
    (4, 64, 33, 33, 7, 3, 2, 11, True),     # stride 2
    (128, 64, 6, 6, 3, 1, 1, 600, False),   # 384 slices: uniform
    (2, 64, 9, 9, 11, 5, 1, 5, True),       # 11x11 (3x3 filter blocks)
]


@pytest.mark.parametrize("idx", range(len(DW_BALANCED_CASES)))
def test_depthwise_balanced_slices(idx):
    import torch
    import implicit_gemm_amd as iga
    N, C, H, W, R, pad, stride, split_k, bias = DW_BALANCED_CASES[idx]
    log("depthwise balanced case", idx, DW_BALANCED_CASES[idx])
    shp = wd.ConvShape(N, C, H, W, C, R, R, pad=pad, stride=stride, groups=C)
    x, dy = wd.make_inputs(wd.Workload("dwb%d" % idx, shp, "bf16", wd.Dist("normal", 1.0), wd.Dist("normal", 0.1),
                                       9700 + idx, ""))
    xd, dyd = to_device(x, "bf16"), to_device(dy, "bf16")
    plan = iga.get_plan(iga.desc_for(xd, dyd, R, R, pad, stride, 1, C, split_k))
    ups = -(-plan.units // min(split_k, plan.units))
    assert plan.variant == 12 and plan.ks_count == -(-plan.units // ups)
    out = iga.wgrad(xd, dyd, R, R, pad, stride, 1, C, split_k=split_k, bias=bias)
    torch.cuda.synchronize()
    got = (out[0] if bias else out).cpu().numpy().astype(np.float64)
    ref, den = oracle.wgrad_ref(x, dy, R, R, pad, stride, 1, C)
    err = oracle.normalised_error(got, ref, den)
    log("  ks", plan.ks_count, "longest slice", plan.units_per_slice, "error %.3e" % err)
    assert err <= oracle.TOL["bf16"]
    assert np.all(np.isfinite(got)) and np.count_nonzero(got == 0.0) == 0
    if bias:
        check_bias_against_oracle(dy, out[1].cpu().numpy(), "bf16")
