"""GPU parity of the general 2-D QLinearConv (implicit GEMM) against the CPU
oracle: every output code bit-exact.

Cases: the attribute sets pinned on the CPU (strides, asymmetric pads,
dilations, groups, depthwise, 1x1 with stride), both 8-bit types of x, w
and y, per-tensor and per-channel w zero points (the correction that needs
the per-pixel sums), bias, multi-chunk channel counts, channel tiles that
end inside a group, a ResNet stem (7x7 / 2 over 224x224), and the page's
printed uint8 example.
"""
import json
import os
import zlib

import numpy as np
import pytest

import oracle
from gpu_case import log

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _seed(*key):
    return zlib.crc32(repr(key).encode())


def _codes(r, shape, t):
    return (r.integers(0, 256, shape).astype(np.uint8) if t == "u8"
            else r.integers(-128, 128, shape).astype(np.int8))


def _run(dq, x, x_scale, x_zp, w, w_scale, w_zp, y_scale, y_zp, y_type, *, bias=None, strides=(1, 1),
         pads=(0, 0, 0, 0), dilations=(1, 1), group=1, repeat=1):
    import torch

    N, C, H, W = x.shape
    M, _, kH, kW = w.shape
    T = {"u8": dq.DQ_U8, "i8": dq.DQ_I8}
    tag = lambda a: "u8" if a.dtype == np.uint8 else "i8"  # noqa: E731
    ctx = dq.dq_qconv_init(C, H, W, M, kH, kW, T[tag(x)], T[tag(w)], T[y_type], strides=strides,
                           pads=pads, dilations=dilations, group=group)
    try:
        oH, oW = dq.dq_qconv_output_shape(ctx)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        ws = dev(np.atleast_1d(np.asarray(w_scale, np.float32)))
        wz = None if w_zp is None else dev(np.atleast_1d(np.asarray(w_zp)).astype(w.dtype))
        dq.dq_qconv_set_w(ctx, dev(w), ws, wz, None if bias is None else dev(bias.astype(np.int32)))
        y = torch.empty((N, M, oH, oW), dtype=torch.uint8 if y_type == "u8" else torch.int8,
                        device="cuda")
        xd = dev(x)
        xs = dev(np.array([x_scale], np.float32))
        xz = dev(np.array([x_zp], x.dtype))
        ysd = dev(np.array([y_scale], np.float32))
        yz = dev(np.array([y_zp], np.uint8 if y_type == "u8" else np.int8))
        outs = []
        for _ in range(repeat):
            y.fill_(0)
            dq.dq_qconv_forward(ctx, xd, xs, xz, ysd, yz, y)
            torch.cuda.synchronize()
            outs.append(y.cpu().numpy())
        return outs, dq.dq_qconv_info(ctx)
    finally:
        dq.dq_qconv_release(ctx)


CASES = [  # (N, C, H, W, M, kH, kW, strides, pads, dilations, group)
    (1, 3, 9, 11, 4, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
    (2, 4, 8, 8, 6, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 2),
    (1, 6, 10, 7, 6, 3, 2, (1, 2), (0, 1, 2, 0), (2, 1), 3),
    (1, 8, 7, 7, 8, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 8),
    (2, 2, 5, 6, 3, 1, 1, (2, 3), (0, 0, 1, 1), (1, 1), 1),
    (1, 5, 12, 12, 4, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1), 1),
    (1, 40, 9, 9, 70, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),      # two chunks, two channel tiles
    (1, 64, 6, 20, 130, 3, 3, (1, 1), (0, 2, 1, 3), (1, 2), 2),    # groups of 65 channels
    (2, 33, 17, 3, 65, 2, 3, (3, 1), (2, 0, 0, 1), (1, 1), 1),
    (3, 16, 15, 15, 16, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 16),   # depthwise 3x3
    (2, 6, 13, 10, 6, 3, 3, (2, 1), (1, 0, 2, 1), (2, 1), 6),      # depthwise: strides, dilations, ragged rows
    (1, 4, 9, 9, 4, 2, 4, (1, 3), (0, 1, 1, 2), (1, 1), 4),        # depthwise: even kernel, column stride 3
    (2, 3, 20, 23, 16, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 1),     # virtual channels (kernel column, channel)
    (1, 4, 15, 17, 8, 5, 4, (1, 2), (2, 1, 0, 3), (1, 2), 1),      # virtual channels: 4 channels, column dilation
    (1, 6, 9, 14, 12, 3, 8, (1, 3), (0, 2, 1, 4), (2, 1), 2),      # virtual channels: 8 kernel columns, 2 groups
]


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("types", [("u8", "i8", "u8"), ("i8", "u8", "i8"), ("u8", "u8", "u8")])
@pytest.mark.parametrize("per_channel", [False, True])
def test_qconv_matches_oracle(gpu, case, types, per_channel):
    N, C, H, W, M, kH, kW, st, pads, dil, group = case
    xt, wt, yt = types
    r = np.random.default_rng(_seed(case, types, per_channel))
    x = _codes(r, (N, C, H, W), xt)
    w = _codes(r, (M, C // group, kH, kW), wt)
    nw = M if per_channel else 1
    ws = r.uniform(0.002, 0.01, nw).astype(np.float32)
    lo, hi = (0, 256) if wt == "u8" else (-128, 128)
    wz = r.integers(lo, hi, nw) if per_channel else np.array([128 if wt == "u8" else 0])
    xz = int(r.integers(0, 256)) if xt == "u8" else int(r.integers(-128, 128))
    bias = r.integers(-20000, 20000, M).astype(np.int32)
    ys, yz = np.float32(r.uniform(0.05, 0.5)), (128 if yt == "u8" else 0)
    log(f"qconv {case} {types} per_channel={per_channel}")
    want = oracle.qlinear_conv2d(x, 0.02, xz, w, ws, wz, ys, yz, bias=bias, strides=st, pads=pads,
                                 dilations=dil, group=group, y_type=yt)
    (got,), info = _run(gpu, x, 0.02, xz, w, ws, wz, ys, yz, yt, bias=bias, strides=st, pads=pads,
                        dilations=dil, group=group)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ ({info})"


@pytest.mark.parametrize("shape", [
    (2, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1, 1, 1), 1),      # ResNet stage 1, one wave over channels
    (2, 128, 28, 28, 256, 3, 3, (2, 2), (1, 1, 1, 1), 1),    # stride 2, 256 output channels
    (1, 3, 224, 224, 64, 7, 7, (2, 2), (3, 3, 3, 3), 1),     # the stem: 3 channels in a 32-channel chunk
    (1, 32, 64, 64, 256, 3, 3, (1, 1), (1, 1, 1, 1), 1),    # two MFMA pixel rows a wave
    (2, 96, 28, 28, 96, 3, 3, (1, 1), (1, 1, 1, 1), 96),     # depthwise (a plane a workgroup in LDS)
    (1, 2, 200, 200, 2, 3, 3, (1, 1), (1, 1, 1, 1), 2),      # depthwise plane too large for LDS: the direct kernel
    (2, 96, 28, 28, 192, 3, 3, (2, 2), (0, 0, 1, 1), 96),    # depthwise, two outputs a channel, stride 2
    (20, 64, 56, 56, 64, 3, 3, (1, 1), (1, 1, 1, 1), 1),     # 260 workgroups: two chunks, reduction not split
    (8, 256, 14, 14, 256, 3, 3, (1, 1), (1, 1, 1, 1), 1),    # deep layer: the reduction split over 8 workgroups
    (4, 512, 7, 7, 512, 3, 3, (1, 1), (1, 1, 1, 1), 1),      # deepest ResNet stage, 16 chunks in 8 splits
])
def test_qconv_network_layers(gpu, shape):
    N, C, H, W, M, kH, kW, st, pads, group = shape
    r = np.random.default_rng(_seed(shape))
    x = _codes(r, (N, C, H, W), "u8")
    w = _codes(r, (M, C // group, kH, kW), "i8")
    ws = r.uniform(0.0005, 0.002, M).astype(np.float32)
    bias = r.integers(-5000, 5000, M).astype(np.int32)
    log(f"qconv layer {shape}")
    want = oracle.qlinear_conv2d(x, 0.02, 128, w, ws, np.zeros(M, np.int32), 0.1, 128, bias=bias,
                                 strides=st, pads=pads, group=group, y_type="u8")
    outs, info = _run(gpu, x, 0.02, 128, w, ws, None, 0.1, 128, "u8", bias=bias, strides=st, pads=pads,
                      group=group, repeat=2)
    for got in outs:
        assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ ({info})"


@pytest.mark.parametrize("shape", [
    (3, 96, 14, 14, 160, 3, 3, (1, 1), (1, 1, 1, 1), 1),     # split, three chunks, per-channel w zero points
    (2, 70, 9, 13, 33, 3, 2, (2, 1), (0, 1, 2, 0), 1),       # split with ragged pixels and channels
])
def test_qconv_split_reduction_with_pixel_sums(gpu, shape):
    """The split path with w zero points that differ from w's shift, so the
    per-pixel sums of x travel through the partial buffer too."""
    N, C, H, W, M, kH, kW, st, pads, group = shape
    r = np.random.default_rng(_seed("split", shape))
    x = _codes(r, (N, C, H, W), "u8")
    w = _codes(r, (M, C // group, kH, kW), "i8")
    ws = r.uniform(0.0005, 0.002, M).astype(np.float32)
    wz = r.integers(-128, 128, M)
    bias = r.integers(-5000, 5000, M).astype(np.int32)
    log(f"qconv split {shape}")
    want = oracle.qlinear_conv2d(x, 0.02, 117, w, ws, wz, 0.1, 128, bias=bias, strides=st, pads=pads,
                                 group=group, y_type="u8")
    outs, info = _run(gpu, x, 0.02, 117, w, ws, wz, 0.1, 128, "u8", bias=bias, strides=st, pads=pads,
                      group=group, repeat=2)
    for got in outs:
        assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ ({info})"


def test_qconv_printed_uint8_example(gpu):
    g = json.load(open(os.path.join(GOLDEN, "qlinearconv_u8.json")))
    x = np.array(g["x"], np.uint8).reshape(g["x_shape"])
    w = np.array(g["w"], np.uint8).reshape(g["w_shape"])
    (got,), _ = _run(gpu, x, g["x_scale"], g["x_zero_point"], w, g["w_scale"], g["w_zero_point"],
                     g["y_scale"], g["y_zero_point"], "u8")
    assert got.reshape(-1).tolist() == g["y"]


def test_qconv_printed_int8_example(gpu):
    g = json.load(open(os.path.join(GOLDEN, "qlinearconv_i8.json")))
    x = np.array(g["x"], np.int8).reshape(g["x_shape"])
    w = np.array(g["w"], np.int8).reshape(g["w_shape"])
    (got,), _ = _run(gpu, x, g["x_scale"], g["x_zero_point"], w, g["w_scale"], g["w_zero_point"],
                     g["y_scale"], g["y_zero_point"], "i8")
    assert got.reshape(-1).tolist() == g["y"]


@pytest.mark.parametrize("name", [
    "resnet_3x3_64_56", "resnet_3x3_256_56", "resnet_3x3_256_14", "resnet_stem_7x7_s2",
    "depthwise_3x3_256_56"])
def test_qconv_benchmark_layers_full_size(gpu, name):
    """Each timed ResNet-shaped layer (batch 8) at its full size, seed and
    arguments, in the same launch. The oracle computes a slice of it
    exactly: output image n reads only x[n], and output channel m only
    w[m], its scale, its bias and its group's input channels. The slice is
    the first and last image, with 32 output channels spread over the layer
    (32 whole groups for the depthwise layer)."""
    import workloads

    N, C, H, W, M, k, st, pad, grp = workloads.QCONV_LAYERS[name]
    c = workloads.qconv_layer_case(name)
    log(f"qconv benchmark layer {name}: {workloads.QCONV_LAYERS[name]}")
    x, w = c["x"], c["w"]
    (got,), info = _run(gpu, x, c["x_scale"], 128, w, c["w_scale"], None, c["y_scale"], 128, "u8",
                        bias=c["bias"], strides=(st, st), pads=(pad,) * 4, group=grp)
    imgs = [0, N - 1]
    if grp == 1:
        ms = np.unique(np.linspace(0, M - 1, 32).astype(int))
        xs, g = x[imgs], 1
    else:
        per, cg = M // grp, C // grp
        g0 = grp // 2
        g = min(32, grp - g0)
        ms = np.arange(g0 * per, (g0 + g) * per)
        xs = x[imgs][:, g0 * cg:(g0 + g) * cg]
    want = oracle.qlinear_conv2d(xs, c["x_scale"], 128, w[ms], c["w_scale"][ms], np.zeros(len(ms), np.int32),
                                 c["y_scale"], 128, bias=c["bias"][ms], strides=(st, st), pads=(pad,) * 4,
                                 group=g, y_type="u8")
    part = got[imgs][:, ms]
    assert part.shape == want.shape
    assert np.array_equal(part, want), f"{(part != want).sum()} of {part.size} differ ({info})"


def test_contexts_with_different_patch_sizes_coexist(gpu):
    """The conv kernels' dynamic-LDS limit is one setting per kernel shared
    by every context: a context with a large patch (the 7x7 / 2 stem's, 92
    KiB) keeps running, with the same codes, after a context with a small
    patch has been created and released; a slice checked against the
    oracle."""
    import torch

    log("qconv contexts with different patch sizes")
    r = np.random.default_rng(_seed("coexist"))
    x = _codes(r, (1, 3, 224, 224), "u8")
    w = _codes(r, (64, 3, 7, 7), "i8")
    ws = r.uniform(0.001, 0.01, 64).astype(np.float32)
    bias = r.integers(-2000, 2000, 64).astype(np.int32)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    xs, ys = dev(np.float32([0.02])), dev(np.float32([0.05]))
    z = dev(np.uint8([128]))
    big = gpu.dq_qconv_init(3, 224, 224, 64, 7, 7, gpu.DQ_U8, gpu.DQ_I8, gpu.DQ_U8, strides=(2, 2),
                            pads=(3, 3, 3, 3))
    try:
        oh, ow = gpu.dq_qconv_output_shape(big)
        gpu.dq_qconv_set_w(big, dev(w), dev(ws), None, dev(bias))
        xd = dev(x)
        y = torch.empty((1, 64, oh, ow), dtype=torch.uint8, device="cuda")
        outs = []

        def run_big():
            y.fill_(0)
            gpu.dq_qconv_forward(big, xd, xs, z, ys, z, y)
            torch.cuda.synchronize()
            outs.append(y.cpu().numpy())

        run_big()
        small = gpu.dq_qconv_init(8, 9, 9, 8, 3, 3, gpu.DQ_U8, gpu.DQ_I8, gpu.DQ_U8, pads=(1, 1, 1, 1))
        try:
            gpu.dq_qconv_set_w(small, dev(_codes(r, (8, 8, 3, 3), "i8")), dev(np.float32([0.01])))
            ysm = torch.empty((1, 8, 9, 9), dtype=torch.uint8, device="cuda")
            gpu.dq_qconv_forward(small, dev(_codes(r, (1, 8, 9, 9), "u8")), xs, z, ys, z, ysm)
            run_big()
        finally:
            gpu.dq_qconv_release(small)
        run_big()
    finally:
        gpu.dq_qconv_release(big)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    ms = np.array([0, 21, 42, 63])
    want = oracle.qlinear_conv2d(x, 0.02, 128, w[ms], ws[ms], np.zeros(len(ms), np.int32), 0.05, 128,
                                 bias=bias[ms], strides=(2, 2), pads=(3, 3, 3, 3), group=1, y_type="u8")
    assert np.array_equal(outs[0][:, ms], want)


def _random_conv_cases(seed, n):
    """Seeded random 2-D convolutions: 1 or 2 images, groups (1, 2, 4 or
    depthwise, with a channel multiplier of 1 or 2), 1-80 channels a group,
    kernels 1-7 each way, strides 1-3, dilations 1-2, each pad drawn on its
    own, 1-40 rows and columns; at most about 2e8 multiply-adds a case."""
    r = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        N = int(r.integers(1, 3))
        kH, kW = int(r.integers(1, 8)), int(r.integers(1, 8))
        st = (int(r.integers(1, 4)), int(r.integers(1, 4)))
        dil = (int(r.integers(1, 3)), int(r.integers(1, 3)))
        pads = tuple(int(r.integers(0, k)) if k > 1 else 0 for k in (kH, kW, kH, kW))
        H, W = int(r.integers(1, 41)), int(r.integers(1, 41))
        if H + pads[0] + pads[2] < dil[0] * (kH - 1) + 1 or W + pads[1] + pads[3] < dil[1] * (kW - 1) + 1:
            continue
        kind = int(r.integers(4))
        if kind == 3:  # depthwise
            C = int(r.integers(1, 65))
            group, M = C, C * int(r.integers(1, 3))
        else:
            group = (1, 2, 4)[kind]
            C, M = group * int(r.integers(1, 81)), group * int(r.integers(1, 81))
        oH = (H + pads[0] + pads[2] - dil[0] * (kH - 1) - 1) // st[0] + 1
        oW = (W + pads[1] + pads[3] - dil[1] * (kW - 1) - 1) // st[1] + 1
        if N * M * oH * oW * (C // group) * kH * kW > 2e8:
            continue
        types = [("u8", "i8", "u8"), ("i8", "u8", "i8"), ("u8", "u8", "u8"), ("i8", "i8", "u8")][int(r.integers(4))]
        cases.append(dict(case=(N, C, H, W, M, kH, kW, st, pads, dil, group), types=types,
                          per_channel=bool(r.integers(2)), seed=int(r.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("p", _random_conv_cases(2031, 30), ids=lambda p: "-".join(map(str, p["case"][:7])))
def test_qconv_random_attributes(gpu, p):
    """Every output code bit-exact against the oracle on seeded random
    attribute sets (the kernels picked by shape: implicit GEMM with or
    without virtual channels and split reduction, depthwise, direct)."""
    N, C, H, W, M, kH, kW, st, pads, dil, group = p["case"]
    xt, wt, yt = p["types"]
    r = np.random.default_rng(p["seed"])
    x = _codes(r, (N, C, H, W), xt)
    w = _codes(r, (M, C // group, kH, kW), wt)
    nw = M if p["per_channel"] else 1
    ws = r.uniform(0.002, 0.01, nw).astype(np.float32)
    lo, hi = (0, 256) if wt == "u8" else (-128, 128)
    wz = r.integers(lo, hi, nw) if p["per_channel"] else np.array([128 if wt == "u8" else 0])
    xz = int(r.integers(0, 256)) if xt == "u8" else int(r.integers(-128, 128))
    bias = r.integers(-20000, 20000, M).astype(np.int32)
    ys, yz = np.float32(r.uniform(0.05, 0.5)), (128 if yt == "u8" else 0)
    log(f"qconv random {p['case']} {p['types']} per_channel={p['per_channel']}")
    want = oracle.qlinear_conv2d(x, 0.02, xz, w, ws, wz, ys, yz, bias=bias, strides=st, pads=pads,
                                 dilations=dil, group=group, y_type=yt)
    (got,), info = _run(gpu, x, 0.02, xz, w, ws, wz, ys, yz, yt, bias=bias, strides=st, pads=pads,
                        dilations=dil, group=group)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ ({info})"
