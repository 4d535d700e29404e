"""Pins of the oracle's general 2-D QLinearConv (R11, R25).

ONNX QLinearConv (opset 10): x and w 8-bit with zero points, w per tensor or
per output channel, int32 bias, requantized y; the output size follows the
kernel, strides, pads and dilations, and w is [M, C / group, kH, kW]. The
integer sums are pinned against torch's float64 conv2d of (x - x_zp) and
(w - w_zp) (exact: every partial sum is an integer far below 2^53), with
asymmetric pads applied by torch's pad; the page's printed examples are run
through the general function; the requantization matches the pinned
1x1 oracle where the shapes coincide.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

CASES = [  # (N, C, H, W, M, kH, kW, strides, pads (t, l, b, r), dilations, group)
    (1, 3, 9, 11, 4, 3, 3, (1, 1), (1, 1, 1, 1), (1, 1), 1),
    (2, 4, 8, 8, 6, 3, 3, (2, 2), (1, 1, 1, 1), (1, 1), 2),
    (1, 6, 10, 7, 6, 3, 2, (1, 2), (0, 1, 2, 0), (2, 1), 3),
    (1, 8, 7, 7, 8, 5, 5, (1, 1), (2, 2, 2, 2), (1, 1), 8),   # depthwise
    (2, 2, 5, 6, 3, 1, 1, (2, 3), (0, 0, 1, 1), (1, 1), 1),
    (1, 5, 12, 12, 4, 7, 7, (2, 2), (3, 3, 3, 3), (1, 1), 1),
]


def _torch_acc(x, xz, w, wz, bias, strides, pads, dil, group):
    import torch

    xt = torch.from_numpy(x.astype(np.float64) - xz)
    wt = torch.from_numpy(w.astype(np.float64) - np.asarray(wz, np.float64).reshape(-1, 1, 1, 1))
    xt = torch.nn.functional.pad(xt, (pads[1], pads[3], pads[0], pads[2]))  # zeros = x_zp
    out = torch.nn.functional.conv2d(xt, wt, stride=strides, dilation=dil, groups=group)
    out = out.numpy()
    if bias is not None:
        out = out + bias.reshape(1, -1, 1, 1)
    return np.rint(out).astype(np.int64)


@pytest.mark.parametrize("case", CASES)
@pytest.mark.parametrize("types", [("u8", "i8"), ("i8", "u8"), ("u8", "u8")])
def test_conv2d_sums_match_torch_conv2d(case, types):
    N, C, H, W, M, kH, kW, st, pads, dil, group = case
    r = np.random.default_rng(sum(case[:7]))
    xt, wt = types
    x = (r.integers(0, 256, (N, C, H, W)) if xt == "u8" else r.integers(-128, 128, (N, C, H, W)))
    x = x.astype(np.uint8 if xt == "u8" else np.int8)
    w = (r.integers(0, 256, (M, C // group, kH, kW)) if wt == "u8"
         else r.integers(-128, 128, (M, C // group, kH, kW))).astype(np.uint8 if wt == "u8" else np.int8)
    xz = int(r.integers(0, 256)) if xt == "u8" else int(r.integers(-128, 128))
    wz = (r.integers(0, 256, M) if wt == "u8" else r.integers(-128, 128, M)).astype(np.int32)
    bias = r.integers(-5000, 5000, M).astype(np.int32)
    ws = r.uniform(0.001, 0.01, M).astype(np.float32)
    y, acc = oracle.qlinear_conv2d(x, 0.02, xz, w, ws, wz, 0.5, 3, bias=bias, strides=st, pads=pads,
                                   dilations=dil, group=group, y_type="u8", with_acc=True)
    want = _torch_acc(x, xz, w, wz, bias, st, pads, dil, group)
    assert acc.shape == want.shape
    assert np.array_equal(acc.astype(np.int64), want)


def test_conv2d_requantizes_like_the_pinned_1x1_oracle():
    r = np.random.default_rng(3)
    x = r.integers(0, 256, (2, 16, 5, 7)).astype(np.uint8)
    w = r.integers(-128, 128, (8, 16, 1, 1)).astype(np.int8)
    ws = r.uniform(0.001, 0.004, 8).astype(np.float32)
    b = r.integers(-1000, 1000, 8).astype(np.int32)
    got = oracle.qlinear_conv2d(x, 0.01, 128, w, ws, np.zeros(8, np.int32), 0.02, 128, bias=b)
    want = oracle.qlinear_conv(x, 0.01, 128, w, ws, np.zeros(8, np.int32), 0.02, 128, bias=b)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("fname", ["qlinearconv_u8.json", "qlinearconv_i8.json"])
def test_conv2d_printed_examples(fname):
    g = json.load(open(os.path.join(GOLDEN, fname)))
    dt = {"uint8": np.uint8, "int8": np.int8}
    x = np.array(g["x"], dt[g["x_dtype"]]).reshape(g["x_shape"])
    w = np.array(g["w"], dt[g["w_dtype"]]).reshape(g["w_shape"])
    y = oracle.qlinear_conv2d(x, g["x_scale"], g["x_zero_point"], w, g["w_scale"],
                              g["w_zero_point"], g["y_scale"], g["y_zero_point"])
    assert y.reshape(-1).tolist() == g["y"]


def test_conv2d_padding_reads_the_zero_point():
    # a 3x3 all-ones kernel over a 1x1 image of value x_zp + 5 with pad 1:
    # every output pixel sees the one real pixel (5) and eight pads (0)
    x = np.array([[[[105]]]], np.uint8)
    w = np.ones((1, 1, 3, 3), np.int8)
    y, acc = oracle.qlinear_conv2d(x, 1.0, 100, w, 1.0, 0, 1.0, 0, pads=(1, 1, 1, 1), y_type="u8",
                                   with_acc=True)
    assert acc.reshape(-1).tolist() == [5] and y.reshape(-1).tolist() == [5]
    # stride 2 over a 4x4 image with a 2x2 kernel: four disjoint windows
    x = np.arange(16, dtype=np.uint8).reshape(1, 1, 4, 4)
    y, acc = oracle.qlinear_conv2d(x, 1.0, 0, np.ones((1, 1, 2, 2), np.int8), 1.0, 0, 1.0, 0,
                                   strides=(2, 2), y_type="u8", with_acc=True)
    assert acc.reshape(-1).tolist() == [0 + 1 + 4 + 5, 2 + 3 + 6 + 7, 8 + 9 + 12 + 13, 10 + 11 + 14 + 15]
