"""GPU parity of the requantizing 1x1 QLinearConv against the CPU oracle:
every output code bit-exact (both sides divide by y_scale in IEEE fp32 and
round half to even)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_case import log

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dev(a, torch, dtype=None):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    return t.cuda() if dtype is None else t.to(dtype).cuda()


def run_qconv(dq, case):
    import torch

    tmap = {"u8": dq.DQ_U8, "i8": dq.DQ_I8}
    x, w = case["x"], case["w"]
    N, C, HW = x.shape[0], x.shape[1], int(np.prod(x.shape[2:]))
    M = w.shape[0]
    xd = _dev(x.reshape(N, C, HW), torch)
    wd = _dev(w.reshape(M, C), torch)
    xs = _dev(np.atleast_1d(np.float32(case["x_scale"])), torch)
    ys = _dev(np.atleast_1d(np.float32(case["y_scale"])), torch)
    ws = _dev(np.atleast_1d(case["w_scale"]).astype(np.float32), torch)
    xz = None if case["x_zp"] is None else _dev(np.atleast_1d(case["x_zp"]), torch)
    yz = None if case["y_zp"] is None else _dev(np.atleast_1d(case["y_zp"]), torch)
    wz = None if case["w_zp"] is None else _dev(np.atleast_1d(case["w_zp"]), torch)
    b = None if case["bias"] is None else _dev(case["bias"], torch)
    ydt = torch.uint8 if case["y_type"] == "u8" else torch.int8
    y = torch.full((N, M, HW), 7, dtype=ydt, device="cuda")
    dq.qlinear_conv1x1(xd, tmap[case["x_type"]], xs, xz, wd, tmap[case["w_type"]], ws, wz, ys, yz,
                       tmap[case["y_type"]], b, y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def oracle_qconv(case, images=None):
    x = case["x"]
    N, C = x.shape[0], x.shape[1]
    HW = int(np.prod(x.shape[2:]))
    if images is not None:
        x = x[images]
        N = len(images)
    wl = np.atleast_1d(case["w_scale"]).size
    wz = np.zeros(wl, np.int32) if case["w_zp"] is None else np.atleast_1d(case["w_zp"]).astype(np.int32)
    xz = 0 if case["x_zp"] is None else int(np.atleast_1d(case["x_zp"])[0])
    yz = 0 if case["y_zp"] is None else int(np.atleast_1d(case["y_zp"])[0])
    y = oracle.qlinear_conv(x.reshape(N, C, HW, 1), case["x_scale"], xz, case["w"].reshape(case["w"].shape[0], C),
                            np.atleast_1d(case["w_scale"]), wz, case["y_scale"], yz, bias=case["bias"],
                            y_type=case["y_type"])
    return y.reshape(N, -1, HW)


def test_printed_uint8_example(gpu):
    """The QLinearConv page's uint8 example is itself a 1x1 convolution: a
    7x7 uint8 image, w = 0 with w_zero_point 255 (so S[p] is needed), and the
    printed y = 255 - x."""
    log("qconv1x1 printed uint8 example")
    with open(os.path.join(GOLDEN, "qlinearconv_u8.json")) as f:
        g = json.load(f)
    case = dict(x=np.array(g["x"], np.uint8).reshape(g["x_shape"]), x_type="u8",
                x_scale=np.float32(g["x_scale"]), x_zp=np.array([g["x_zero_point"]], np.uint8),
                w=np.array(g["w"], np.uint8).reshape(1, 1), w_type="u8",
                w_scale=np.array(g["w_scale"], np.float32), w_zp=np.array(g["w_zero_point"], np.uint8),
                bias=None, y_scale=np.float32(g["y_scale"]), y_zp=np.array([g["y_zero_point"]], np.uint8),
                y_type="u8")
    got = run_qconv(gpu, case).reshape(-1)
    assert np.array_equal(got, np.array(g["y"], np.uint8))
    assert np.array_equal(got, oracle_qconv(case).reshape(-1))


SWEEP = [
    # N, C, HW, M, x, w, y, per_channel, bias, w_zp
    (1, 1, 1, 1, "u8", "i8", "u8", False, False, False),
    (2, 64, 200, 48, "u8", "i8", "u8", True, True, False),
    (1, 300, 130, 260, "i8", "u8", "i8", False, True, True),
    (3, 17, 64, 5, "u8", "u8", "u8", True, False, True),
    (2, 512, 256, 128, "u8", "i8", "u8", True, True, True),
    (1, 256, 3136, 256, "i8", "i8", "u8", True, True, False),
    (2, 40, 4099, 70, "i8", "i8", "i8", True, True, True),
    (1, 33, 48, 300, "u8", "u8", "i8", True, True, False),
]


@pytest.mark.parametrize("N,C,HW,M,xt,wt,yt,pc,bias,wzp", SWEEP)
def test_sweep(gpu, N, C, HW, M, xt, wt, yt, pc, bias, wzp):
    log(f"qconv1x1 N{N} C{C} HW{HW} M{M} x:{xt} w:{wt} y:{yt} per_channel:{pc} bias:{bias} w_zp:{wzp}")
    case = W.qconv_random(N, C, HW, M, seed=N + 3 * C + 7 * HW + 11 * M, x_type=xt, w_type=wt,
                          y_type=yt, per_channel=pc, bias=bias, w_zp=wzp)
    got = run_qconv(gpu, case)
    want = oracle_qconv(case)
    assert np.array_equal(got, want), f"{np.sum(got != want)} codes differ"


def test_zero_size_is_a_no_op(gpu):
    import torch

    log("qconv1x1 empty")
    y = torch.full((0, 4, 16), 7, dtype=torch.uint8, device="cuda")
    gpu.qlinear_conv1x1(None, gpu.DQ_U8, None, None, None, gpu.DQ_I8, None, None, None, None,
                        gpu.DQ_U8, None, y, N=0, C_=8, HW=16, M=4, w_len=1)


def test_full_size_8x256x56x56(gpu):
    """The full 1x1 QLinearConv workload: every output code of all eight
    images bit-exact against the oracle, on two calls in a row."""
    log("qconv1x1 full [8,256,56,56] -> 256 channels")
    c = W.qconv1x1()
    case = dict(x=c["x"], x_type="u8", x_scale=c["x_scale"], x_zp=np.array([c["x_zp"]], np.uint8),
                w=c["w"], w_type="i8", w_scale=c["w_scale"], w_zp=None, bias=c["bias"],
                y_scale=c["y_scale"], y_zp=np.array([c["y_zp"]], np.uint8), y_type="u8")
    want = oracle_qconv(case)
    for call in range(2):
        got = run_qconv(gpu, case)
        for n in range(got.shape[0]):
            assert np.array_equal(got[n], want[n]), f"call {call} image {n}: {np.sum(got[n] != want[n])} codes differ"


def _random_conv_cases(seed, n):
    """Seeded random 1x1 QLinearConv cases: batch 1-2, channels 1-600 in and
    out (both sides of the persistent kernel's 256 limit), pixels 1-1200
    (ragged against the 32-pixel items), every 8-bit type of x, w and y,
    per-tensor or per-channel w scales, bias and w zero points on or off."""
    r = np.random.default_rng(seed)
    t8 = lambda: ["u8", "i8"][int(r.integers(2))]
    return [dict(N=int(r.integers(1, 3)), C=int(r.integers(1, 600)), HW=int(r.integers(1, 1200)),
                 M=int(r.integers(1, 600)), xt=t8(), wt=t8(), yt=t8(), pc=bool(r.integers(2)),
                 bias=bool(r.integers(2)), wzp=bool(r.integers(2)), seed=int(r.integers(1 << 30)))
            for _ in range(n)]


@pytest.mark.parametrize("p", _random_conv_cases(2029, 20),
                         ids=lambda p: f"N{p['N']}C{p['C']}HW{p['HW']}M{p['M']}")
def test_random_shapes(gpu, p):
    """Every output code bit-exact against the oracle on seeded random cases."""
    log(f"qconv1x1 random {p}")
    case = W.qconv_random(p["N"], p["C"], p["HW"], p["M"], seed=p["seed"], x_type=p["xt"], w_type=p["wt"],
                          y_type=p["yt"], per_channel=p["pc"], bias=p["bias"], w_zp=p["wzp"])
    got = run_qconv(gpu, case)
    want = oracle_qconv(case)
    assert np.array_equal(got, want), f"{np.sum(got != want)} codes differ"
