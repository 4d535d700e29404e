"""GPU parity of QuantizeLinear / DequantizeLinear against the CPU oracle:
bit-exact on every element (integer codes and single-rounding fp32)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_case import log

pytestmark = pytest.mark.gpu


def _run_q(dq, x, scale, zp, axis, y_type):
    import torch

    xd = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    sd = torch.from_numpy(np.atleast_1d(scale).astype(np.float32)).cuda()
    zd = None if zp is None else torch.from_numpy(np.atleast_1d(zp)).cuda()
    y = torch.empty(x.shape, dtype=torch.int8 if y_type == "i8" else torch.uint8, device="cuda")
    dq.qlinear_quantize(xd, sd, zd, dq.DQ_I8 if y_type == "i8" else dq.DQ_U8, y,
                        axis=dq.DQ_PER_TENSOR if axis is None else axis)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _run_dq(dq, q, scale, zp, axis):
    import torch

    qd = torch.from_numpy(np.ascontiguousarray(q)).cuda()
    sd = torch.from_numpy(np.atleast_1d(scale).astype(np.float32)).cuda()
    zd = None if zp is None else torch.from_numpy(np.atleast_1d(zp)).cuda()
    y = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dq.qlinear_dequantize(qd, dq.DQ_U8 if q.dtype == np.uint8 else dq.DQ_I8, sd, zd, y,
                          axis=dq.DQ_PER_TENSOR if axis is None else axis)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _check_both(dq, x, scale, zp, axis, y_type):
    ax = None if axis is None else axis
    want = oracle.quantize_linear(x, scale, zp, axis=ax, y_type=y_type)
    got = _run_q(dq, x, scale, zp, axis, y_type)
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"
    back_want = oracle.dequantize_linear(want, scale, zp, axis=ax)
    back = _run_dq(dq, want, scale, zp, axis)
    assert np.array_equal(back.view(np.uint32), back_want.view(np.uint32))


@pytest.mark.parametrize("shape,axis", [
    ((2, 16, 9, 11), 1),     # inner 99: channel per element
    ((4, 32, 8, 8), 1),      # inner 64: channel per 16-vector
    ((5, 48, 4, 4), 1),      # inner 16: a new channel every 16 elements
    ((7, 3, 32), 1),         # inner 32
    ((3, 5, 7), 0),          # leading axis
    ((3, 5, 7), 2),          # last axis, inner 1
    ((3, 5, 7), -2),         # negative axis
    ((1000003,), None),      # per tensor, ragged tail
    ((17,), 0),              # tiny, per element scales
])
@pytest.mark.parametrize("y_type", ["i8", "u8"])
def test_qdq_parity_small(gpu, shape, axis, y_type):
    log(f"qdq small shape={shape} axis={axis} {y_type}")
    ax = 0 if axis is None else axis
    case = W.qdq_per_axis(seed=7, shape=shape, axis=ax % len(shape), plant_every=13)
    x = case["x"]
    C = shape[ax]
    if axis is None:
        scale, zp = np.float32([0.02]), np.array([3 if y_type == "u8" else -3])
    else:
        scale = case["scale"]
        zp = case["zp"]
    if y_type == "u8":
        zp = (np.asarray(zp).astype(np.int32) + 120).astype(np.uint8)
    else:
        zp = np.asarray(zp).astype(np.int8)
    _check_both(gpu, x, scale, zp, axis, y_type)


def test_qdq_zero_point_absent_means_zero(gpu):
    log("qdq zp NULL")
    x = W.qdq_per_axis(seed=8, shape=(2, 4, 33), axis=1, plant_every=5)["x"]
    s = np.float32([0.01, 0.02, 0.03, 0.04])
    got = _run_q(gpu, x, s, None, 1, "i8")
    assert np.array_equal(got, oracle.quantize_linear(x, s, np.zeros(4, np.int8), axis=1))


def test_qdq_unaligned_views_take_the_scalar_path(gpu):
    import torch

    log("qdq unaligned")
    x = W.qdq_per_axis(seed=9, shape=(3, 7, 41), axis=1, plant_every=7)["x"]
    scale = np.linspace(0.01, 0.05, 7).astype(np.float32)
    zp = np.arange(-3, 4).astype(np.int8)
    flat = torch.from_numpy(np.concatenate([[0.0], x.reshape(-1)]).astype(np.float32)).cuda()
    xv = flat[1:]  # 4-byte aligned, not 16-byte aligned
    y = torch.empty(x.size + 1, dtype=torch.int8, device="cuda")[1:]
    gpu.qlinear_quantize(xv, torch.from_numpy(scale).cuda(), torch.from_numpy(zp).cuda(),
                         gpu.DQ_I8, y, axis=1, shape=x.shape)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().reshape(x.shape),
                          oracle.quantize_linear(x, scale, zp, axis=1))


def test_qdq_empty_tensor_is_a_no_op(gpu):
    import torch

    x = torch.empty((4, 0, 3), dtype=torch.float32, device="cuda")
    y = torch.empty((4, 0, 3), dtype=torch.int8, device="cuda")
    s = torch.ones(1, device="cuda")
    gpu.qlinear_quantize(x, s, None, gpu.DQ_I8, y)
    torch.cuda.synchronize()


def test_qdq_full_size_per_axis(gpu):
    """The per-channel workload at its full size, [64,256,56,56] NCHW, axis 1,
    int8 output with ties and saturation planted: every element compared."""
    log("qdq full [64,256,56,56]")
    case = W.qdq_per_axis(seed=1)
    assert case["n_ties"] > 1000
    _check_both(gpu, case["x"], case["scale"], case["zp"], 1, "i8")


# ------------------------------------------------------------- fp16 tensors

def _f16_dev(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.float16)


@pytest.mark.parametrize("shape,axis", [
    ((4, 32, 8, 8), 1), ((2, 16, 9, 11), 1), ((3, 5, 7), 2), ((1000003,), None), ((17,), 0),
    ((64, 256, 28, 28), 1),
])
@pytest.mark.parametrize("y_type", ["i8", "u8"])
def test_quantize_f16_matches_oracle(gpu, shape, axis, y_type):
    import torch

    r = np.random.default_rng(len(shape) * 7 + (axis or 0))
    x = (r.standard_normal(shape) * 4).astype(np.float16)
    nch = 1 if axis is None else shape[axis]
    s = r.uniform(0.005, 0.05, nch).astype(np.float16)
    lo, hi = (0, 256) if y_type == "u8" else (-10, 10)
    z = r.integers(lo, hi, nch)
    # planted exact ties: x = (k + 1/2) * s for a few elements of channel 0
    xf = x.reshape(-1)
    xf[:8] = ((np.arange(8) - 4 + 0.5) * s[0].astype(np.float32)).astype(np.float16)
    want = oracle.quantize_linear_f16(x.view(np.uint16), s.view(np.uint16), z, axis=axis,
                                      y_type=y_type)
    zd = torch.from_numpy(z.astype(np.uint8 if y_type == "u8" else np.int8)).cuda()
    y = torch.empty(shape, dtype=torch.uint8 if y_type == "u8" else torch.int8, device="cuda")
    gpu.qlinear_quantize_f16(_f16_dev(x.view(np.uint16)), _f16_dev(s.view(np.uint16)), zd,
                             gpu.DQ_U8 if y_type == "u8" else gpu.DQ_I8, y,
                             axis=gpu.DQ_PER_TENSOR if axis is None else axis)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"


@pytest.mark.parametrize("shape,axis", [((4, 32, 8, 8), 1), ((3, 5, 7), 2), ((1000003,), None),
                                        ((64, 256, 28, 28), 1)])
@pytest.mark.parametrize("y_type", ["f16", "f32"])
def test_dequantize_f16_matches_oracle(gpu, shape, axis, y_type):
    import torch

    r = np.random.default_rng(len(shape) + 3)
    q = r.integers(0, 256, shape).astype(np.uint8)
    nch = 1 if axis is None else shape[axis]
    s = r.uniform(1e-4, 2.0, nch).astype(np.float16)
    s[0] = np.float16(6e-8)          # a subnormal fp16 scale
    z = r.integers(0, 256, nch)
    want = oracle.dequantize_linear_f16(q, s.view(np.uint16), z, axis=axis, y_type=y_type)
    y = torch.empty(shape, dtype=torch.float16 if y_type == "f16" else torch.float32, device="cuda")
    gpu.qlinear_dequantize_f16(torch.from_numpy(q).cuda(), gpu.DQ_U8, _f16_dev(s.view(np.uint16)),
                               torch.from_numpy(z.astype(np.uint8)).cuda(),
                               gpu.DQ_F16 if y_type == "f16" else gpu.DQ_F32, y,
                               axis=gpu.DQ_PER_TENSOR if axis is None else axis)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    if y_type == "f16":
        assert np.array_equal(got.view(np.uint16), want)
    else:
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def _random_qdq_cases(seed, n):
    """Seeded random tensors of 1 to 5 dimensions (up to ~2 M elements, sizes
    ragged against the kernels' 16-element vectors and 4096-element blocks),
    an axis drawn over every position, negative ones included, or per tensor,
    int8 or uint8 codes, with or without a zero point."""
    r = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        nd = int(r.integers(1, 6))
        while True:
            shape = tuple(int(v) for v in r.integers(1, 90, nd))
            if np.prod(shape) <= 2_000_000:
                break
        axis = None if r.integers(4) == 0 else int(r.integers(-nd, nd))
        cases.append(dict(shape=shape, axis=axis, y_type=["i8", "u8"][int(r.integers(2))],
                          has_zp=bool(r.integers(4)), seed=int(r.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("p", _random_qdq_cases(2028, 24), ids=lambda p: f"{p['shape']}-{p['axis']}")
def test_qdq_random_shapes(gpu, p):
    """Every code and every dequantized value bit-exact against the oracle, on
    seeded random shapes and axes, with planted ties and saturating values."""
    shape, axis, y_type = p["shape"], p["axis"], p["y_type"]
    log(f"qdq random shape={shape} axis={axis} {y_type} zp={p['has_zp']} seed={p['seed']}")
    ax = 0 if axis is None else axis % len(shape)
    case = W.qdq_per_axis(seed=p["seed"], shape=shape, axis=ax, plant_every=29)
    if axis is None:
        scale, zp = np.float32([0.03]), np.array([5 if y_type == "u8" else -5])
    else:
        scale, zp = case["scale"], case["zp"]
    if y_type == "u8":
        zp = (np.asarray(zp).astype(np.int32) + 120).astype(np.uint8)
    else:
        zp = np.asarray(zp).astype(np.int8)
    _check_both(gpu, case["x"], scale, zp if p["has_zp"] else None, axis, y_type)
