"""Seeded synthetic inputs for the dynamic quantized inner product and for
QuantizeLinear / DequantizeLinear.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no scales, no rounding to integer codes, no sums), so the
CPU oracle and the HIP library can both be fed from it without sharing any
computation. Every generator is a numpy PCG64 stream with a fixed seed.

The shapes and value distributions follow the workloads that the method's
pages describe in words (no public dataset or benchmark suite is involved):

* ``dqip_small``   -- inner product M=64, N=64, K=128, fp32 A and constant fp32 B.
* ``dqip_ramp``    -- the 4x8x16 ramp of the usage example in the
  "SynetDynamicQuantizedInnerProduct16b" class reference (Detailed
  Description): A[i] = i*0.01f, B[i] = i*0.02f, bias 0.1f, avoidOverflow on.
* ``qdq_per_axis`` -- QuantizeLinear input [64,256,56,56] NCHW, per-channel
  (axis 1) scales and int8 zero points, with planted half-way ties and
  far-out-of-range values.
* ``dqip_large``   -- 4096^3, bf16 A with 1% outliers, constant int8 B.
* ``dqip_lstm``    -- the input and the recurrent gate projections of a
  quantized LSTM (hidden 512, input 512, seq 128 x batch 32).
* ``dqip_dynamic_b`` -- 8192^2 fp32 A and fp32 B quantized on every call,
  avoidOverflow on.
* ``qconv1x1``     -- a 1x1 QLinearConv over uint8 x [8,256,56,56].
* ``qgemm_case``   -- the quantized matrix products of the ORT schemas
  (MatMulIntegerToFloat, DynamicQuantizeMatMul, QGemm) at M=N=K=4096 by
  default: uint8 A with a zero point (or fp32 A ~N(0,1) with 1% x20
  outliers), int8 B with per-column scales and small per-column zero
  points, bias / int32 C per column, uint8 output for QGemm.
* ``elementwise_case`` -- the element-wise quantized operators of the ORT
  schemas at the sizes the benchmark times: uniform 8-bit codes, per-tensor
  scales and zero points (QLinearAdd / Mul and MulInteger over [8192, 8192]
  or [4096, 8192], optionally against a broadcast row vector; LeakyRelu /
  Sigmoid over 64 Mi codes; ReduceSumInteger / QLinearReduceMean over
  [16384, 4096] rows, [4096, 16384] columns and NCHW / NHWC global pooling
  of [64, 2048, 7, 7]; QLinearConcat of two [32, 256, 56, 56] maps).
* ``qconv_layer_case`` -- general QLinearConv layers of a ResNet-style
  network at a batch of 8 (3x3 at 56x56 with 64 and 256 channels, 3x3 at
  14x14 with 256, the 7x7 / 2 stem over 224x224, a depthwise 3x3): uniform
  uint8 x, int8 w ~U{-127..127} with per-channel scales ~U(0.0005, 0.002),
  int32 bias ~U{-5000..5000}.
"""
from __future__ import annotations

import numpy as np

F32_MAX = np.float32(np.finfo(np.float32).max)

# dtype tags shared by both sides' Python wrappers (plain names, no arithmetic)
F32, BF16, I8, U8 = "f32", "bf16", "i8", "u8"
IDENTITY, RELU, LEAKY_RELU = "identity", "relu", "leaky_relu"


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (torch's round-to-nearest-even conversion)
    and return the raw 16-bit patterns as uint16."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact: the bits become the high half)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def _case(M, N, K, A, B, *, typeA, typeB, typeC, constB, bias, act,
          avoid, scaleB=None, alpha=0.01, name=""):
    return dict(name=name, M=M, N=N, K=K, A=A, B=B, typeA=typeA, typeB=typeB,
                typeC=typeC, constB=constB, bias=bias, act=act, alpha=alpha,
                avoid=avoid, scaleB=scaleB)


# ----------------------------------------------------------------------------
# dynamic quantized inner product cases
# ----------------------------------------------------------------------------

def dqip_small(seed: int = 0):
    """M=64, N=64, K=128: A ~U(-1,1), constant fp32 B ~N(0,0.05) quantized per
    column to [-127,127], bias ~U(-0.1,0.1), identity, fp32 out."""
    r = rng(seed)
    M, N, K = 64, 64, 128
    A = r.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    B = r.normal(0.0, 0.05, (K, N)).astype(np.float32)
    bias = r.uniform(-0.1, 0.1, N).astype(np.float32)
    return _case(M, N, K, A, B, typeA=F32, typeB=F32, typeC=F32, constB=True,
                 bias=bias, act=IDENTITY, avoid=False, name="dqip 64x64x128 f32")


def dqip_ramp():
    """The usage example's 4x8x16 ramp (no randomness)."""
    M, N, K = 4, 8, 16
    A = (np.arange(M * K, dtype=np.float32) * np.float32(0.01)).reshape(M, K)
    B = (np.arange(K * N, dtype=np.float32) * np.float32(0.02)).reshape(K, N)
    bias = np.full(N, 0.1, dtype=np.float32)
    return _case(M, N, K, A, B, typeA=F32, typeB=F32, typeC=F32, constB=True,
                 bias=bias, act=IDENTITY, avoid=True, name="ramp 4x8x16")


def dqip_random(M, N, K, *, seed, typeA=F32, typeB=F32, typeC=F32, constB=True,
                bias=True, act=IDENTITY, avoid=False, alpha=0.01,
                a_dist="normal", b_std=0.05, outliers=0.0, zero_rows=(),
                zero_cols=()):
    """A general random case for parity sweeps over odd shapes.

    typeB=I8 draws B ~U{-127..127} with scaleB ~U(0.001,0.01); otherwise B is
    fp32 ~N(0,b_std) (stored as bf16 bits for typeB=BF16). ``zero_rows`` /
    ``zero_cols`` plant all-zero rows of A / columns of B."""
    r = rng(seed)
    if a_dist == "uniform":
        A = r.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    else:
        A = r.normal(0.0, 1.0, (M, K)).astype(np.float32)
    if outliers:
        mask = r.random((M, K)) < outliers
        A = np.where(mask, A * np.float32(20.0), A).astype(np.float32)
    for i in zero_rows:
        A[i, :] = 0.0
    scaleB = None
    if typeB == I8:
        B = r.integers(-127, 128, (K, N), dtype=np.int64).astype(np.int8)
        scaleB = r.uniform(0.001, 0.01, N).astype(np.float32)
        for j in zero_cols:
            B[:, j] = 0
    else:
        B = r.normal(0.0, b_std, (K, N)).astype(np.float32)
        for j in zero_cols:
            B[:, j] = 0.0
    biasv = r.uniform(-0.1, 0.1, N).astype(np.float32) if bias else None
    if typeA == BF16:
        A = to_bf16_bits(A)
    if typeB == BF16:
        B = to_bf16_bits(B)
    return _case(M, N, K, A, B, typeA=typeA, typeB=typeB, typeC=typeC,
                 constB=constB, bias=biasv, act=act, avoid=avoid,
                 scaleB=scaleB, alpha=alpha, name=f"dqip {M}x{N}x{K} seed{seed}")


def dqip_large(seed: int = 2, M: int = 4096, N: int = 4096, K: int = 4096):
    """4096^3: A bf16 from N(0,1) with a Bernoulli(0.01) mask of x20 outliers,
    constant pre-quantized int8 B ~U{-127..127}, scaleB ~U(0.001,0.01),
    bias ~U(-1,1), ReLU, bf16 out."""
    r = rng(seed)
    A = r.standard_normal((M, K), dtype=np.float32)
    mask = r.random((M, K), dtype=np.float32) < np.float32(0.01)
    A[mask] *= np.float32(20.0)
    B = r.integers(-127, 128, (K, N), dtype=np.int8)
    scaleB = r.uniform(0.001, 0.01, N).astype(np.float32)
    bias = r.uniform(-1.0, 1.0, N).astype(np.float32)
    return _case(M, N, K, to_bf16_bits(A), B, typeA=BF16, typeB=I8, typeC=BF16,
                 constB=True, bias=bias, act=RELU, avoid=False, scaleB=scaleB,
                 name=f"dqip {M}x{N}x{K} bf16 A, const int8 B, relu, bf16 out")


def dqip_lstm(seed: int = 3, recurrent: bool = False):
    """Quantized LSTM gate projections, hidden 512, input 512, 4*hidden = 2048
    gate columns. Input GEMM: M = seq 128 x batch 32 = 4096, K = 512.
    Recurrent step: M = batch 32, K = hidden 512. Per-channel int8 weights
    ~U{-127..127}, scales ~U(0.001,0.01), bias ~U(-0.1,0.1), A ~U(-1,1),
    identity, fp32 out."""
    r = rng(seed + (100 if recurrent else 0))
    M = 32 if recurrent else 4096
    K, N = 512, 2048
    A = r.uniform(-1.0, 1.0, (M, K)).astype(np.float32)
    W = r.integers(-127, 128, (K, N), dtype=np.int8)
    scale = r.uniform(0.001, 0.01, N).astype(np.float32)
    bias = r.uniform(-0.1, 0.1, N).astype(np.float32)
    kind = "recurrent" if recurrent else "input"
    return _case(M, N, K, A, W, typeA=F32, typeB=I8, typeC=F32, constB=True,
                 bias=bias, act=IDENTITY, avoid=False, scaleB=scale,
                 name=f"lstm {kind} gates {M}x{N}x{K}")


def dqip_dynamic_b(seed: int = 4, M: int = 8192, N: int = 8192, K: int = 8192):
    """Non-constant B: A fp32 ~N(0,1), B fp32 ~N(0,0.02) quantized per column
    on every call with avoidOverflow, no bias, identity, fp32 out."""
    r = rng(seed)
    A = r.standard_normal((M, K), dtype=np.float32)
    B = (r.standard_normal((K, N), dtype=np.float32) * np.float32(0.02))
    return _case(M, N, K, A, B, typeA=F32, typeB=F32, typeC=F32, constB=False,
                 bias=None, act=IDENTITY, avoid=True,
                 name=f"dqip {M}x{N}x{K} dynamic fp32 B, avoidOverflow")


# ----------------------------------------------------------------------------
# QuantizeLinear / DequantizeLinear
# ----------------------------------------------------------------------------

def qdq_per_axis(seed: int = 1, shape=(64, 256, 56, 56), axis: int = 1,
                 plant_every: int = 4096):
    """x ~N(0,1) NCHW, per-channel y_scale ~U(0.005,0.05) and int8 zero points
    ~U{-10..10}. At 1 in ``plant_every`` seeded positions x is set to a value
    whose quotient x/scale is exactly k+1/2 (k ~U{-140..140}); at another 1 in
    ``plant_every`` positions x is one of +-{1e3, 1e6, FLT_MAX}."""
    r = rng(seed)
    shape = tuple(int(s) for s in shape)
    C = shape[axis]
    x = r.standard_normal(shape, dtype=np.float32)
    scale = r.uniform(0.005, 0.05, C).astype(np.float32)
    zp = r.integers(-10, 11, C).astype(np.int8)
    inner = int(np.prod(shape[axis + 1:], dtype=np.int64))
    flat = x.reshape(-1)
    n = flat.size
    n_plant = max(1, n // plant_every)
    # half-way ties: x = fl32((k + 1/2) * s), kept only where fl32(x / s) is
    # exactly k + 1/2 (the check is IEEE fp32 division, done by numpy)
    pos = r.choice(n, size=n_plant, replace=False)
    ch = (pos // inner) % C
    k = r.integers(-140, 141, n_plant).astype(np.float32)
    half = k + np.float32(0.5)
    cand = (half * scale[ch]).astype(np.float32)
    exact = (cand / scale[ch]).astype(np.float32) == half
    flat[pos[exact]] = cand[exact]
    # far out of range
    pos2 = r.choice(n, size=n_plant, replace=False)
    mags = np.array([1e3, 1e6, F32_MAX], dtype=np.float32)
    vals = mags[r.integers(0, 3, n_plant)] * np.where(
        r.random(n_plant) < 0.5, np.float32(-1.0), np.float32(1.0))
    flat[pos2] = vals.astype(np.float32)
    return dict(x=x, axis=axis, scale=scale, zp=zp, n_ties=int(exact.sum()),
                name=f"qdq {list(shape)} axis {axis}")


# ----------------------------------------------------------------------------
# 1x1 QLinearConv
# ----------------------------------------------------------------------------

def qconv1x1(seed: int = 4, batch: int = 8, C: int = 256, M: int = 256,
             H: int = 56, W: int = 56):
    """uint8 x ~U{0..255} with x_zp 128 and x_scale 0.01; int8 w [M,C]
    ~U{-127..127}, w_zp 0, per-output-channel w_scale ~U(0.0005,0.002);
    int32 bias ~U{-10000..10000}; y_scale 0.02, y_zp 128, uint8 y."""
    r = rng(seed + 1000)
    x = r.integers(0, 256, (batch, C, H, W), dtype=np.int64).astype(np.uint8)
    w = r.integers(-127, 128, (M, C), dtype=np.int64).astype(np.int8)
    w_scale = r.uniform(0.0005, 0.002, M).astype(np.float32)
    bias = r.integers(-10000, 10001, M, dtype=np.int64).astype(np.int32)
    return dict(x=x, x_scale=np.float32(0.01), x_zp=128, w=w, w_scale=w_scale,
                bias=bias, y_scale=np.float32(0.02), y_zp=128,
                name=f"qlinearconv 1x1 x[{batch},{C},{H},{W}] -> {M} ch")


def qconv_random(N: int, C: int, HW: int, M: int, *, seed: int, x_type: str = "u8",
                 w_type: str = "i8", y_type: str = "u8", per_channel: bool = True,
                 bias: bool = True, w_zp: bool = False):
    """A random 1x1 QLinearConv case: x [N,C,HW] and w [M,C] uniform over
    their 8-bit ranges, zero points uniform over the type's range (w's only
    when w_zp, else absent = 0), x_scale 0.01, w_scale ~U(0.0005,0.002),
    int32 bias ~U{-20000..20000}. y_scale is set from C so that the outputs
    spread over the 8-bit range and both saturation ends occur."""
    r = rng(seed + 2000)

    def codes(t, shape):
        lo, hi = (0, 256) if t == "u8" else (-128, 128)
        return r.integers(lo, hi, shape, dtype=np.int64).astype(np.uint8 if t == "u8" else np.int8)

    x = codes(x_type, (N, C, HW))
    w = codes(w_type, (M, C))
    wl = M if per_channel else 1
    wz = codes(w_type, (wl,)) if w_zp else None
    x_zp = codes(x_type, (1,))
    y_zp = codes(y_type, (1,))
    w_scale = r.uniform(0.0005, 0.002, wl).astype(np.float32)
    b = r.integers(-20000, 20001, M, dtype=np.int64).astype(np.int32) if bias else None
    # a w zero point away from w's centre adds a coherent term of size ~C
    spread = 20.0 if (w_zp or w_type == "u8") else 1.0
    y_scale = np.float32(spread * 0.01 * 0.00125 * 128.0 * 74.0 * np.sqrt(C) / 100.0)
    return dict(x=x, x_type=x_type, x_scale=np.float32(0.01), x_zp=x_zp, w=w, w_type=w_type,
                w_scale=w_scale, w_zp=wz, bias=b, y_scale=y_scale, y_zp=y_zp, y_type=y_type,
                name=f"qconv1x1 N{N} C{C} HW{HW} M{M} x:{x_type} w:{w_type} y:{y_type}")


def qgemm_case(kind: str, seed: int = 5, M: int = 4096, N: int = 4096, K: int = 4096):
    """kind: "mitf" (MatMulIntegerToFloat: uint8 A ~U{0..255}, a_zp 128,
    a_scale 0.02; fp32 Y with bias), "dqmm" (DynamicQuantizeMatMul: fp32 A
    ~N(0,1) with a Bernoulli(0.01) mask of x20 outliers; bias) or "qgemm"
    (QGemm: uint8 A as for mitf, int32 C per column ~U{-20000..20000},
    alpha 1, uint8 Y with y_scale 0.05, y_zp 128). B is int8 ~U{-127..127}
    [K,N] with per-column scales ~U(0.0005, 0.002) and zero points
    ~U{-8..8}; bias ~U(-1, 1)."""
    r = rng(seed)
    case = dict(kind=kind, M=M, N=N, K=K, name=f"{kind} {M}x{N}x{K}")
    if kind == "dqmm":
        A = r.normal(0.0, 1.0, (M, K)).astype(np.float32)
        mask = r.random((M, K)) < 0.01
        case["A"] = np.where(mask, A * np.float32(20.0), A).astype(np.float32)
    else:
        case["A"] = r.integers(0, 256, (M, K), dtype=np.int64).astype(np.uint8)
        case["a_scale"], case["a_zp"] = np.float32(0.02), 128
    case["B"] = r.integers(-127, 128, (K, N), dtype=np.int64).astype(np.int8)
    case["b_scale"] = r.uniform(0.0005, 0.002, N).astype(np.float32)
    case["b_zp"] = r.integers(-8, 9, N).astype(np.int32)
    if kind == "qgemm":
        case["C"] = r.integers(-20000, 20001, N).astype(np.int32)
        case["y_scale"], case["y_zp"] = np.float32(0.05), 128
    else:
        case["bias"] = r.uniform(-1.0, 1.0, N).astype(np.float32)
    return case


def _codes(r, shape, t):
    """Uniform 8-bit codes: raw random bytes viewed as uint8 or int8."""
    n = int(np.prod(shape, dtype=np.int64))
    w = r.integers(0, np.iinfo(np.uint64).max, (n + 7) // 8, dtype=np.uint64, endpoint=True)
    b = w.view(np.uint8)[:n].reshape(shape)
    return b if t == "u8" else b.view(np.int8)


# shapes and per-tensor parameters of the element-wise workloads:
# kind -> (input shapes, type, extra)
ELEMENTWISE = {
    "add": ([(8192, 8192), (8192, 8192)], "u8", {}),
    "add_rowvec": ([(8192, 8192), (8192,)], "u8", {}),
    "mul": ([(8192, 8192), (8192, 8192)], "u8", {}),
    "mul_integer": ([(4096, 8192), (4096, 8192)], "u8", {}),
    "sigmoid": ([(64 << 20,)], "u8", {}),
    "leaky_relu": ([(64 << 20,)], "u8", {"alpha": 0.1}),
    "sum_rows": ([(16384, 4096)], "u8", {"axes": [1]}),
    "sum_cols": ([(4096, 16384)], "u8", {"axes": [0]}),
    "mean_rows": ([(16384, 4096)], "u8", {"axes": [1]}),
    "mean_pool_nchw": ([(64, 2048, 7, 7)], "u8", {"axes": [2, 3]}),
    "mean_pool_nhwc": ([(64, 49, 2048)], "u8", {"axes": [1]}),
    "concat": ([(32, 256, 56, 56), (32, 256, 56, 56)], "u8", {"axis": 1}),
}


def elementwise_case(kind: str, seed: int = 6):
    """Inputs of one element-wise workload: uniform codes of the listed
    shapes and per-tensor scales / zero points (one per input plus the
    output's), all fixed by the seed."""
    shapes, t, extra = ELEMENTWISE[kind]
    r = rng(seed)
    xs = [_codes(r, s, t) for s in shapes]
    scales = [np.float32(v) for v in r.uniform(0.005, 0.05, len(shapes) + 1)]
    lo, hi = (0, 256) if t == "u8" else (-128, 128)
    zps = [int(v) for v in r.integers(lo, hi, len(shapes) + 1)]
    if kind == "mul":
        scales[-1] = np.float32(r.uniform(0.5, 4.0))
    if kind == "sigmoid":
        scales[-1], zps[-1] = np.float32(1.0 / 256), lo
    return dict(name=kind, xs=xs, type=t, scales=scales, zps=zps, **extra)


# name -> (N, C, H, W, M, k, stride, pad, group)
QCONV_LAYERS = {
    "resnet_3x3_64_56": (8, 64, 56, 56, 64, 3, 1, 1, 1),
    "resnet_3x3_256_56": (8, 256, 56, 56, 256, 3, 1, 1, 1),
    "resnet_3x3_256_14": (8, 256, 14, 14, 256, 3, 1, 1, 1),
    "resnet_stem_7x7_s2": (8, 3, 224, 224, 64, 7, 2, 3, 1),
    "depthwise_3x3_256_56": (8, 256, 56, 56, 256, 3, 1, 1, 256),
}


def qconv_layer_case(name: str, seed: int = 7):
    """Inputs of one QLinearConv layer of QCONV_LAYERS (x [N,C,H,W] uint8,
    w [M, C/group, k, k] int8, per-channel scales, bias)."""
    N, C, H, W, M, k, st, pad, grp = QCONV_LAYERS[name]
    r = rng(seed)
    x = _codes(r, (N, C, H, W), "u8")
    w = r.integers(-127, 128, (M, C // grp, k, k)).astype(np.int8)
    return dict(name=name, x=x, w=w, w_scale=r.uniform(0.0005, 0.002, M).astype(np.float32),
                bias=r.integers(-5000, 5000, M).astype(np.int32), x_scale=np.float32(0.02),
                y_scale=np.float32(0.1))


def lstm_case(seq: int = 128, batch: int = 32, input_size: int = 512, hidden: int = 512, *,
              seed: int = 8, direction: str = "forward", w_type: str = "i8", r_type: str = "i8",
              per_channel: bool = True, zero_points: bool = False, bias: bool = True,
              peepholes: bool = False, initial: bool = True, lens=None):
    """A DynamicQuantizeLSTM case (the gate-projection shapes above for the
    defaults): X ~U(-1,1) [seq, batch, input]; W [dirs, input, 4h] and R
    [dirs, h, 4h] uniform 8-bit codes (int8 in [-127, 127], uint8 in
    [0, 255]) with scales ~U(0.5, 1.5) / (127 sqrt(K)) per column (or one
    per direction), so gate inputs are O(1); zero points 0 (int8) / 128
    (uint8) unless zero_points draws them per column from +-8 around that;
    B ~U(-0.5, 0.5) [dirs, 8h]; P ~U(-0.5, 0.5) [dirs, 3h]; initial_h /
    initial_c ~U(-1, 1); lens: None, or the int32 sequence_lens."""
    dirs = 2 if direction == "bidirectional" else 1
    r = rng(seed)
    g = 4 * hidden

    def weights(rows, t):
        if t == "u8":
            w = r.integers(0, 256, (dirs, rows, g)).astype(np.uint8)
            base, dt = 128, np.uint8
        else:
            w = r.integers(-127, 128, (dirs, rows, g)).astype(np.int8)
            base, dt = 0, np.int8
        n = (dirs, g) if per_channel else (dirs,)
        sc = (r.uniform(0.5, 1.5, n) / (127.0 * np.sqrt(rows))).astype(np.float32)
        zp = (base + r.integers(-8, 9, n) if zero_points else np.full(n, base)).astype(dt)
        return w, sc, zp

    W, ws, wz = weights(input_size, w_type)
    R, rs, rz = weights(hidden, r_type)
    return dict(
        X=r.uniform(-1, 1, (seq, batch, input_size)).astype(np.float32), W=W, W_scale=ws,
        W_zp=wz, R=R, R_scale=rs, R_zp=rz, hidden=hidden, direction=direction,
        B=r.uniform(-0.5, 0.5, (dirs, 8 * hidden)).astype(np.float32) if bias else None,
        P=r.uniform(-0.5, 0.5, (dirs, 3 * hidden)).astype(np.float32) if peepholes else None,
        initial_h=r.uniform(-1, 1, (dirs, batch, hidden)).astype(np.float32) if initial else None,
        initial_c=r.uniform(-1, 1, (dirs, batch, hidden)).astype(np.float32) if initial else None,
        sequence_lens=None if lens is None else np.asarray(lens, np.int32))
