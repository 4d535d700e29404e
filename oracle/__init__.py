"""Python wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It never imports the
HIP library package and the HIP library never imports it.

Every function takes and returns numpy arrays. Element types are named by
the tags of ``workloads`` ("f32", "bf16", "i8", "u8"); bf16 tensors travel
as uint16 bit patterns. The DynamicQuantizeLSTM reference (readings
R26-R28) is the module ``oracle.lstm``, written in numpy over this package's
DynamicQuantizeMatMul.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_TYPE = {"f32": 0, "bf16": 1, "i8": 2, "u8": 3}
_ACT = {"identity": 0, "relu": 1, "leaky_relu": 2}

_lib = None


def lib() -> C.CDLL:
    """Load oracle/liboracle.so, compiling it with gcc first if it is absent
    or older than oracle.c."""
    global _lib
    if _lib is None:
        # DQ_ORACLE_LIB: another build of oracle.c (the test suite's
        # sanitizer build); else the in-tree library, rebuilt when stale
        path = os.environ.get("DQ_ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = C.CDLL(path)
        vp, i64, i32, f32 = C.c_void_p, C.c_int64, C.c_int, C.c_float
        L.oracle_bf16_to_f32.argtypes = [C.c_uint16]
        L.oracle_bf16_to_f32.restype = C.c_float
        L.oracle_f32_to_bf16.argtypes = [C.c_float]
        L.oracle_f32_to_bf16.restype = C.c_uint16
        L.oracle_quantize_linear.argtypes = [vp, i32, vp, i32, vp, vp, i32, vp]
        L.oracle_dequantize_linear.argtypes = [vp, i32, i32, vp, i32, vp, vp, vp]
        L.oracle_quantize_rows.argtypes = [vp, i32, i64, i64, vp, i64, vp, vp, vp]
        L.oracle_quantize_cols.argtypes = [vp, i32, i64, i64, i32, vp, vp]
        L.oracle_colsum.argtypes = [vp, i64, i64, vp]
        L.oracle_int_gemm.argtypes = [vp, vp, vp, i64, i64, i64, vp]
        L.oracle_epilogue.argtypes = [vp, vp, vp, i32, vp, i32, f32, i64, i64, i32, vp]
        L.oracle_dqip_forward.argtypes = [vp, i32, vp, i32, vp, i64, i64, i64,
                                          vp, i64, i32, i32, vp, i32, f32, i32,
                                          vp, vp, vp, vp, vp, vp, vp]
        L.oracle_qlinear_conv.argtypes = [vp, i32, i64, i64, i64, i64, f32, i32,
                                          vp, i32, i64, i64, i64, vp, vp, i64, vp,
                                          f32, i32, i32, vp]
        L.oracle_quantize_tensor_u8.argtypes = [vp, i64, vp, vp, vp]
        L.oracle_qgemm.argtypes = [vp, i32, i32, i64, i64, f32, i32, vp, i32, i32, i64,
                                   vp, i64, vp, i64, vp, i64, i64, f32, vp, i32, f32, i32,
                                   vp, vp]
        L.oracle_f16_to_f32.argtypes = [C.c_uint16]
        L.oracle_f16_to_f32.restype = C.c_float
        L.oracle_f32_to_f16.argtypes = [C.c_float]
        L.oracle_f32_to_f16.restype = C.c_uint16
        L.oracle_f16_to_f32_array.argtypes = [vp, i64, vp]
        L.oracle_f32_to_f16_array.argtypes = [vp, i64, vp]
        L.oracle_qlinear_conv2d.argtypes = [vp, i32, i64, i64, i64, i64, f32, i32, vp, i32, i64,
                                             i64, i64, i64, i64, i64, i64, i64, i64, i64, i64,
                                             i64, vp, vp, i64, vp, f32, i32, i32, vp, vp]
        L.oracle_broadcast_shape.argtypes = [i32, vp, i32, vp, vp, vp]
        L.oracle_qlinear_binary.argtypes = [i32, i32, vp, i32, vp, f32, i32, vp, i32, vp,
                                            f32, i32, f32, i32, vp]
        L.oracle_qlinear_unary.argtypes = [i32, i32, vp, i64, f32, i32, f32, i32, f32, vp]
        L.oracle_reduce.argtypes = [i32, i32, vp, i32, vp, i32, f32, i32, f32, i32, vp]
        L.oracle_qlinear_concat.argtypes = [i32, i32, vp, vp, vp, vp, i64, i64, f32, i32, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with status {rc}")


def _np_type(tag):
    return {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "u8": np.uint8}[tag]


# ------------------------------------------------------------------ helpers

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    L = lib()
    b = _c(bits, np.uint16).reshape(-1)
    return np.array([L.oracle_bf16_to_f32(int(v)) for v in b], np.float32).reshape(np.shape(bits))


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    L = lib()
    a = _c(x, np.float32).reshape(-1)
    return np.array([L.oracle_f32_to_bf16(float(v)) for v in a], np.uint16).reshape(np.shape(x))


def _axis(ndim, axis):
    if axis is None:
        return -1
    if axis < -ndim or axis >= ndim:
        raise ValueError("axis out of range")
    return axis + ndim if axis < 0 else axis


def _params(scale, zp, n_expected):
    s = _c(np.atleast_1d(scale), np.float32)
    z = _c(np.atleast_1d(np.zeros_like(s, dtype=np.int32) if zp is None else zp), np.int32)
    if s.size != n_expected or z.size != n_expected:
        raise ValueError("scale / zero point length does not match the axis")
    return s, z


# ------------------------------------------------------- QuantizeLinear etc.

def quantize_linear(x, scale, zp, *, axis=None, y_type="i8"):
    """y = saturate(rne(x / scale) + zp); axis None = per tensor."""
    x = _c(x, np.float32)
    ax = _axis(x.ndim, axis)
    s, z = _params(scale, zp, 1 if ax < 0 else x.shape[ax])
    shape = np.array(x.shape if x.ndim else (1,), np.int64)
    y = np.empty(x.shape, _np_type(y_type))
    rc = lib().oracle_quantize_linear(_p(x), max(x.ndim, 1), _p(shape), ax, _p(s), _p(z),
                                      _TYPE[y_type], _p(y))
    _check(rc, "quantize_linear")
    return y


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """binary16 bit patterns (uint16) -> fp32, exactly (R24)."""
    b = _c(bits, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().oracle_f16_to_f32_array(_p(b), b.size, _p(out))
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """fp32 -> binary16 bit patterns, round to nearest even (R24)."""
    a = _c(x, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_f16_array(_p(a), a.size, _p(out))
    return out


def quantize_linear_f16(x_bits, scale_bits, zp, *, axis=None, y_type="i8"):
    """QuantizeLinear of an fp16 x with fp16 scales (bit patterns), R24."""
    return quantize_linear(f16_to_f32(x_bits), f16_to_f32(np.atleast_1d(scale_bits)), zp,
                           axis=axis, y_type=y_type)


def dequantize_linear_f16(x, scale_bits, zp, *, axis=None, y_type="f16"):
    """DequantizeLinear with fp16 scales: fp16 y (bit patterns) or fp32 y, R24."""
    y = dequantize_linear(x, f16_to_f32(np.atleast_1d(scale_bits)), zp, axis=axis)
    return f32_to_f16(y) if y_type == "f16" else y


def dequantize_linear(x, scale, zp, *, axis=None):
    """y = (x - zp) * scale; x int8 or uint8; axis None = per tensor."""
    x = np.ascontiguousarray(x)
    xt = "u8" if x.dtype == np.uint8 else "i8"
    ax = _axis(x.ndim, axis)
    s, z = _params(scale, zp, 1 if ax < 0 else x.shape[ax])
    shape = np.array(x.shape if x.ndim else (1,), np.int64)
    y = np.empty(x.shape, np.float32)
    rc = lib().oracle_dequantize_linear(_p(x), _TYPE[xt], max(x.ndim, 1), _p(shape), ax,
                                        _p(s), _p(z), _p(y))
    _check(rc, "dequantize_linear")
    return y


# ---------------------------------------- dynamic quantized inner product

def quantize_rows(A, typeA="f32", rows=None):
    """Per-row dynamic quantization of A [M,K] -> (uA, scaleA, zeroA)."""
    A = _c(A, _np_type(typeA))
    M, K = A.shape
    r = None if rows is None else _c(rows, np.int64)
    n = M if r is None else r.size
    uA = np.empty((n, K), np.uint8)
    sA = np.empty(n, np.float32)
    zA = np.empty(n, np.int32)
    _check(lib().oracle_quantize_rows(_p(A), _TYPE[typeA], M, K, _p(r), n, _p(uA),
                                      _p(sA), _p(zA)), "quantize_rows")
    return uA, sA, zA


def quantize_cols(B, typeB="f32", avoid=False):
    """Per-column dynamic quantization of B [K,N] -> (iB [K,N], scaleB [N])."""
    B = _c(B, _np_type(typeB))
    K, N = B.shape
    iB = np.empty((K, N), np.int8)
    sB = np.empty(N, np.float32)
    _check(lib().oracle_quantize_cols(_p(B), _TYPE[typeB], K, N, int(bool(avoid)), _p(iB),
                                      _p(sB)), "quantize_cols")
    return iB, sB


def colsum(iB):
    iB = _c(iB, np.int8)
    K, N = iB.shape
    out = np.empty(N, np.int32)
    _check(lib().oracle_colsum(_p(iB), K, N, _p(out)), "colsum")
    return out


def int_gemm(uA, zeroA, iB):
    uA = _c(uA, np.uint8)
    zA = _c(zeroA, np.int32)
    iB = _c(iB, np.int8)
    M, K = uA.shape
    N = iB.shape[1]
    acc = np.empty((M, N), np.int32)
    _check(lib().oracle_int_gemm(_p(uA), _p(zA), _p(iB), M, N, K, _p(acc)), "int_gemm")
    return acc


def epilogue(acc, scaleA, scaleB, bias=None, *, has_bias=None, act="identity",
             alpha=0.01, typeC="f32"):
    acc = _c(acc, np.int32)
    M, N = acc.shape
    sA = _c(scaleA, np.float32)
    sB = _c(scaleB, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    hb = (b is not None) if has_bias is None else bool(has_bias)
    C_ = np.empty((M, N), _np_type(typeC))
    _check(lib().oracle_epilogue(_p(acc), _p(sA), _p(sB), int(hb), _p(b), _ACT[act],
                                 float(alpha), M, N, _TYPE[typeC], _p(C_)), "epilogue")
    return C_


def dqip_forward(case, rows=None):
    """Forward of one inner-product case (a dict as made by ``workloads``).

    Returns a dict with C and every intermediate: uA, scaleA, zeroA (for the
    selected rows), iB [K,N], scaleB, colsumB, acc. ``rows`` selects a subset
    of the rows of A (all rows when None)."""
    M, N, K = case["M"], case["N"], case["K"]
    A = _c(case["A"], _np_type(case["typeA"]))
    B = _c(case["B"], _np_type(case["typeB"]))
    sB_in = None if case.get("scaleB") is None else _c(case["scaleB"], np.float32)
    if case["typeB"] == "i8" and sB_in is None:
        raise ValueError("an int8 B needs its per-column scales")
    r = None if rows is None else _c(rows, np.int64)
    n = M if r is None else r.size
    bias = case.get("bias")
    b = None if bias is None else _c(bias, np.float32)
    hb = int(case.get("has_bias", b is not None))
    out = dict(uA=np.empty((n, K), np.uint8), scaleA=np.empty(n, np.float32),
               zeroA=np.empty(n, np.int32), iB=np.empty((K, N), np.int8),
               scaleB=np.empty(N, np.float32), acc=np.empty((n, N), np.int32),
               C=np.empty((n, N), _np_type(case["typeC"])))
    rc = lib().oracle_dqip_forward(
        _p(A), _TYPE[case["typeA"]], _p(B), _TYPE[case["typeB"]], _p(sB_in), M, N, K,
        _p(r), n, int(bool(case["avoid"])), hb, _p(b), _ACT[case["act"]],
        float(case.get("alpha", 0.01)), _TYPE[case["typeC"]], _p(out["C"]), _p(out["uA"]),
        _p(out["scaleA"]), _p(out["zeroA"]), _p(out["iB"]), _p(out["scaleB"]), _p(out["acc"]))
    _check(rc, "dqip_forward")
    out["colsumB"] = colsum(out["iB"])
    return out


# ------------------------------------------------------------- QLinearConv

def qlinear_conv(x, x_scale, x_zp, w, w_scale, w_zp, y_scale, y_zp, *, bias=None,
                 y_type="u8"):
    """2-D QLinearConv, stride 1, no padding, group 1; x [N,C,H,W], w [M,C,kH,kW]."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    if w.ndim == 2:
        w = w.reshape(w.shape[0], w.shape[1], 1, 1)
    Nb, Cc, H, W = x.shape
    M, Cw, kH, kW = w.shape
    if Cw != Cc:
        raise ValueError("channel mismatch")
    ws = _c(np.atleast_1d(w_scale), np.float32)
    wz = _c(np.atleast_1d(w_zp), np.int32)
    if ws.size != wz.size:
        raise ValueError("w_scale / w_zero_point shapes differ")
    b = None if bias is None else _c(bias, np.int32)
    y = np.empty((Nb, M, H - kH + 1, W - kW + 1), _np_type(y_type))
    xt = "u8" if x.dtype == np.uint8 else "i8"
    wt = "u8" if w.dtype == np.uint8 else "i8"
    rc = lib().oracle_qlinear_conv(_p(x), _TYPE[xt], Nb, Cc, H, W, float(np.float32(x_scale)),
                                   int(x_zp), _p(w), _TYPE[wt], M, kH, kW, _p(ws), _p(wz),
                                   ws.size, _p(b), float(np.float32(y_scale)), int(y_zp),
                                   _TYPE[y_type], _p(y))
    _check(rc, "qlinear_conv")
    return y


# ------------------------------------------------ QGemm family (R15-R19)

def qlinear_conv2d(x, x_scale, x_zp, w, w_scale, w_zp, y_scale, y_zp, *, bias=None,
                   strides=(1, 1), pads=(0, 0, 0, 0), dilations=(1, 1), group=1,
                   y_type=None, with_acc=False):
    """General 2-D QLinearConv (R11, R25). x [N, C, H, W], w [M, C/group, kH, kW]
    8-bit; pads = (top, left, bottom, right); w_scale / w_zp scalars or per
    output channel. Returns y (and the int32 sums with the bias)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    N, C, H, W = x.shape
    M, _, kH, kW = w.shape
    ws = _c(np.atleast_1d(w_scale), np.float32)
    wz = _c(np.atleast_1d(w_zp), np.int32)
    if wz.size != ws.size:
        wz = np.broadcast_to(wz, ws.shape).astype(np.int32).copy()
    b = None if bias is None else _c(bias, np.int32)
    oH = (H + pads[0] + pads[2] - dilations[0] * (kH - 1) - 1) // strides[0] + 1
    oW = (W + pads[1] + pads[3] - dilations[1] * (kW - 1) - 1) // strides[1] + 1
    yt = y_type or _tag8(x)
    y = np.empty((N, M, oH, oW), _np_type(yt))
    acc = np.empty((N, M, oH, oW), np.int32) if with_acc else None
    rc = lib().oracle_qlinear_conv2d(_p(x), _TYPE[_tag8(x)], N, C, H, W, float(np.float32(x_scale)),
                                     int(x_zp), _p(w), _TYPE[_tag8(w)], M, kH, kW, strides[0],
                                     strides[1], pads[0], pads[1], pads[2], pads[3], dilations[0],
                                     dilations[1], group, _p(ws), _p(wz), ws.size, _p(b),
                                     float(np.float32(y_scale)), int(y_zp), _TYPE[yt], _p(y), _p(acc))
    _check(rc, "qlinear_conv2d")
    return (y, acc) if with_acc else y


def _tag8(a):
    return "u8" if a.dtype == np.uint8 else "i8"


def quantize_tensor_u8(A):
    """Whole-tensor dynamic quantization to uint8 (R19): (scale, zero point, q)."""
    a = _c(A, np.float32)
    q = np.empty(a.shape, np.uint8)
    sc = np.zeros(1, np.float32)
    zp = np.zeros(1, np.int32)
    _check(lib().oracle_quantize_tensor_u8(_p(a), a.size, _p(sc), _p(zp), _p(q)),
           "quantize_tensor_u8")
    return np.float32(sc[0]), int(zp[0]), q


def qgemm(A, B, a_scale, a_zp, b_scale, b_zp=None, *, transA=False, transB=False, C=None,
          alpha=1.0, bias=None, y_scale=None, y_zp=0, y_type=None, with_acc=False):
    """R15-R18. A: (M,K) 8-bit, or (K,M) with transA; B: (K,N), or (N,K) with
    transB. b_scale / b_zp: scalars or length N. C: int32 broadcastable to
    (M,N) (shapes (), (N,), (1,N), (M,1), (M,N)). y_type None: float Y;
    "u8" / "i8": requantized with y_scale / y_zp. with_acc also returns the
    int32 sums sum + C."""
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    M, K = (A.shape[1], A.shape[0]) if transA else A.shape
    Kb, N = (B.shape[1], B.shape[0]) if transB else B.shape
    if Kb != K:
        raise ValueError("inner dimensions differ")
    bs = _c(np.atleast_1d(b_scale), np.float32)
    bz = None if b_zp is None else _c(np.atleast_1d(b_zp), np.int32)
    cm, c_rs, c_cs = None, 0, 0
    if C is not None:
        c = np.asarray(C, np.int32)
        if c.ndim == 0 or c.size == 1:
            cm = _c(c.reshape(1), np.int32)
        elif c.ndim == 1:
            if c.shape[0] != N:
                raise ValueError("C does not broadcast")
            cm, c_cs = _c(c, np.int32), 1
        else:
            if c.shape[0] not in (1, M) or c.shape[1] not in (1, N):
                raise ValueError("C does not broadcast")
            cm = _c(c, np.int32)
            c_rs = c.shape[1] if c.shape[0] == M else 0
            c_cs = 1 if c.shape[1] == N else 0
    bv = None if bias is None else _c(bias, np.float32)
    if y_type is None:
        Y = np.empty((M, N), np.float32)
        yt, ys = "f32", 1.0
    else:
        Y = np.empty((M, N), _np_type(y_type))
        yt, ys = y_type, float(np.float32(y_scale))
    acc = np.empty((M, N), np.int32) if with_acc else None
    rc = lib().oracle_qgemm(_p(A), _TYPE[_tag8(A)], int(bool(transA)), M, K,
                            float(np.float32(a_scale)), int(a_zp), _p(B), _TYPE[_tag8(B)],
                            int(bool(transB)), N, _p(bs), bs.size, _p(bz),
                            0 if bz is None else bz.size, _p(cm), c_rs, c_cs,
                            float(np.float32(alpha)), _p(bv), _TYPE[yt], ys, int(y_zp), _p(Y),
                            _p(acc))
    _check(rc, "qgemm")
    return (Y, acc) if with_acc else Y


def matmul_integer_to_float(A, B, a_scale, b_scale, a_zp=0, b_zp=None, bias=None):
    """MatMulIntegerToFloat (R15, R17): float Y = sum * a_scale * b_scale + bias."""
    return qgemm(A, B, a_scale, a_zp, b_scale, b_zp, bias=bias)


def dynamic_quantize_matmul(A, B, b_scale, b_zp=None, bias=None):
    """DynamicQuantizeMatMul (R19): A float quantized per tensor to uint8,
    then MatMulIntegerToFloat."""
    sc, zp, q = quantize_tensor_u8(A)
    return qgemm(q, B, sc, zp, b_scale, b_zp, bias=bias)


def matmul_batches(a_shape, b_shape):
    """R29: the shapes of an N-dimensional matrix product, by numpy.matmul's
    rules (the schemas' shape inference is ONNX MatMul's, which follows
    numpy). A 1-D A is a single row (that dimension is dropped from Y), a
    1-D B a single column (likewise); the last two dimensions are the
    matrices, the others are batch dimensions, aligned from the right and
    broadcast where one side has 1. Returns (M, N, K, batch shape of Y,
    output shape, [(a batch, b batch) for each Y batch in row-major order]),
    the batch numbers counting A's and B's own batches in row-major order."""
    a_shape, b_shape = tuple(int(d) for d in a_shape), tuple(int(d) for d in b_shape)
    if len(a_shape) == 0 or len(b_shape) == 0:
        raise ValueError("matmul needs at least one dimension per operand")
    a_vec, b_vec = len(a_shape) == 1, len(b_shape) == 1
    a2 = (1,) + a_shape if a_vec else a_shape
    b2 = b_shape + (1,) if b_vec else b_shape
    M, K = a2[-2], a2[-1]
    Kb, N = b2[-2], b2[-1]
    if Kb != K:
        raise ValueError(f"inner dimensions differ: {K} and {Kb}")
    ab, bb = a2[:-2], b2[:-2]
    rank = max(len(ab), len(bb))
    ab = (1,) * (rank - len(ab)) + ab
    bb = (1,) * (rank - len(bb)) + bb
    yb = []
    for da, db in zip(ab, bb):
        if da != db and da != 1 and db != 1:
            raise ValueError(f"batch dimensions {a_shape[:-2]} and {b_shape[:-2]} do not broadcast")
        yb.append(db if da == 1 else da)
    pairs = []
    for idx in np.ndindex(*yb):
        ia = ib = 0
        for d in range(rank):
            ia = ia * ab[d] + (idx[d] if ab[d] > 1 else 0)
            ib = ib * bb[d] + (idx[d] if bb[d] > 1 else 0)
        pairs.append((ia, ib))
    out = tuple(yb) + (() if a_vec else (M,)) + (() if b_vec else (N,))
    return M, N, K, tuple(yb), out, pairs


def matmul_integer_to_float_nd(A, B, a_scale, b_scale, a_zp=0, b_zp=None, bias=None):
    """MatMulIntegerToFloat on N-dimensional A and B (R29): each batch of Y
    is the 2-D product (R15, R17) of its A and B batches; b_scale, b_zp and
    bias (1 or N values) serve every batch."""
    A, B = np.ascontiguousarray(A), np.ascontiguousarray(B)
    M, N, K, yb, out, pairs = matmul_batches(A.shape, B.shape)
    Ab, Bb = A.reshape(-1, M, K), B.reshape(-1, K, N)
    Y = np.empty((len(pairs), M, N), np.float32)
    for z, (ia, ib) in enumerate(pairs):
        Y[z] = matmul_integer_to_float(Ab[ia], Bb[ib], a_scale, b_scale, a_zp, b_zp, bias)
    return Y.reshape(out)


def dynamic_quantize_matmul_nd(A, B, b_scale, b_zp=None, bias=None):
    """DynamicQuantizeMatMul on N-dimensional A and B (R19, R29): A is
    quantized per tensor over all of its batches at once, then
    MatMulIntegerToFloat on the codes."""
    sc, zp, q = quantize_tensor_u8(A)
    return matmul_integer_to_float_nd(q, B, sc, b_scale, zp, b_zp, bias)


# ------------------------------------ element-wise quantized family (R20-R23)

def broadcast_shape(sa, sb):
    """numpy multidirectional broadcasting of two shapes, as the oracle does it."""
    a = np.asarray(sa, np.int64)
    b = np.asarray(sb, np.int64)
    out = np.zeros(8, np.int64)
    ny = C.c_int(0)
    rc = lib().oracle_broadcast_shape(a.size, _p(a), b.size, _p(b), C.byref(ny), _p(out))
    if rc != 0:
        raise ValueError("shapes do not broadcast")
    return tuple(int(v) for v in out[:ny.value])


def _binary(op, A, a_scale, a_zp, B, b_scale, b_zp, c_scale, c_zp):
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if A.dtype != B.dtype or A.dtype not in (np.uint8, np.int8):
        raise ValueError("A and B must share one 8-bit type")
    shape = broadcast_shape(A.shape, B.shape)
    Y = np.empty(shape, np.int32 if op == 2 else A.dtype)
    sa = np.asarray(A.shape, np.int64)
    sb = np.asarray(B.shape, np.int64)
    rc = lib().oracle_qlinear_binary(op, _TYPE[_tag8(A)], _p(A), A.ndim, _p(sa),
                                     float(np.float32(a_scale)), int(a_zp), _p(B), B.ndim,
                                     _p(sb), float(np.float32(b_scale)), int(b_zp),
                                     float(np.float32(c_scale)), int(c_zp), _p(Y))
    _check(rc, "qlinear_binary")
    return Y


def qlinear_add(A, a_scale, a_zp, B, b_scale, b_zp, c_scale, c_zp):
    """QLinearAdd (R20): quantize(A_scale*(A-A_zp) + B_scale*(B-B_zp))."""
    return _binary(0, A, a_scale, a_zp, B, b_scale, b_zp, c_scale, c_zp)


def qlinear_mul(A, a_scale, a_zp, B, b_scale, b_zp, c_scale, c_zp):
    """QLinearMul (R20): quantize((A-A_zp)*(B-B_zp) * (A_scale*B_scale))."""
    return _binary(1, A, a_scale, a_zp, B, b_scale, b_zp, c_scale, c_zp)


def mul_integer(A, a_zp, B, b_zp):
    """MulInteger: int32 (A-A_zp)*(B-B_zp), broadcast."""
    return _binary(2, A, 1.0, a_zp, B, 1.0, b_zp, 1.0, 0)


def _unary(op, X, x_scale, x_zp, y_scale, y_zp, alpha):
    X = np.ascontiguousarray(X)
    Y = np.empty(X.shape, X.dtype)
    rc = lib().oracle_qlinear_unary(op, _TYPE[_tag8(X)], _p(X), X.size,
                                    float(np.float32(x_scale)), int(x_zp),
                                    float(np.float32(y_scale)), int(y_zp),
                                    float(np.float32(alpha)), _p(Y))
    _check(rc, "qlinear_unary")
    return Y


def qlinear_leaky_relu(X, x_scale, x_zp, y_scale, y_zp, alpha=0.01):
    """QLinearLeakyRelu (R20): quantize(alpha*x) for x < 0, else quantize(x)."""
    return _unary(0, X, x_scale, x_zp, y_scale, y_zp, alpha)


def qlinear_sigmoid(X, x_scale, x_zp, y_scale, y_zp):
    """QLinearSigmoid (R21)."""
    return _unary(1, X, x_scale, x_zp, y_scale, y_zp, 0.0)


def _axes_mask(ndim, axes):
    if axes is None:
        return (1 << ndim) - 1
    m = 0
    for a in axes:
        if not -ndim <= a < ndim:
            raise ValueError("axis out of range")
        m |= 1 << (a % ndim)
    return m


def _reduced_shape(shape, mask, keepdims):
    out = []
    for d, n in enumerate(shape):
        if mask & (1 << d):
            if keepdims:
                out.append(1)
        else:
            out.append(n)
    return tuple(out)


def reduce_sum_integer(X, axes=None, keepdims=True):
    """ReduceSumInteger: exact sum; int32 for int8 input, uint32 for uint8."""
    X = np.ascontiguousarray(X)
    mask = _axes_mask(X.ndim, axes)
    Y = np.empty(_reduced_shape(X.shape, mask, keepdims),
                 np.uint32 if X.dtype == np.uint8 else np.int32)
    s = np.asarray(X.shape, np.int64)
    rc = lib().oracle_reduce(0, _TYPE[_tag8(X)], _p(X), X.ndim, _p(s), mask, 1.0, 0, 1.0, 0,
                             _p(Y))
    _check(rc, "reduce_sum_integer")
    return Y


def qlinear_reduce_mean(X, x_scale, x_zp, y_scale, y_zp, axes=None, keepdims=True):
    """QLinearReduceMean (R22)."""
    X = np.ascontiguousarray(X)
    mask = _axes_mask(X.ndim, axes)
    Y = np.empty(_reduced_shape(X.shape, mask, keepdims), X.dtype)
    s = np.asarray(X.shape, np.int64)
    rc = lib().oracle_reduce(1, _TYPE[_tag8(X)], _p(X), X.ndim, _p(s), mask,
                             float(np.float32(x_scale)), int(x_zp),
                             float(np.float32(y_scale)), int(y_zp), _p(Y))
    _check(rc, "qlinear_reduce_mean")
    return Y


def qlinear_concat(inputs, y_scale, y_zp, axis):
    """QLinearConcat (R23). inputs: list of (tensor, scale, zero point), all
    of one 8-bit type and one shape except along axis."""
    xs = [np.ascontiguousarray(t) for t, _, _ in inputs]
    t0 = xs[0]
    ax = axis % t0.ndim
    for x in xs:
        if x.dtype != t0.dtype or x.ndim != t0.ndim or \
                x.shape[:ax] != t0.shape[:ax] or x.shape[ax + 1:] != t0.shape[ax + 1:]:
            raise ValueError("inputs do not concatenate")
    lens = np.asarray([x.shape[ax] for x in xs], np.int64)
    shape = t0.shape[:ax] + (int(lens.sum()),) + t0.shape[ax + 1:]
    Y = np.empty(shape, t0.dtype)
    outer = int(np.prod(t0.shape[:ax], dtype=np.int64))
    inner = int(np.prod(t0.shape[ax + 1:], dtype=np.int64))
    ptrs = (C.c_void_p * len(xs))(*[x.ctypes.data for x in xs])
    sc = np.asarray([np.float32(s) for _, s, _ in inputs], np.float32)
    zp = np.asarray([int(z) for _, _, z in inputs], np.int32)
    rc = lib().oracle_qlinear_concat(_TYPE[_tag8(t0)], len(xs), ptrs, _p(lens), _p(sc), _p(zp),
                                     outer, inner, float(np.float32(y_scale)), int(y_zp), _p(Y))
    _check(rc, "qlinear_concat")
    return Y
