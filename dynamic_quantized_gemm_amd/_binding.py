"""ctypes binding of libdqip.so (see include/dqip.h for the contract of each
entry point). Only marshalling: tensors become device pointers, shapes
become host int64 arrays, None becomes NULL, a non-zero status becomes a
DQError carrying dqip_last_error()."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
# DQIP_LIB_PATH selects another build of the same library (the test suite's
# sanitizer build of the host code); the default is the in-tree library
LIB_PATH = os.environ.get("DQIP_LIB_PATH") or os.path.join(PKG, "libdqip.so")

DQ_F32, DQ_BF16, DQ_I8, DQ_U8, DQ_F16 = 0, 1, 2, 3, 4
DQ_ACT_IDENTITY, DQ_ACT_RELU, DQ_ACT_LEAKY_RELU = 0, 1, 2
DQ_OK, DQ_ERR_ARG, DQ_ERR_TYPE, DQ_ERR_STATE, DQ_ERR_RANGE, DQ_ERR_ALLOC, DQ_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6)
DQ_PER_TENSOR = -(2 ** 31)
DQ_K_MAX = 65536
DQ_QGEMM_K_MAX = 32768
DQ_QGEMM_BATCH_RANK_MAX = 8
DQ_QGEMM_BATCH_MAX = 65536
DQ_LSTM_FORWARD, DQ_LSTM_REVERSE, DQ_LSTM_BIDIRECTIONAL = 0, 1, 2
DQ_LSTM_HIDDEN_MAX = 4096
# dq_rnn_act: ONNX RNN activation name -> (code, takes alpha, default alpha,
# takes beta, default beta)
RNN_ACTIVATIONS = {
    "sigmoid": (0, False, 0.0, False, 0.0), "tanh": (1, False, 0.0, False, 0.0),
    "relu": (2, False, 0.0, False, 0.0), "affine": (3, True, 1.0, True, 0.0),
    "leakyrelu": (4, True, 0.01, False, 0.0), "thresholdedrelu": (5, True, 1.0, False, 0.0),
    "scaledtanh": (6, True, 1.0, True, 1.0), "hardsigmoid": (7, True, 0.2, True, 0.5),
    "elu": (8, True, 1.0, False, 0.0), "softsign": (9, False, 0.0, False, 0.0),
    "softplus": (10, False, 0.0, False, 0.0),
}

_lib = None

_SIGNATURES = {
    # name: (restype, argtypes)
    "dqip_init": (C.c_int, [C.POINTER(C.c_void_p), C.c_size_t, C.c_size_t, C.c_size_t, C.c_int,
                            C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int]),
    "dqip_enabled": (C.c_int, [C.c_void_p]),
    "dqip_internal_buffer_size": (C.c_size_t, [C.c_void_p]),
    "dqip_external_buffer_size": (C.c_size_t, [C.c_void_p]),
    "dqip_info": (C.c_char_p, [C.c_void_p]),
    "dqip_set_params": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p]),
    "dqip_forward": (C.c_int, [C.c_void_p] + [C.c_void_p] * 5),
    "dqip_forward_noalloc": (C.c_int, [C.c_void_p] * 5),
    "dqip_release": (None, [C.c_void_p]),
    "dqip_last_error": (C.c_char_p, []),
    "dqip_read_quantized_a": (C.c_int, [C.c_void_p] * 6),
    "dqip_read_quantized_b": (C.c_int, [C.c_void_p] * 6),
    "dqip_forward_accumulators": (C.c_int, [C.c_void_p] * 6),
    "dqip_profile_begin": (C.c_int, [C.c_void_p, C.c_int]),
    "dqip_profile_end": (C.c_int, [C.c_void_p, C.POINTER(C.c_float), C.POINTER(C.c_int)]),
    "dq_probe_mfma_loop": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p]),
    "dq_probe_copy": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "qlinear_quantize": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                   C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "qlinear_dequantize": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                     C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "qlinear_conv1x1": (C.c_int, [C.c_void_p, C.c_int, C.c_int64, C.c_int64, C.c_int64,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_int64,
                                  C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                  C.c_int, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_qgemm_init": (C.c_int, [C.POINTER(C.c_void_p), C.c_int64, C.c_int64, C.c_int64, C.c_int,
                                C.c_int, C.c_int, C.c_int, C.c_int, C.c_float]),
    "dq_qgemm_init_batched": (C.c_int, [C.POINTER(C.c_void_p), C.c_int, C.c_void_p, C.c_void_p,
                                        C.c_int64, C.c_int64, C.c_int64, C.c_int, C.c_int]),
    "dq_qgemm_set_b": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                                 C.c_int64, C.c_void_p]),
    "dq_qgemm_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_int64, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p]),
    "dq_qgemm_forward_accumulators": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                                C.c_void_p, C.c_int64, C.c_int64, C.c_void_p,
                                                C.c_void_p]),
    "dq_qgemm_info": (C.c_char_p, [C.c_void_p]),
    "dq_qgemm_release": (None, [C.c_void_p]),
    "qlinear_quantize_f16": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int, C.c_void_p,
                                       C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "qlinear_dequantize_f16": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_int,
                                         C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "dq_qconv_init": (C.c_int, [C.POINTER(C.c_void_p), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                                C.c_int64, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                C.c_int, C.c_int, C.c_int]),
    "dq_qconv_output_shape": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_qconv_set_w": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                 C.c_void_p, C.c_void_p]),
    "dq_qconv_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                   C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_qconv_info": (C.c_char_p, [C.c_void_p]),
    "dq_lstm_init": (C.c_int, [C.POINTER(C.c_void_p), C.c_int64, C.c_int64, C.c_int64, C.c_int64,
                               C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_float, C.c_int]),
    "dq_lstm_set_weights": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p]),
    "dq_lstm_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "dq_lstm_info": (C.c_char_p, [C.c_void_p]),
    "dq_lstm_release": (None, [C.c_void_p]),
    "dq_qconv_release": (None, [C.c_void_p]),
    "qlinear_add": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "qlinear_mul": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "dq_mul_integer": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                 C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                 C.c_void_p]),
    "qlinear_leaky_relu": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                     C.c_void_p, C.c_float, C.c_int, C.c_void_p, C.c_void_p]),
    "qlinear_sigmoid": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]),
    "dq_reduce_sum_integer": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                        C.c_int, C.c_void_p, C.c_void_p]),
    "qlinear_reduce_mean": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_void_p,
                                      C.c_int, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_void_p, C.c_void_p]),
    "qlinear_concat": (C.c_int, [C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                 C.c_void_p]),
}


class DQError(RuntimeError):
    def __init__(self, status: int, what: str, message: str):
        super().__init__(f"{what} failed with status {status}: {message}")
        self.status = status


def load() -> C.CDLL:
    """Load libdqip.so (built by ``python dynamic_quantized_gemm_amd/build.py``).
    Raises when it is missing: the library has no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run dynamic_quantized_gemm_amd/build.py")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


_ELEM = {DQ_F32: 4, DQ_BF16: 2, DQ_I8: 1, DQ_U8: 1, DQ_F16: 2}


def _ptr(t, what="tensor", nbytes=0):
    """Device pointer of a tensor / int / None. A tensor must be a dense
    (contiguous) device tensor of at least `nbytes` bytes: the kernels index
    it as such, and a short or strided buffer would be read or written out of
    bounds. A plain int is taken as a device pointer whose extent is the
    caller's to guarantee."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if t.device.type != "cuda":
        raise DQError(DQ_ERR_ARG, what, "not a device tensor")
    if not t.is_contiguous():
        raise DQError(DQ_ERR_ARG, what, "not contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise DQError(DQ_ERR_ARG, what, f"holds {have} bytes, {nbytes} needed")
    return t.data_ptr()


# sizes of each context made by dqip_init, for the binding's extent checks
_DQIP_DIMS = {}


def _current_stream():
    """Handle of torch's current stream on the current device. The raw
    accessor skips building a Stream object (about 2.5 us a call); the
    public call is the fallback where torch lacks it."""
    import torch

    raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
    if raw is not None:
        return raw(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream(stream):
    if stream is None:
        return _current_stream()
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str):
    if rc != DQ_OK:
        msg = load().dqip_last_error()
        raise DQError(rc, what, msg.decode() if msg else "")


# ------------------------------------------------------------------ DQIP

def dqip_init(M, N, K, typeA, typeB, typeC, constB, bias, activation, avoidOverflow, ctx=None):
    """Returns the context handle (an int); pass the previous one as ``ctx``
    to re-initialize (kept as is when nothing changed)."""
    h = C.c_void_p(ctx)
    _check(load().dqip_init(C.byref(h), M, N, K, typeA, typeB, typeC, int(bool(constB)),
                            int(bool(bias)), activation, int(bool(avoidOverflow))), "dqip_init")
    if ctx is not None and ctx != h.value:
        _DQIP_DIMS.pop(ctx, None)
    _DQIP_DIMS[h.value] = (int(M), int(N), int(K), typeA, typeB, typeC)
    return h.value


def _dims(ctx):
    return _DQIP_DIMS.get(ctx, (0, 0, 0, DQ_I8, DQ_I8, DQ_I8))


def _ext_bytes(ctx, buf):
    """Bytes a work-buffer tensor must hold (0: no tensor to check)."""
    if ctx in _DQIP_DIMS and buf is not None and not isinstance(buf, int):
        return dqip_external_buffer_size(ctx)
    return 0


def dqip_enabled(ctx) -> bool:
    return bool(load().dqip_enabled(ctx))


def dqip_internal_buffer_size(ctx) -> int:
    return int(load().dqip_internal_buffer_size(ctx))


def dqip_external_buffer_size(ctx) -> int:
    return int(load().dqip_external_buffer_size(ctx))


def dqip_info(ctx):
    s = load().dqip_info(ctx)
    return None if s is None else s.decode()


def dqip_set_params(ctx, weight, scale=None, bias=None, params=None, stream=None):
    """params: a sequence of floats (host), e.g. [slope] for leaky ReLU."""
    p = None
    if params is not None:
        arr = (C.c_float * len(params))(*params)
        p = C.addressof(arr)
    M, N, K, tA, tB, tC = _dims(ctx)
    w = "dqip_set_params"
    _check(load().dqip_set_params(ctx, _ptr(weight, w, K * N * _ELEM[tB]), _ptr(scale, w, 4 * N),
                                  _ptr(bias, w, 4 * N), p, _stream(stream)), w)


def _fwd_args(ctx, A, B, buf, out, out_elem, w):
    M, N, K, tA, tB, tC = _dims(ctx)
    ext = _ext_bytes(ctx, buf)
    return (_ptr(A, w, M * K * _ELEM[tA]), _ptr(B, w, K * N * _ELEM[tB]), _ptr(buf, w, ext),
            _ptr(out, w, M * N * (out_elem or _ELEM[tC])))


def dqip_forward(ctx, A, B, buf, C_, stream=None):
    _check(load().dqip_forward(ctx, *_fwd_args(ctx, A, B, buf, C_, 0, "dqip_forward"),
                               _stream(stream)), "dqip_forward")


DQIP_NOALLOC_SCRATCH_BYTES = 32 << 20


def dqip_forward_noalloc(ctx, A, B, C_, stream=None):
    a, b, _, c = _fwd_args(ctx, A, B, None, C_, 0, "dqip_forward_noalloc")
    _check(load().dqip_forward_noalloc(ctx, a, b, c, _stream(stream)), "dqip_forward_noalloc")


def dqip_forward_accumulators(ctx, A, B, buf, acc, stream=None):
    _check(load().dqip_forward_accumulators(ctx, *_fwd_args(ctx, A, B, buf, acc, 4,
                                                            "dqip_forward_accumulators"),
                                            _stream(stream)), "dqip_forward_accumulators")


def dqip_release(ctx):
    _DQIP_DIMS.pop(ctx, None)
    load().dqip_release(ctx)


def dqip_last_error() -> str:
    s = load().dqip_last_error()
    return s.decode() if s else ""


def dqip_read_quantized_a(ctx, buf, uA=None, scaleA=None, zeroA=None, stream=None):
    M, N, K = _dims(ctx)[:3]
    w = "dqip_read_quantized_a"
    ext = _ext_bytes(ctx, buf)
    _check(load().dqip_read_quantized_a(ctx, _ptr(buf, w, ext), _ptr(uA, w, M * K), _ptr(scaleA, w, 4 * M),
                                        _ptr(zeroA, w, 4 * M), _stream(stream)), w)


def dqip_read_quantized_b(ctx, buf, iB=None, scaleB=None, colsumB=None, stream=None):
    M, N, K = _dims(ctx)[:3]
    w = "dqip_read_quantized_b"
    ext = _ext_bytes(ctx, buf)
    _check(load().dqip_read_quantized_b(ctx, _ptr(buf, w, ext), _ptr(iB, w, K * N), _ptr(scaleB, w, 4 * N),
                                        _ptr(colsumB, w, 4 * N), _stream(stream)), w)


def dqip_profile_begin(ctx, capacity):
    _check(load().dqip_profile_begin(ctx, int(capacity)), "dqip_profile_begin")


def dqip_profile_end(ctx):
    """Returns (summed ms per phase [quant_a, quant_b, gemm], recorded calls)."""
    ms = (C.c_float * 3)()
    n = C.c_int(0)
    _check(load().dqip_profile_end(ctx, ms, C.byref(n)), "dqip_profile_end")
    return [float(v) for v in ms], int(n.value)


# ------------------------------------------------------ measurement probes

def dq_probe_mfma_loop(operands, shape, iters, workgroups, sink, stream=None):
    """operands: >= 64 KiB device tensor; shape 16 or 32; sink: >= workgroups * 256 int32."""
    w = "dq_probe_mfma_loop"
    _check(load().dq_probe_mfma_loop(_ptr(operands, w, 65536), int(shape), int(iters), int(workgroups),
                                     _ptr(sink, w, 1024 * int(workgroups)), _stream(stream)), w)


def dq_probe_copy(src, dst, nbytes, stream=None):
    w = "dq_probe_copy"
    _check(load().dq_probe_copy(_ptr(src, w, nbytes), _ptr(dst, w, nbytes), int(nbytes), _stream(stream)), w)


# ------------------------------------------------------ Q / DQ operators

def _numel(shape):
    n = 1
    for d in shape:
        n *= int(d)
    return n


def _shape_arg(shape):
    arr = (C.c_int64 * max(1, len(shape)))(*[int(s) for s in shape])
    return C.addressof(arr), arr


def _axis_len(shape, axis):
    """Entries of a per-axis scale / zero point (1 per tensor); 0 when the
    axis is out of range (the library reports that error itself)."""
    if axis == DQ_PER_TENSOR:
        return 1
    a = int(axis) + (len(shape) if axis < 0 else 0)
    return int(shape[a]) if 0 <= a < len(shape) else 0


def _bcast_numel(sa, sb):
    """Elements of the numpy broadcast of two shapes (0 if they do not
    broadcast: the library reports that error itself)."""
    n = max(len(sa), len(sb))
    a = (1,) * (n - len(sa)) + tuple(int(v) for v in sa)
    b = (1,) * (n - len(sb)) + tuple(int(v) for v in sb)
    out = 1
    for x, y in zip(a, b):
        if x != y and x != 1 and y != 1:
            return 0
        out *= y if x == 1 else x
    return out


def _kept_numel(shape, axes):
    """Elements left after reducing `axes` (None or empty: all) of `shape`."""
    if not axes:
        return 1
    nd = len(shape)
    red = {int(a) + (nd if a < 0 else 0) for a in axes}
    return _numel([d for i, d in enumerate(shape) if i not in red])


def qlinear_quantize(x, y_scale, y_zero_point, y_type, y, axis=DQ_PER_TENSOR, shape=None,
                     stream=None):
    """x: fp32 tensor; y: int8/uint8 tensor of the same shape (written)."""
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, keep = _shape_arg(shp)
    n, w, na = _numel(shp), "qlinear_quantize", _axis_len(shp, axis)
    _check(load().qlinear_quantize(_ptr(x, w, 4 * n), len(shp), sp, axis, _ptr(y_scale, w, 4 * na),
                                   _ptr(y_zero_point, w, na), y_type, _ptr(y, w, n), _stream(stream)), w)
    del keep


def qlinear_dequantize(x, x_type, x_scale, x_zero_point, y, axis=DQ_PER_TENSOR, shape=None,
                       stream=None):
    """x: int8/uint8 tensor; y: fp32 tensor of the same shape (written)."""
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, keep = _shape_arg(shp)
    n, w, na = _numel(shp), "qlinear_dequantize", _axis_len(shp, axis)
    _check(load().qlinear_dequantize(_ptr(x, w, n), x_type, len(shp), sp, axis, _ptr(x_scale, w, 4 * na),
                                     _ptr(x_zero_point, w, na), _ptr(y, w, 4 * n), _stream(stream)), w)
    del keep


def qlinear_quantize_f16(x, y_scale, y_zero_point, y_type, y, axis=DQ_PER_TENSOR, shape=None,
                         stream=None):
    """x, y_scale: fp16 tensors; y: int8/uint8 tensor of x's shape (written)."""
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, keep = _shape_arg(shp)
    n, w, na = _numel(shp), "qlinear_quantize_f16", _axis_len(shp, axis)
    _check(load().qlinear_quantize_f16(_ptr(x, w, 2 * n), len(shp), sp, axis, _ptr(y_scale, w, 2 * na),
                                       _ptr(y_zero_point, w, na), y_type, _ptr(y, w, n), _stream(stream)),
           w)
    del keep


def qlinear_dequantize_f16(x, x_type, x_scale, x_zero_point, y_type, y, axis=DQ_PER_TENSOR,
                           shape=None, stream=None):
    """x_scale: fp16 tensor; y: fp16 (y_type DQ_F16) or fp32 (DQ_F32) tensor."""
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, keep = _shape_arg(shp)
    n, w, na = _numel(shp), "qlinear_dequantize_f16", _axis_len(shp, axis)
    ye = 2 if y_type == DQ_F16 else 4
    _check(load().qlinear_dequantize_f16(_ptr(x, w, n), x_type, len(shp), sp, axis, _ptr(x_scale, w, 2 * na),
                                         _ptr(x_zero_point, w, na), y_type, _ptr(y, w, ye * n),
                                         _stream(stream)),
           w)
    del keep


def qlinear_conv1x1(x, x_type, x_scale, x_zero_point, w, w_type, w_scale, w_zero_point,
                    y_scale, y_zero_point, y_type, bias, y, *, N=None, C_=None, HW=None, M=None,
                    w_len=None, stream=None):
    """x: [N, C, H, W] (or [N, C, HW]) 8-bit tensor; w: [M, C] (or [M, C, 1, 1]);
    y: [N, M, H, W] 8-bit tensor (written). Scales / zero points / bias are
    device tensors or None (zero points and bias); sizes default to the
    tensors' shapes."""
    if N is None:
        N, C_ = int(x.shape[0]), int(x.shape[1])
        HW = 1
        for d in x.shape[2:]:
            HW *= int(d)
        M = int(w.shape[0])
    if w_len is None:
        w_len = int(w_scale.numel())
    n = "qlinear_conv1x1"
    _check(load().qlinear_conv1x1(_ptr(x, n, N * C_ * HW), x_type, N, C_, HW, _ptr(x_scale, n, 4),
                                  _ptr(x_zero_point, n, 1), _ptr(w, n, M * C_), w_type, M,
                                  _ptr(w_scale, n, 4 * w_len), _ptr(w_zero_point, n, w_len), w_len,
                                  _ptr(y_scale, n, 4), _ptr(y_zero_point, n, 1), y_type,
                                  _ptr(bias, n, 4 * M), _ptr(y, n, N * M * HW), _stream(stream)), n)


# ------------------------------------------- QGemm / MatMulIntegerToFloat

# sizes of each context made by dq_qgemm_init, for the extent checks
_QGEMM_DIMS = {}


def dq_qgemm_init(M, N, K, a_type, transA, b_type, transB, y_type, alpha=1.0):
    """Returns the context handle (an int)."""
    h = C.c_void_p()
    _check(load().dq_qgemm_init(C.byref(h), M, N, K, a_type, int(bool(transA)), b_type,
                                int(bool(transB)), y_type, float(alpha)), "dq_qgemm_init")
    _QGEMM_DIMS[h.value] = (int(M), int(N), int(K), a_type, y_type, 1, 1, 1)
    return h.value


def dq_qgemm_init_batched(a_batch, b_batch, M, N, K, a_type, b_type):
    """a_batch / b_batch: the batch dimensions of A and B (sequences, the
    shorter left-padded with 1 here). Returns the context handle (an int).
    A is then [prod(a_batch), M, K], B [prod(b_batch), K, N] and Y (fp32)
    [prod(broadcast batch), M, N]."""
    ab, bb = [int(d) for d in a_batch], [int(d) for d in b_batch]
    rank = max(len(ab), len(bb))
    ab = [1] * (rank - len(ab)) + ab
    bb = [1] * (rank - len(bb)) + bb
    arr = C.c_int64 * max(rank, 1)
    pa, pb = arr(*ab), arr(*bb)
    h = C.c_void_p()
    _check(load().dq_qgemm_init_batched(C.byref(h), rank, C.addressof(pa), C.addressof(pb), M, N, K,
                                        a_type, b_type), "dq_qgemm_init_batched")
    na = nb = ny = 1
    for da, db in zip(ab, bb):
        na, nb, ny = na * da, nb * db, ny * (db if da == 1 else da)
    _QGEMM_DIMS[h.value] = (int(M), int(N), int(K), a_type, DQ_F32, na, nb, ny)
    return h.value


def _qgemm_dims(ctx):
    return _QGEMM_DIMS.get(ctx, (0, 0, 0, DQ_U8, DQ_U8, 1, 1, 1))


def dq_qgemm_set_b(ctx, B, b_scale, b_zero_point=None, stream=None):
    """B: 8-bit tensor ([K,N], or [N,K] with transB; [B batches, K, N] for a
    batched context); b_scale: fp32 tensor of 1 or N values; b_zero_point:
    tensor of B's type (1 or N values) or None."""
    bz_len = 0 if b_zero_point is None else int(b_zero_point.numel())
    M, N, K, _, _, _, nb, _ = _qgemm_dims(ctx)
    w = "dq_qgemm_set_b"
    _check(load().dq_qgemm_set_b(ctx, _ptr(B, w, nb * K * N), _ptr(b_scale, w, 4 * int(b_scale.numel())),
                                 int(b_scale.numel()), _ptr(b_zero_point, w, bz_len), bz_len,
                                 _stream(stream)), w)


def _c_shape(C_):
    if C_ is None:
        return 0, 0
    if C_.dim() <= 1:
        return 1, int(C_.numel())
    return int(C_.shape[0]), int(C_.shape[1])


def dq_qgemm_forward(ctx, A, a_scale, a_zero_point, C_, bias, y_scale, y_zero_point, Y,
                     stream=None):
    """C_: int32 tensor of shape (), (N,), (1, N), (M, 1) or (M, N), or None."""
    cr, cc = _c_shape(C_)
    M, N, K, ta, ty, na, _, ny = _qgemm_dims(ctx)
    w = "dq_qgemm_forward"
    _check(load().dq_qgemm_forward(ctx, _ptr(A, w, na * M * K * _ELEM[ta]), _ptr(a_scale, w, 4),
                                   _ptr(a_zero_point, w, 1), _ptr(C_, w, 4 * cr * cc), cr, cc,
                                   _ptr(bias, w, 4 * N), _ptr(y_scale, w, 4), _ptr(y_zero_point, w, 1),
                                   _ptr(Y, w, ny * M * N * _ELEM[ty]), _stream(stream)), w)


def dq_qgemm_forward_accumulators(ctx, A, a_scale, a_zero_point, C_, acc, stream=None):
    cr, cc = _c_shape(C_)
    M, N, K, ta, _, na, _, ny = _qgemm_dims(ctx)
    w = "dq_qgemm_forward_accumulators"
    _check(load().dq_qgemm_forward_accumulators(ctx, _ptr(A, w, na * M * K * _ELEM[ta]), _ptr(a_scale, w, 4),
                                                _ptr(a_zero_point, w, 1), _ptr(C_, w, 4 * cr * cc), cr,
                                                cc, _ptr(acc, w, 4 * ny * M * N), _stream(stream)), w)


def dq_qgemm_info(ctx):
    r = load().dq_qgemm_info(ctx)
    return r.decode() if r else None


def dq_qgemm_release(ctx):
    _QGEMM_DIMS.pop(ctx, None)
    load().dq_qgemm_release(ctx)


# ----------------------------------------- element-wise quantized operators

def _binary(fn, what, A, a_scale, a_zero_point, B, b_scale, b_zero_point, c_scale, c_zero_point,
            type_, C_, stream, a_shape, b_shape):
    sa = tuple(A.shape) if a_shape is None else tuple(a_shape)
    sb = tuple(B.shape) if b_shape is None else tuple(b_shape)
    pa, ka = _shape_arg(sa)
    pb, kb = _shape_arg(sb)
    nc = _bcast_numel(sa, sb)
    if fn == "dq_mul_integer":
        rc = load().dq_mul_integer(_ptr(A, what, _numel(sa)), len(sa), pa, _ptr(a_zero_point, what, 1),
                                   _ptr(B, what, _numel(sb)), len(sb), pb, _ptr(b_zero_point, what, 1),
                                   type_, _ptr(C_, what, 4 * nc), _stream(stream))
    else:
        rc = getattr(load(), fn)(_ptr(A, what, _numel(sa)), len(sa), pa, _ptr(a_scale, what, 4),
                                 _ptr(a_zero_point, what, 1), _ptr(B, what, _numel(sb)), len(sb), pb,
                                 _ptr(b_scale, what, 4), _ptr(b_zero_point, what, 1),
                                 _ptr(c_scale, what, 4), _ptr(c_zero_point, what, 1), type_,
                                 _ptr(C_, what, nc), _stream(stream))
    del ka, kb
    _check(rc, what)


def qlinear_add(A, a_scale, a_zero_point, B, b_scale, b_zero_point, c_scale, c_zero_point, type_,
                C_, stream=None, a_shape=None, b_shape=None):
    """A, B: 8-bit tensors broadcasting to C_'s shape (C_ written)."""
    _binary("qlinear_add", "qlinear_add", A, a_scale, a_zero_point, B, b_scale, b_zero_point,
            c_scale, c_zero_point, type_, C_, stream, a_shape, b_shape)


def qlinear_mul(A, a_scale, a_zero_point, B, b_scale, b_zero_point, c_scale, c_zero_point, type_,
                C_, stream=None, a_shape=None, b_shape=None):
    _binary("qlinear_mul", "qlinear_mul", A, a_scale, a_zero_point, B, b_scale, b_zero_point,
            c_scale, c_zero_point, type_, C_, stream, a_shape, b_shape)


def dq_mul_integer(A, a_zero_point, B, b_zero_point, type_, C_, stream=None, a_shape=None,
                   b_shape=None):
    """C_: int32 tensor of the broadcast shape (written)."""
    _binary("dq_mul_integer", "dq_mul_integer", A, None, a_zero_point, B, None, b_zero_point,
            None, None, type_, C_, stream, a_shape, b_shape)


def qlinear_leaky_relu(x, x_scale, x_zero_point, y_scale, y_zero_point, type_, y, alpha=0.01,
                       n=None, stream=None):
    n = int(x.numel()) if n is None else int(n)
    w = "qlinear_leaky_relu"
    _check(load().qlinear_leaky_relu(_ptr(x, w, n), n, _ptr(x_scale, w, 4), _ptr(x_zero_point, w, 1),
                                     _ptr(y_scale, w, 4), _ptr(y_zero_point, w, 1), float(alpha), type_,
                                     _ptr(y, w, n), _stream(stream)), w)


def qlinear_sigmoid(x, x_scale, x_zero_point, y_scale, y_zero_point, type_, y, n=None,
                    stream=None):
    n = int(x.numel()) if n is None else int(n)
    w = "qlinear_sigmoid"
    _check(load().qlinear_sigmoid(_ptr(x, w, n), n, _ptr(x_scale, w, 4), _ptr(x_zero_point, w, 1),
                                  _ptr(y_scale, w, 4), _ptr(y_zero_point, w, 1), type_, _ptr(y, w, n),
                                  _stream(stream)), w)


def _axes_arg(axes):
    axes = [] if axes is None else [int(a) for a in axes]
    arr = (C.c_int32 * max(1, len(axes)))(*axes)
    return C.addressof(arr), len(axes), arr


def dq_reduce_sum_integer(x, type_, axes, y, shape=None, stream=None):
    """y: int32 tensor holding the kept dims (written); axes None = all."""
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, ks = _shape_arg(shp)
    ap, na, ka = _axes_arg(axes)
    w = "dq_reduce_sum_integer"
    _check(load().dq_reduce_sum_integer(_ptr(x, w, _numel(shp)), type_, len(shp), sp, ap if na else None,
                                        na, _ptr(y, w, 4 * _kept_numel(shp, axes)), _stream(stream)), w)
    del ks, ka


def qlinear_reduce_mean(x, type_, axes, x_scale, x_zero_point, y_scale, y_zero_point, y,
                        shape=None, stream=None):
    shp = tuple(x.shape) if shape is None else tuple(shape)
    sp, ks = _shape_arg(shp)
    ap, na, ka = _axes_arg(axes)
    w = "qlinear_reduce_mean"
    _check(load().qlinear_reduce_mean(_ptr(x, w, _numel(shp)), type_, len(shp), sp, ap if na else None,
                                      na, _ptr(x_scale, w, 4), _ptr(x_zero_point, w, 1),
                                      _ptr(y_scale, w, 4), _ptr(y_zero_point, w, 1),
                                      _ptr(y, w, _kept_numel(shp, axes)), _stream(stream)), w)
    del ks, ka


def qlinear_concat(inputs, axis, y_scale, y_zero_point, type_, y, shapes=None, stream=None):
    """inputs: sequence of (tensor, scale tensor, zero point tensor or None)."""
    n = len(inputs)
    shp = [tuple(t.shape) for t, _, _ in inputs] if shapes is None else [tuple(s) for s in shapes]
    nd = len(shp[0]) if shp else 0
    flat = (C.c_int64 * max(1, n * nd))(*[int(v) for s in shp for v in s])
    w = "qlinear_concat"
    xs = (C.c_void_p * max(1, n))(*[_ptr(t, w, _numel(s)) for (t, _, _), s in zip(inputs, shp)])
    sc = (C.c_void_p * max(1, n))(*[_ptr(s, w, 4) for _, s, _ in inputs])
    zp = (C.c_void_p * max(1, n))(*[_ptr(z, w, 1) for _, _, z in inputs])
    _ptr(y, w, sum(_numel(s) for s in shp))
    _check(load().qlinear_concat(n, C.addressof(xs), C.addressof(flat), nd, int(axis),
                                 C.addressof(sc), C.addressof(zp), _ptr(y_scale),
                                 _ptr(y_zero_point), type_, _ptr(y), _stream(stream)),
           "qlinear_concat")


# ------------------------------------------------------ general QLinearConv

def dq_qconv_init(C_, H, W, M, kH, kW, x_type, w_type, y_type, strides=(1, 1),
                  pads=(0, 0, 0, 0), dilations=(1, 1), group=1):
    """Returns the context handle (an int). pads = (top, left, bottom, right)."""
    st = (C.c_int64 * 2)(*[int(v) for v in strides])
    pd = (C.c_int64 * 4)(*[int(v) for v in pads])
    dl = (C.c_int64 * 2)(*[int(v) for v in dilations])
    h = C.c_void_p()
    _check(load().dq_qconv_init(C.byref(h), C_, H, W, M, kH, kW, C.addressof(st),
                                C.addressof(pd), C.addressof(dl), group, x_type,
                                w_type, y_type), "dq_qconv_init")
    oh, ow = dq_qconv_output_shape(h.value)
    _QCONV_DIMS[h.value] = (int(C_), int(H), int(W), int(M), int(kH), int(kW), int(group), oh, ow)
    return h.value


# sizes of each context made by dq_qconv_init, for the extent checks
_QCONV_DIMS = {}


def dq_qconv_output_shape(ctx):
    oh, ow = C.c_int64(), C.c_int64()
    _check(load().dq_qconv_output_shape(ctx, C.byref(oh), C.byref(ow)), "dq_qconv_output_shape")
    return int(oh.value), int(ow.value)


def dq_qconv_set_w(ctx, w, w_scale, w_zero_point=None, bias=None, stream=None):
    C_, H, W, M, kH, kW, g = _QCONV_DIMS.get(ctx, (0, 0, 0, 0, 0, 0, 1, 0, 0))[:7]
    n, wl = "dq_qconv_set_w", int(w_scale.numel())
    _check(load().dq_qconv_set_w(ctx, _ptr(w, n, M * (C_ // max(g, 1)) * kH * kW), _ptr(w_scale, n, 4 * wl),
                                 _ptr(w_zero_point, n, wl), wl, _ptr(bias, n, 4 * M), _stream(stream)),
           n)


def dq_qconv_forward(ctx, x, x_scale, x_zero_point, y_scale, y_zero_point, y, N=None,
                     stream=None):
    n = int(x.shape[0]) if N is None else int(N)
    C_, H, W, M, _, _, _, oh, ow = _QCONV_DIMS.get(ctx, (0, 0, 0, 0, 0, 0, 1, 0, 0))
    w = "dq_qconv_forward"
    _check(load().dq_qconv_forward(ctx, _ptr(x, w, n * C_ * H * W), n, _ptr(x_scale, w, 4),
                                   _ptr(x_zero_point, w, 1), _ptr(y_scale, w, 4), _ptr(y_zero_point, w, 1),
                                   _ptr(y, w, n * M * oh * ow), _stream(stream)), w)


def dq_qconv_info(ctx):
    r = load().dq_qconv_info(ctx)
    return r.decode() if r else None


def dq_qconv_release(ctx):
    _QCONV_DIMS.pop(ctx, None)
    load().dq_qconv_release(ctx)


# ------------------------------------------------------ DynamicQuantizeLSTM

def lstm_activation_slots(activations=None, activation_alpha=None, activation_beta=None, dirs=1):
    """The ONNX attributes (names, and alpha / beta lists consumed in order by
    the activations that take the parameter) as per-slot arrays for
    dq_lstm_init: (codes, alphas, betas), 3 * dirs each."""
    names = ["Sigmoid", "Tanh", "Tanh"] * dirs if activations is None else list(activations)
    if len(names) != 3 * dirs:
        raise ValueError(f"{3 * dirs} activations expected")
    al = list(activation_alpha or [])
    be = list(activation_beta or [])
    codes, alphas, betas = [], [], []
    for n in names:
        key = n.lower()
        if key not in RNN_ACTIVATIONS:
            raise ValueError(f"activation {n} is not supported")
        code, ta, da, tb, db = RNN_ACTIVATIONS[key]
        codes.append(code)
        alphas.append(al.pop(0) if ta and al else da)
        betas.append(be.pop(0) if tb and be else db)
    return codes, alphas, betas


def dq_lstm_init(seq_length, batch_size, input_size, hidden_size, direction, w_type, r_type,
                 activations=None, activation_alpha=None, activation_beta=None, clip=0.0,
                 input_forget=0):
    """direction: DQ_LSTM_* code or "forward" / "reverse" / "bidirectional";
    activations etc. as the ONNX attributes. Returns the context handle."""
    if isinstance(direction, str):
        direction = {"forward": DQ_LSTM_FORWARD, "reverse": DQ_LSTM_REVERSE,
                     "bidirectional": DQ_LSTM_BIDIRECTIONAL}[direction]
    dirs = 2 if direction == DQ_LSTM_BIDIRECTIONAL else 1
    codes, alphas, betas = lstm_activation_slots(activations, activation_alpha, activation_beta, dirs)
    ca = (C.c_int * len(codes))(*codes)
    aa = (C.c_float * len(alphas))(*alphas)
    ba = (C.c_float * len(betas))(*betas)
    h = C.c_void_p()
    _check(load().dq_lstm_init(C.byref(h), int(seq_length), int(batch_size), int(input_size),
                               int(hidden_size), int(direction), int(w_type), int(r_type),
                               C.addressof(ca), C.addressof(aa),
                               C.addressof(ba), float(clip or 0.0), int(input_forget)),
           "dq_lstm_init")
    _LSTM_DIMS[h.value] = (int(seq_length), int(batch_size), int(input_size), int(hidden_size), dirs)
    return h.value


# sizes of each context made by dq_lstm_init, for the extent checks
_LSTM_DIMS = {}


def dq_lstm_set_weights(ctx, W, W_scale, W_zero_point, R, R_scale, R_zero_point, B=None, P=None,
                        stream=None):
    seq, bt, ni, h, d = _LSTM_DIMS.get(ctx, (0, 0, 0, 0, 0))
    n, ws, rs = "dq_lstm_set_weights", int(W_scale.numel()), int(R_scale.numel())
    _check(load().dq_lstm_set_weights(ctx, _ptr(W, n, d * ni * 4 * h), _ptr(W_scale, n, 4 * ws), ws,
                                      _ptr(W_zero_point, n, ws), _ptr(R, n, d * h * 4 * h),
                                      _ptr(R_scale, n, 4 * rs), rs, _ptr(R_zero_point, n, rs),
                                      _ptr(B, n, 4 * d * 8 * h), _ptr(P, n, 4 * d * 3 * h),
                                      _stream(stream)), n)


def dq_lstm_forward(ctx, X, sequence_lens=None, initial_h=None, initial_c=None, Y=None, Y_h=None,
                    Y_c=None, stream=None):
    seq, bt, ni, h, d = _LSTM_DIMS.get(ctx, (0, 0, 0, 0, 0))
    n, st = "dq_lstm_forward", 4 * d * bt * h
    _check(load().dq_lstm_forward(ctx, _ptr(X, n, 4 * seq * bt * ni), _ptr(sequence_lens, n, 4 * bt),
                                  _ptr(initial_h, n, st), _ptr(initial_c, n, st),
                                  _ptr(Y, n, 4 * seq * d * bt * h), _ptr(Y_h, n, st), _ptr(Y_c, n, st),
                                  _stream(stream)), n)


def dq_lstm_info(ctx):
    r = load().dq_lstm_info(ctx)
    return r.decode() if r else None


def dq_lstm_release(ctx):
    _LSTM_DIMS.pop(ctx, None)
    load().dq_lstm_release(ctx)
