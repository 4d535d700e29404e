"""Pins of the oracle's element-wise quantized operators.

onnxruntime quantization_defs.cc (the contrib schemas of QLinearAdd,
QLinearMul, MulInteger, QLinearLeakyRelu, QLinearSigmoid, ReduceSumInteger,
QLinearReduceMean and QLinearConcat) prints each operator's formula. Every
check here is independent of the oracle's code: hand-derived tables (the
derivation beside each row), numpy's own broadcasting, sums and
concatenation, scipy's logistic function, and closed forms in exact rational
arithmetic where power-of-two scales make every fp32 step exact.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rne(fr: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def _sat(v, t):
    return max(0, min(255, v)) if t == np.uint8 else max(-128, min(127, v))


# ============================================================ broadcasting

SHAPE_PAIRS = [((3, 4), (4,)), ((3, 1), (1, 4)), ((2, 3, 4), (3, 1)), ((1,), (5, 2)),
               ((2, 1, 3), (4, 1)), ((6,), (6,)), ((), (2, 3)), ((1, 1, 1), (7,)),
               ((2, 3, 1, 5), (3, 4, 1)), ((4, 1, 1), (1, 3, 2))]


@pytest.mark.parametrize("sa,sb", SHAPE_PAIRS)
def test_broadcast_shape_matches_numpy(sa, sb):
    assert oracle.broadcast_shape(sa, sb) == np.broadcast_shapes(sa, sb)
    assert oracle.broadcast_shape(sb, sa) == np.broadcast_shapes(sb, sa)


@pytest.mark.parametrize("sa,sb", [((3,), (4,)), ((2, 3), (3, 2)), ((5, 4), (2, 1, 3))])
def test_broadcast_shape_rejects_what_numpy_rejects(sa, sb):
    with pytest.raises(ValueError):
        np.broadcast_shapes(sa, sb)
    with pytest.raises(ValueError):
        oracle.broadcast_shape(sa, sb)


# ============================================================== MulInteger
# C (int32) = (A - A_zp) * (B - B_zp), numpy-style broadcasting.

@pytest.mark.parametrize("sa,sb", SHAPE_PAIRS)
@pytest.mark.parametrize("dt", [np.uint8, np.int8])
def test_mul_integer_is_numpys_broadcast_product(sa, sb, dt):
    r = np.random.default_rng(hash((sa, sb)) & 0xFFFF)
    lo, hi = (0, 256) if dt == np.uint8 else (-128, 128)
    A = r.integers(lo, hi, sa).astype(dt)
    B = r.integers(lo, hi, sb).astype(dt)
    za, zb = int(r.integers(lo, hi)), int(r.integers(lo, hi))
    Y = oracle.mul_integer(A, za, B, zb)
    ref = (A.astype(np.int64) - za) * (B.astype(np.int64) - zb)
    assert Y.dtype == np.int32 and Y.shape == ref.shape
    assert np.array_equal(Y, ref)


def test_mul_integer_extremes():
    # the largest magnitude: (0 - 255) * (255 - 0) = -65025, (-128-127)^2
    assert oracle.mul_integer(np.uint8([0]), 255, np.uint8([255]), 0)[0] == -65025
    assert oracle.mul_integer(np.int8([-128]), 127, np.int8([-128]), 127)[0] == 65025


# ============================================================== QLinearAdd
# C = (A_scale*(A-A_zp) + B_scale*(B-B_zp)) / C_scale + C_zp, rounded half to
# even and saturated like QuantizeLinear.

def test_qlinear_add_hand_table_u8():
    # a_scale 0.5, a_zp 10, b_scale 0.25, b_zp 20, c_scale 1, c_zp 5
    rows = [  # A,   B,  real sum,            C
        (11, 22, 6),    # 0.5 + 0.5 = 1.0      -> 1 + 5
        (11, 21, 6),    # 0.5 + 0.25 = 0.75    -> 1 + 5
        (10, 22, 5),    # 0 + 0.5 = 0.5 tie    -> 0 + 5
        (13, 20, 7),    # 1.5 tie              -> 2 + 5
        (15, 20, 7),    # 2.5 tie              -> 2 + 5
        (9, 20, 5),     # -0.5 tie             -> 0 + 5
        (7, 20, 3),     # -1.5 tie             -> -2 + 5
        (0, 0, 0),      # -5 - 5 = -10         -> -5, saturated to 0
        (255, 255, 186),  # 122.5 + 58.75 = 181.25 -> 181 + 5
    ]
    A = np.uint8([r[0] for r in rows])
    B = np.uint8([r[1] for r in rows])
    C = oracle.qlinear_add(A, 0.5, 10, B, 0.25, 20, 1.0, 5)
    assert C.tolist() == [r[2] for r in rows]


def test_qlinear_add_unit_scales_is_the_saturating_integer_add():
    # all scales 1: C = sat((A - a_zp) + (B - b_zp) + c_zp), every step exact
    r = np.random.default_rng(60)
    for dt, lo, hi in ((np.uint8, 0, 256), (np.int8, -128, 128)):
        A = r.integers(lo, hi, (5, 17)).astype(dt)
        B = r.integers(lo, hi, (17,)).astype(dt)
        za, zb, zc = (int(v) for v in r.integers(lo, hi, 3))
        C = oracle.qlinear_add(A, 1.0, za, B, 1.0, zb, 1.0, zc)
        ref = (A.astype(np.int64) - za) + (B.astype(np.int64) - zb) + zc
        ref = np.clip(ref, lo, hi - 1)
        assert np.array_equal(C, ref.astype(dt))


def _exact_binary(op, A, sa, za, B, sb, zb, sc, zc, dt):
    """Closed form in rationals; exact when the scales are powers of two."""
    Ab, Bb = np.broadcast_arrays(A.astype(np.int64), B.astype(np.int64))
    out = np.empty(Ab.shape, np.int64)
    fa, fb, fc = Fraction(float(sa)), Fraction(float(sb)), Fraction(float(sc))
    for idx in np.ndindex(Ab.shape):
        a, b = int(Ab[idx]) - za, int(Bb[idx]) - zb
        v = fa * a + fb * b if op == "add" else Fraction(a * b) * fa * fb
        out[idx] = _sat(_rne(v / fc) + zc, dt)
    return out.astype(dt)


@pytest.mark.parametrize("op", ["add", "mul"])
@pytest.mark.parametrize("dt", [np.uint8, np.int8])
def test_qlinear_binary_power_of_two_scales_closed_form(op, dt):
    r = np.random.default_rng(61)
    lo, hi = (0, 256) if dt == np.uint8 else (-128, 128)
    fn = oracle.qlinear_add if op == "add" else oracle.qlinear_mul
    for sa_, sb_ in (((3, 1, 4), (5, 1)), ((6,), (2, 6)), ((2, 3), (2, 3))):
        A = r.integers(lo, hi, sa_).astype(dt)
        B = r.integers(lo, hi, sb_).astype(dt)
        sa, sb, sc = (float(2.0 ** int(e)) for e in r.integers(-6, 3, 3))
        if op == "mul":
            sc = float(2.0 ** int(r.integers(2, 9)))
        za, zb, zc = (int(v) for v in r.integers(lo, hi, 3))
        C = fn(A, sa, za, B, sb, zb, sc, zc)
        assert np.array_equal(C, _exact_binary(op, A, sa, za, B, sb, zb, sc, zc, dt))


@pytest.mark.parametrize("op", ["add", "mul"])
def test_qlinear_binary_general_scales_within_half_a_code(op):
    # generic fp32 scales: each fp32 rounding is relative 2^-24, so away from
    # saturation the code is within 0.5 (+ a few ulps) of the exact quotient
    r = np.random.default_rng(62)
    A = r.integers(0, 256, (40, 33)).astype(np.uint8)
    B = r.integers(0, 256, (33,)).astype(np.uint8)
    sa, sb = np.float32(r.uniform(0.01, 0.05)), np.float32(r.uniform(0.01, 0.05))
    sc = np.float32(r.uniform(0.02, 0.1)) if op == "add" else np.float32(r.uniform(5, 9))
    za, zb, zc = 120, 131, 128
    fn = oracle.qlinear_add if op == "add" else oracle.qlinear_mul
    C = fn(A, sa, za, B, sb, zb, sc, zc).astype(np.float64)
    a = A.astype(np.float64) - za
    b = B.astype(np.float64) - zb
    v = (a * float(sa) + b * float(sb)) if op == "add" else (a * b) * float(sa) * float(sb)
    q = v / float(sc) + zc
    inside = (q > 0.5) & (q < 254.5)
    assert inside.mean() > 0.5
    assert np.all(np.abs(C - q)[inside] <= 0.5 + 1e-4)
    assert np.all(C[q <= -0.5] == 0) and np.all(C[q >= 255.5] == 255)


@pytest.mark.parametrize("op", ["add", "mul"])
def test_qlinear_binary_swaps_operands(op):
    # both formulas are symmetric in (A, a_scale, a_zp) <-> (B, b_scale, b_zp)
    r = np.random.default_rng(63)
    A = r.integers(-128, 128, (4, 1, 6)).astype(np.int8)
    B = r.integers(-128, 128, (5, 1)).astype(np.int8)
    fn = oracle.qlinear_add if op == "add" else oracle.qlinear_mul
    args = (np.float32(0.037), 3, np.float32(0.011), -7, np.float32(0.05 if op == "add" else 0.3), 2)
    C1 = fn(A, args[0], args[1], B, args[2], args[3], args[4], args[5])
    C2 = fn(B, args[2], args[3], A, args[0], args[1], args[4], args[5])
    assert C1.shape == (4, 5, 6) and np.array_equal(C1, C2)


def test_qlinear_mul_hand_table_i8():
    # a_scale 0.5, a_zp 1, b_scale 0.5, b_zp -1, c_scale 0.5, c_zp 0
    rows = [  # A,    B,    (A-1)*(B+1) * 0.25 / 0.5           C
        (3, 1, 2),         # 4 * 0.25 = 1.0 / 0.5 = 2
        (2, 0, 0),         # 1 -> 0.5 tie -> 0
        (4, 0, 2),         # 3 -> 1.5 tie -> 2
        (6, 0, 2),         # 5 -> 2.5 tie -> 2
        (0, 2, -2),        # -3 -> -1.5 tie -> -2
        (1, 5, 0),         # 0
        (-128, -128, 127),  # 16383 -> 8191.5 -> saturated 127
        (127, -128, -128),  # 126 * -127 -> saturated -128
    ]
    A = np.int8([r[0] for r in rows])
    B = np.int8([r[1] for r in rows])
    C = oracle.qlinear_mul(A, 0.5, 1, B, 0.5, -1, 0.5, 0)
    assert C.tolist() == [r[2] for r in rows]


# ===================================================== QLinearLeakyRelu
# f(x) = quantize(alpha * dequantize(x)) where dequantize(x) < 0, else
# quantize(dequantize(x)); alpha defaults to 0.01.

def test_leaky_relu_hand_table():
    # x_scale 1, x_zp 0, y_scale 1, y_zp 0, alpha 0.25
    X = np.int8([-2, -6, -10, -14, -4, 0, 3, 127, -128])
    # alpha*x: -0.5 -1.5 -2.5 -3.5  -1   0  3  127   -32
    want = [0, -2, -2, -4, -1, 0, 3, 127, -32]
    assert oracle.qlinear_leaky_relu(X, 1.0, 0, 1.0, 0, alpha=0.25).tolist() == want


def test_leaky_relu_zero_point_decides_the_branch():
    # u8 with x_zp 100: codes below 100 are negative reals; x_scale 0.5,
    # y_scale 0.25, y_zp 50, alpha 0.5
    X = np.uint8([99, 98, 100, 101, 0, 255])
    # real:  -0.5  -1  0  0.5  -50  77.5
    # out:   -0.25/0.25=-1 -> 49; -0.5->-2 -> 48; 0 -> 50; 2 -> 52;
    #        -25/0.25 = -100 -> -50 -> sat 0; 310 -> 360 -> sat 255
    assert oracle.qlinear_leaky_relu(X, 0.5, 100, 0.25, 50, alpha=0.5).tolist() == \
        [49, 48, 50, 52, 0, 255]


def test_leaky_relu_alpha_one_same_params_is_identity():
    X = np.arange(-128, 128).astype(np.int8)
    Y = oracle.qlinear_leaky_relu(X, np.float32(0.0371), -5, np.float32(0.0371), -5, alpha=1.0)
    assert np.array_equal(X, Y)


def test_leaky_relu_default_alpha_is_one_percent():
    X = np.int8([-100, -50, 100])
    # -100 * 0.01 = -1 -> -1 ; -0.5 -> tie -> 0 ; 100
    assert oracle.qlinear_leaky_relu(X, 1.0, 0, 1.0, 0).tolist() == [-1, 0, 100]


# ======================================================= QLinearSigmoid
# f(x) = quantize(1 / (1 + exp(-dequantize(x)))).

@pytest.mark.parametrize("dt,x_scale,x_zp,y_scale,y_zp", [
    (np.int8, 0.0625, 0, 1 / 256, -128),
    (np.uint8, 0.05, 128, 1 / 256, 0),
    (np.int8, 0.125, -20, 1 / 255, -128),
    (np.uint8, 0.02, 0, 1 / 250, 3),
])
def test_sigmoid_matches_scipy_expit_every_code(dt, x_scale, x_zp, y_scale, y_zp):
    from scipy.special import expit
    lo, hi = (0, 256) if dt == np.uint8 else (-128, 128)
    X = np.arange(lo, hi).astype(dt)
    x = (X.astype(np.float32) - np.float32(x_zp)) * np.float32(x_scale)
    s = expit(x.astype(np.float64)).astype(np.float32)
    q = np.rint(s / np.float32(y_scale)).astype(np.int64) + y_zp
    want = np.clip(q, lo, hi - 1).astype(dt)
    got = oracle.qlinear_sigmoid(X, x_scale, x_zp, y_scale, y_zp)
    assert np.array_equal(got, want)


def test_sigmoid_odd_symmetry_and_hand_values():
    # with y_scale 1/256, y_zp -128: q(-x) = -q(x) away from the top code,
    # since sigmoid(-x) = 1 - sigmoid(x)
    X = np.arange(-127, 128).astype(np.int8)
    Y = oracle.qlinear_sigmoid(X, 0.05, 0, 1 / 256, -128).astype(np.int64)
    pos = Y[127:]           # x = 0 .. 127
    neg = Y[127::-1]        # x = 0 .. -127
    ok = pos < 127
    assert np.array_equal(neg[ok], -pos[ok])
    # sigmoid(0) = 0.5 -> 128 - 128 = 0; sigmoid(1) = 0.731058... -> 187.15
    # -> 59; sigmoid(2) = 0.880797... -> 225.48 -> 97; sigmoid(-5) =
    # 0.0066929 -> 1.713 -> 2 - 128 = -126
    Z = oracle.qlinear_sigmoid(np.int8([0, 1, 2, -5]), 1.0, 0, 1 / 256, -128)
    assert Z.tolist() == [0, 59, 97, -126]


# ========================================================= ReduceSumInteger

REDUCE_CASES = [((3, 4, 5), [1]), ((3, 4, 5), [0, 2]), ((3, 4, 5), None), ((3, 4, 5), [-1]),
                ((2, 3, 4, 5), [1, 2]), ((2, 3, 4, 5), [0, 3]), ((7,), [0]), ((6, 1, 4), [1]),
                ((2, 3, 4, 5), [3, 1])]


@pytest.mark.parametrize("shape,axes", REDUCE_CASES)
@pytest.mark.parametrize("keepdims", [True, False])
@pytest.mark.parametrize("dt", [np.uint8, np.int8])
def test_reduce_sum_integer_is_numpys_sum(shape, axes, keepdims, dt):
    r = np.random.default_rng(70)
    lo, hi = (0, 256) if dt == np.uint8 else (-128, 128)
    X = r.integers(lo, hi, shape).astype(dt)
    Y = oracle.reduce_sum_integer(X, axes, keepdims)
    ax = None if axes is None else tuple(axes)
    ref = X.astype(np.int64).sum(axis=ax, keepdims=keepdims)
    assert Y.dtype == (np.uint32 if dt == np.uint8 else np.int32)
    assert Y.shape == np.shape(ref) and np.array_equal(Y.astype(np.int64), ref)


# ======================================================== QLinearReduceMean
# Output = Quantize(ReduceMean(Dequantize(X))), per-tensor scales.

def test_reduce_mean_hand_table():
    X = np.uint8([[1, 2], [3, 4]])
    # rows: 1.5 -> 2, 3.5 -> 4; columns: 2, 3; all: 2.5 -> 2 (ties to even)
    assert oracle.qlinear_reduce_mean(X, 1.0, 0, 1.0, 0, [1]).tolist() == [[2], [4]]
    assert oracle.qlinear_reduce_mean(X, 1.0, 0, 1.0, 0, [0], False).tolist() == [2, 3]
    assert oracle.qlinear_reduce_mean(X, 1.0, 0, 1.0, 0).tolist() == [[2]]
    # zero points: x_zp 2 -> rows -0.5, 1.5; y_scale 0.5, y_zp 10:
    # -1 -> 9; 3 -> 13
    assert oracle.qlinear_reduce_mean(X, 1.0, 2, 0.5, 10, [1], False).tolist() == [9, 13]


@pytest.mark.parametrize("shape,axes", REDUCE_CASES)
@pytest.mark.parametrize("dt", [np.uint8, np.int8])
def test_reduce_mean_power_of_two_scales_closed_form(shape, axes, dt):
    # with power-of-two scales, the quotient S*xs/count/ys is within one fp32
    # rounding of the rational S/count * xs/ys, and S/count (count < 2^10) is
    # never that close to a half-way point unless it is one
    r = np.random.default_rng(71)
    lo, hi = (0, 256) if dt == np.uint8 else (-128, 128)
    X = r.integers(lo, hi, shape).astype(dt)
    xs, ys = 2.0 ** -3, 2.0 ** -1
    xz, yz = int(r.integers(lo, hi)), int(r.integers(lo, hi))
    Y = oracle.qlinear_reduce_mean(X, xs, xz, ys, yz, axes, True)
    ax = tuple(range(X.ndim)) if axes is None else tuple(a % X.ndim for a in axes)
    S = X.astype(np.int64).sum(axis=ax, keepdims=True)
    count = int(np.prod([shape[a] for a in ax]))
    want = np.empty(S.shape, np.int64)
    for idx in np.ndindex(S.shape):
        m = Fraction(int(S[idx]) - xz * count, count) * Fraction(xs) / Fraction(ys)
        want[idx] = _sat(_rne(m) + yz, dt)
    assert np.array_equal(Y.astype(np.int64), want)


def test_reduce_mean_equals_numpy_mean_then_quantize_generic_scales():
    # float64 numpy mean of the dequantized values, quantized: equal away
    # from half-way points (none of these quotients is within 1e-3 of one)
    r = np.random.default_rng(72)
    X = r.integers(0, 256, (16, 49)).astype(np.uint8)
    xs, ys = np.float32(0.0213), np.float32(0.0071)
    deq = (X.astype(np.float64) - 121) * float(xs)
    q = deq.mean(axis=1) / float(ys) + 119
    assert np.all(np.abs(q - np.floor(q) - 0.5) > 1e-3)
    want = np.clip(np.rint(q), 0, 255).astype(np.uint8)
    got = oracle.qlinear_reduce_mean(X, xs, 121, ys, 119, [1], False)
    assert np.array_equal(got, want)


# =========================================================== QLinearConcat
# Concatenate along axis; each input is requantized into Y's scale / zp.

@pytest.mark.parametrize("axis", [0, 1, 2, -1])
def test_concat_same_params_is_numpys_concatenate(axis):
    r = np.random.default_rng(80)
    base = [3, 4, 5]
    xs = []
    for n in (2, 1, 3):
        s = list(base)
        s[axis] = n
        xs.append(r.integers(-128, 128, s).astype(np.int8))
    Y = oracle.qlinear_concat([(x, np.float32(0.013), -4) for x in xs], np.float32(0.013), -4, axis)
    assert np.array_equal(Y, np.concatenate(xs, axis=axis))


def test_concat_requantizes_each_input_hand_table():
    a = np.uint8([[10, 11, 12]])
    b = np.uint8([[0, 1], [255, 128]]).reshape(1, 4)
    # a: scale 0.5, zp 10 -> reals 0, 0.5, 1 ; Y scale 1, zp 100 -> 100, 100
    #    (0.5 ties to 0), 101
    # b: scale 2, zp 128 -> reals -256, -254, 254, 0 -> -156 sat 0, -154 sat 0,
    #    354 sat 255, 100
    Y = oracle.qlinear_concat([(a, 0.5, 10), (b, 2.0, 128)], 1.0, 100, 1)
    assert Y.tolist() == [[100, 100, 101, 0, 0, 255, 100]]


def test_concat_power_of_two_closed_form():
    r = np.random.default_rng(81)
    ins = []
    for n in (5, 3, 8):
        x = r.integers(0, 256, (2, n, 6)).astype(np.uint8)
        ins.append((x, float(2.0 ** int(r.integers(-4, 2))), int(r.integers(0, 256))))
    ys, yz = 2.0 ** -2, 77
    Y = oracle.qlinear_concat(ins, ys, yz, 1)
    parts = []
    for x, s, z in ins:
        q = np.vectorize(lambda v: _sat(_rne(Fraction(int(v) - z) * Fraction(s) / Fraction(ys)) + yz,
                                        np.uint8))(x)
        parts.append(q)
    assert np.array_equal(Y, np.concatenate(parts, axis=1).astype(np.uint8))
