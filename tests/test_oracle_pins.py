"""Pins of the CPU oracle to values fixed by the pages and by mathematics.

Every check here is independent of the oracle's own code: hand-derived values
(with the derivation beside them), values printed on the pages (golden files),
closed forms, invariants, brute force with Python integers on tiny inputs, and
the exact product within a derived error bound. A mistake such as a dropped
term, a flipped sign, a wrong index or a transposed operand in the oracle fails
at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32_MAX = np.float32(np.finfo(np.float32).max)


# ============================================================ QuantizeLinear
# onnxruntime quantization_defs.cc, QuantizeLinear doc: y = saturate(x/s + zp),
# x/s rounded to nearest with ties to even, saturating to [0,255] / [-128,127].

def test_quantize_linear_ties_to_even_hand_table():
    # s = 0.25 makes every x/s below exact, so each is a true half-way case.
    x = np.float32([0.125, 0.375, 0.625, -0.125, -0.375, -0.625, 0.875, -0.875])
    # x/s =          0.5    1.5    2.5    -0.5    -1.5    -2.5    3.5    -3.5
    want = np.int8([0, 2, 2, 0, -2, -2, 4, -4])
    assert np.array_equal(oracle.quantize_linear(x, 0.25, 0, y_type="i8"), want)
    # the zero point is added after rounding: zp = 3
    assert np.array_equal(oracle.quantize_linear(x, 0.25, 3, y_type="i8"), want + 3)
    # uint8 with zp 10
    assert np.array_equal(oracle.quantize_linear(x, 0.25, 10, y_type="u8"),
                          (want.astype(np.int32) + 10).astype(np.uint8))


def test_quantize_linear_saturation_hand_table():
    x = np.float32([127.5, 128.0, -128.5, -129.0, 1e6, -1e6, F32_MAX, -F32_MAX])
    # i8, s=1: 127.5 -> 128 -> 127; -128.5 -> -128 (even); huge -> bounds
    assert np.array_equal(oracle.quantize_linear(x, 1.0, 0, y_type="i8"),
                          np.int8([127, 127, -128, -128, 127, -128, 127, -128]))
    # FLT_MAX / 0.01 overflows to +inf, which saturates
    assert np.array_equal(oracle.quantize_linear(np.float32([F32_MAX, -F32_MAX]), 0.01, 0),
                          np.int8([127, -128]))
    # u8, s=1, zp=0: 255.5 -> 256 -> 255; -0.5 -> 0 (even) ; -1 -> 0
    xu = np.float32([255.5, 254.5, -0.5, -1.0, 0.5, 1.5])
    assert np.array_equal(oracle.quantize_linear(xu, 1.0, 0, y_type="u8"),
                          np.uint8([255, 254, 0, 0, 0, 2]))
    # saturation is applied after the zero point: i8, zp=-10, x/s = 120 -> 110;
    # x/s = -120 -> -130 -> -128
    assert np.array_equal(oracle.quantize_linear(np.float32([120, -120]), 1.0, -10),
                          np.int8([110, -128]))


def test_quantize_linear_per_axis_uses_the_axis_index():
    # x[n,c,h] = (c+1) * s_c exactly (s_c a power of two), so y = c+1+zp_c
    C = 5
    s = np.float32([0.5, 0.25, 0.125, 1.0, 2.0])
    zp = np.int32([0, 1, -1, 2, -2])
    x = np.empty((2, C, 3), np.float32)
    for c in range(C):
        x[:, c, :] = (c + 1) * s[c]
    y = oracle.quantize_linear(x, s, zp, axis=1)
    for c in range(C):
        assert np.all(y[:, c, :] == c + 1 + zp[c])
    # negative axis means the same axis
    assert np.array_equal(oracle.quantize_linear(x, s, zp, axis=-2), y)
    # the same tensor per tensor with s=0.125: values (c+1)*s_c/0.125
    yt = oracle.quantize_linear(x, 0.125, 0)
    assert np.array_equal(yt[0, :, 0], np.int8([4, 4, 3, 32, 80]))


def test_quantize_linear_reconstruction_bound_and_monotone():
    r = np.random.default_rng(11)
    s = np.float32(0.037)
    x = np.sort(r.uniform(-4.0, 4.0, 20000).astype(np.float32))
    y = oracle.quantize_linear(x, s, 3)
    # rounding to nearest: every in-range x is within half a step (plus the
    # one fp32 rounding of the quotient) of its reconstruction
    inr = (y > -128) & (y < 127)
    rec = (y[inr].astype(np.float64) - 3) * np.float64(s)
    assert np.all(np.abs(x[inr] - rec) <= 0.5 * s * (1 + 2 ** -20))
    # monotone non-decreasing in x
    assert np.all(np.diff(y.astype(np.int32)) >= 0)


def test_quantize_linear_numpy_cross_check():
    # a cross-check against numpy's half-to-even rint (a library routine of
    # its own) on the per-axis workload recipe, ties and saturation included
    case = W.qdq_per_axis(seed=1, shape=(2, 16, 9, 11), plant_every=37)
    x, s, zp = case["x"], case["scale"], case["zp"]
    y = oracle.quantize_linear(x, s, zp, axis=1)
    with np.errstate(over="ignore"):
        q = np.rint(x / s[None, :, None, None])
    want = np.clip(q.astype(np.float64) + zp[None, :, None, None], -128, 127).astype(np.int8)
    assert case["n_ties"] > 0
    assert np.array_equal(y, want)


# ========================================================== DequantizeLinear
# same page, DequantizeLinear doc: y = (x - x_zero_point) * x_scale

def test_dequantize_linear_is_the_exact_product_rounded_once():
    r = np.random.default_rng(12)
    for xt, lo, hi in (("i8", -128, 128), ("u8", 0, 256)):
        x = r.integers(lo, hi, (3, 7, 5)).astype(np.int8 if xt == "i8" else np.uint8)
        s = r.uniform(0.001, 3.0, 7).astype(np.float32)
        zp = r.integers(lo, hi, 7)
        y = oracle.dequantize_linear(x, s, zp, axis=1)
        # (x - zp) * s is exact in double (8-bit integer times 24-bit
        # significand), so rounding it once to fp32 is the correct result
        exact = (x.astype(np.float64) - zp[None, :, None]) * s[None, :, None].astype(np.float64)
        assert np.array_equal(y, exact.astype(np.float32))
    # hand values: x = zp -> 0, x = zp + 1 -> s
    assert np.array_equal(oracle.dequantize_linear(np.int8([5, 6, 4]), 0.75, 5),
                          np.float32([0.0, 0.75, -0.75]))


def test_quantize_of_dequantize_round_trips_every_code():
    r = np.random.default_rng(13)
    codes_i8 = np.arange(-128, 128).astype(np.int8)
    codes_u8 = np.arange(0, 256).astype(np.uint8)
    for _ in range(20):
        s = np.float32(r.uniform(1e-4, 10.0))
        zi = int(r.integers(-128, 128))
        zu = int(r.integers(0, 256))
        assert np.array_equal(
            oracle.quantize_linear(oracle.dequantize_linear(codes_i8, s, zi), s, zi), codes_i8)
        assert np.array_equal(
            oracle.quantize_linear(oracle.dequantize_linear(codes_u8, s, zu), s, zu,
                                   y_type="u8"), codes_u8)


# ==================================================== dynamic quantization of A
# Simd SynetDynamicQuantizedInnerProduct16b, Detailed Description: A -> uA
# (uint8), scaleA[i], zeroA[i]; the formula is the reading min/max with 0 in
# range, scale (hi-lo)/255, zero rne(-lo/scale), uA = sat(rne(A/s) + zero).

def test_row_quantization_hand_values_power_of_two_scale():
    # lo = -1, hi = 127/128: hi - lo = 255/128 exactly, scale = 1/128 exactly,
    # zero = rne(1 / (1/128)) = 128.  a/s for the row below:
    #   -128, 127, 64, 1.5, 2.5, -1.5, 0, -2.5
    row = np.float32([-1.0, 0.9921875, 0.5, 3 / 256, 5 / 256, -3 / 256, 0.0, -5 / 256])
    want = np.uint8([0, 255, 192, 130, 130, 126, 128, 126])
    for typeA, A in (("f32", row[None, :]), ("bf16", W.to_bf16_bits(row[None, :]))):
        uA, sA, zA = oracle.quantize_rows(A, typeA)
        assert sA[0] == np.float32(1 / 128) and zA[0] == 128
        assert np.array_equal(uA[0], want)


def test_row_quantization_ramp_row0_hand_values():
    # the usage example's A[i] = i*0.01f: row 0 is 0, 0.01, ..., 0.15, so
    # lo = 0, zero = 0, scale = 0.15/255 and A/scale = 17k up to a few ulp
    # (never near a tie), so uA = 17k
    uA, sA, zA = oracle.quantize_rows(W.dqip_ramp()["A"])
    assert zA[0] == 0
    assert np.array_equal(uA[0], (17 * np.arange(16)).astype(np.uint8))


def test_row_quantization_special_rows():
    A = np.zeros((4, 6), np.float32)
    A[1] = [0.5, 1.0, 2.0, 0.25, 0.0, 1.5]      # all >= 0: lo = 0 -> zero 0
    A[2] = [-0.5, -1.0, -2.0, -0.25, 0.0, -1.5]  # all <= 0: hi = 0 -> zero 255
    A[3] = [-2.0, -2.0, -2.0, 4.0, 4.0, 4.0]
    uA, sA, zA = oracle.quantize_rows(A)
    # all-zero row: scale 1, zero point 0, every code 0
    assert sA[0] == 1.0 and zA[0] == 0 and not uA[0].any()
    assert zA[1] == 0 and uA[1, 2] == 255 and uA[1, 4] == 0
    assert zA[2] == 255 and uA[2, 2] == 0 and uA[2, 4] == 255
    # lo = -2, hi = 4: scale = 6/255, zero = rne(2/(6/255)) = rne(85) = 85
    assert zA[3] == 85 and np.array_equal(uA[3], np.uint8([0, 0, 0, 255, 255, 255]))


@pytest.mark.parametrize("typeA", ["f32", "bf16"])
def test_row_quantization_invariants(typeA):
    case = W.dqip_random(37, 5, 301, seed=21, typeA=typeA, outliers=0.02, zero_rows=(3,))
    A = case["A"]
    Af = W.bf16_bits_to_f32(A) if typeA == "bf16" else A
    uA, sA, zA = oracle.quantize_rows(A, typeA)
    for i in range(A.shape[0]):
        a, u, s, z = Af[i], uA[i].astype(np.int64), np.float64(sA[i]), int(zA[i])
        if not a.any():
            continue
        lo, hi = min(a.min(), 0.0), max(a.max(), 0.0)
        # the extremes land on the ends of [0,255], within one code: when
        # -lo/s is an exact half, zero and hi/s both round to even
        assert u[np.argmax(a)] >= 254 or hi == 0
        assert u[np.argmin(a)] <= 1 or lo == 0
        # 0.0 maps exactly to the zero point
        zeros = a == 0
        assert np.all(u[zeros] == z)
        # round to nearest: reconstruction within half a step, plus the fp32
        # rounding of the quotient a/s (|a/s| <= 256, so <= 2^-15 steps)
        assert np.all(np.abs(a - s * (u - z)) <= 0.5 * s + s * 2 ** -15)
        # the step spans the range: 255 steps of s cover [lo, hi]
        assert abs(255 * s - (hi - lo)) <= 1e-6 * (hi - lo)
        # monotone in A
        order = np.argsort(a, kind="stable")
        assert np.all(np.diff(u[order]) >= 0)
    # a subset of rows gives the same rows
    rows = np.array([5, 0, 36, 3])
    uS, sS, zS = oracle.quantize_rows(A, typeA, rows=rows)
    assert np.array_equal(uS, uA[rows]) and np.array_equal(sS, sA[rows])


# ==================================================== dynamic quantization of B
# same page: B[k,j] -> iB (int8), scaleB[j]; avoidOverflow narrows to [-64,63]

def test_col_quantization_ramp_col0_hand_values():
    # B[i] = i*0.02f with N = 8: column 0 is B[8k] = 0.16k, k = 0..15; with
    # avoidOverflow qmax = 63, scale = 2.4/63, B/scale = 4.2k, never a tie:
    # rne(4.2k) = 0 4 8 13 17 21 25 29 34 38 42 46 50 55 59 63
    iB, sB = oracle.quantize_cols(W.dqip_ramp()["B"], avoid=True)
    want = [0, 4, 8, 13, 17, 21, 25, 29, 34, 38, 42, 46, 50, 55, 59, 63]
    assert np.array_equal(iB[:, 0], np.int8(want))
    assert iB.max() == 63 and iB.min() >= -64


def test_col_quantization_hand_values_power_of_two_scale():
    # column 0: amax = 127/64 -> scale 1/64; column 1: all zero -> scale 1;
    # column 2: amax = 127/64 * 2 -> scale 1/32
    B = np.zeros((6, 3), np.float32)
    B[:, 0] = [127 / 64, -127 / 64, 3 / 128, -5 / 128, 0.0, 1 / 64]
    B[:, 2] = 2 * B[:, 0]
    iB, sB = oracle.quantize_cols(B)
    # B/scale column 0: 127, -127, 1.5, -2.5, 0, 1 -> ties to even
    assert np.array_equal(iB[:, 0], np.int8([127, -127, 2, -2, 0, 1]))
    assert np.array_equal(iB[:, 2], iB[:, 0])
    assert np.array_equal(sB, np.float32([1 / 64, 1.0, 1 / 32]))
    assert not iB[:, 1].any()
    # avoidOverflow: amax = 63/64 -> scale 1/64
    B2 = np.float32([[63 / 64], [-63 / 64], [3 / 128], [-5 / 128]])
    iB2, sB2 = oracle.quantize_cols(B2, avoid=True)
    assert np.array_equal(iB2[:, 0], np.int8([63, -63, 2, -2])) and sB2[0] == np.float32(1 / 64)


@pytest.mark.parametrize("avoid", [False, True])
def test_col_quantization_invariants(avoid):
    r = np.random.default_rng(22)
    K, N = 53, 17
    # column j scaled by (j+1): catches a row/column mix-up in the reduction
    B = (r.normal(0, 0.05, (K, N)) * (np.arange(N) + 1)).astype(np.float32)
    B[:, 4] = 0.0
    iB, sB = oracle.quantize_cols(B, avoid=avoid)
    qmax = 63 if avoid else 127
    for j in range(N):
        b, q, s = B[:, j], iB[:, j].astype(np.int64), np.float64(sB[j])
        if not b.any():
            assert s == 1.0 and not q.any()
            continue
        assert np.abs(q).max() == qmax
        assert abs(s * qmax - np.abs(b).max()) <= 1e-6 * np.abs(b).max()
        assert np.all(np.abs(b - s * q) <= 0.5 * s + s * 2 ** -15)
    # scales grow with the column's multiplier
    nz = [j for j in range(N) if j != 4]
    ratio = sB[nz] / (np.arange(N)[nz] + 1)
    assert ratio.max() / ratio.min() < 3.0


def test_colsum_brute_force():
    r = np.random.default_rng(23)
    iB = r.integers(-128, 128, (9, 4)).astype(np.int8)
    got = oracle.colsum(iB)
    for j in range(4):
        assert got[j] == sum(int(iB[k, j]) for k in range(9))


# ================================================== integer inner product
# same page: sum over k of (uA[i,k] - zeroA[i]) * iB[k,j]

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 1), (3, 5, 7), (5, 2, 8), (4, 4, 13)])
def test_int_gemm_brute_force_python_ints(M, N, K):
    r = np.random.default_rng(M * 100 + N * 10 + K)
    uA = r.integers(0, 256, (M, K)).astype(np.uint8)
    zA = r.integers(0, 256, M).astype(np.int32)
    iB = r.integers(-128, 128, (K, N)).astype(np.int8)
    acc = oracle.int_gemm(uA, zA, iB)
    for i in range(M):
        for j in range(N):
            want = 0
            for k in range(K):
                want += (int(uA[i, k]) - int(zA[i])) * int(iB[k, j])
            assert acc[i, j] == want


def test_int_gemm_extreme_fits_int32():
    K = 65536
    uA = np.full((1, K), 255, np.uint8)
    iB = np.full((K, 1), -128, np.int8)
    acc = oracle.int_gemm(uA, np.int32([0]), iB)
    assert acc[0, 0] == 255 * -128 * K == -2139095040
    with pytest.raises(RuntimeError):
        oracle.int_gemm(np.full((1, K + 300), 255, np.uint8), np.int32([0]),
                        np.full((K + 300, 1), -128, np.int8))


def test_int_gemm_shifted_operand_identity():
    # sum (uA-128) iB + (128-zeroA) colsum(iB) = sum (uA-zeroA) iB (algebra)
    r = np.random.default_rng(24)
    uA = r.integers(0, 256, (6, 40)).astype(np.uint8)
    zA = r.integers(0, 256, 6).astype(np.int32)
    iB = r.integers(-128, 128, (40, 9)).astype(np.int8)
    shifted = (uA.astype(np.int64) - 128) @ iB.astype(np.int64)
    cs = oracle.colsum(iB).astype(np.int64)
    assert np.array_equal(oracle.int_gemm(uA, zA, iB),
                          shifted + (128 - zA.astype(np.int64))[:, None] * cs[None, :])


# ============================================================ whole forward

def _error_bound(case, o):
    """|C - (A B + bias)| <= sum_k (dA |B| + |A| dB + dA dB) + fp32 slack,
    with dA = scaleA/2, dB = scaleB/2 (round to nearest) -- derived from the
    quantizers, not stated on the pages."""
    A = case["A"]
    A = W.bf16_bits_to_f32(A) if case["typeA"] == "bf16" else A
    A = A.astype(np.float64)
    if case["typeB"] == "i8":
        Bf = case["B"].astype(np.float64) * case["scaleB"].astype(np.float64)[None, :]
        dB = np.zeros(case["N"])
    else:
        B = case["B"]
        Bf = (W.bf16_bits_to_f32(B) if case["typeB"] == "bf16" else B).astype(np.float64)
        dB = o["scaleB"].astype(np.float64) / 2
    dA = o["scaleA"].astype(np.float64) / 2
    exact = A @ Bf
    if case.get("bias") is not None:
        exact = exact + case["bias"].astype(np.float64)[None, :]
    K = case["K"]
    bound = (dA[:, None] * np.abs(Bf).sum(0)[None, :] + np.abs(A).sum(1)[:, None] * dB[None, :]
             + K * dA[:, None] * dB[None, :])
    slack = 4 * 2.0 ** -24 * (np.abs(exact) + bound) + 1e-30
    return exact, bound + slack


@pytest.mark.parametrize("maker", [
    W.dqip_ramp,
    W.dqip_small,
    lambda: W.dqip_random(7, 11, 29, seed=31),
    lambda: W.dqip_random(5, 3, 64, seed=32, typeA="bf16", typeB="bf16", avoid=True),
    lambda: W.dqip_random(9, 6, 33, seed=33, typeB="i8"),
])
def test_forward_within_quantization_error_bound(maker):
    case = maker()
    o = oracle.dqip_forward(case)
    exact, bound = _error_bound(case, o)
    assert np.all(np.abs(o["C"].astype(np.float64) - exact) <= bound)


def test_forward_ramp_error_is_close_to_its_bound():
    # the ramp's largest error is a sizeable fraction of its bound, so a
    # dropped term (bias, zero point, a scale) would exceed it
    case = W.dqip_ramp()
    o = oracle.dqip_forward(case)
    exact, bound = _error_bound(case, o)
    err = np.abs(o["C"] - exact)
    assert err.max() > 0.25 * bound.max()


def test_epilogue_is_fp32_rounding_of_the_exact_dequantization():
    # val = acc*sA*sB + bias with three fp32 roundings: within 2^-22 relative
    # of the exact value (plus one rounding of the bias sum)
    r = np.random.default_rng(25)
    acc = r.integers(-2 ** 24, 2 ** 24, (7, 9)).astype(np.int32)
    sA = r.uniform(1e-4, 1e-2, 7).astype(np.float32)
    sB = r.uniform(1e-4, 1e-2, 9).astype(np.float32)
    bias = r.uniform(-1, 1, 9).astype(np.float32)
    got = oracle.epilogue(acc, sA, sB, bias).astype(np.float64)
    prod = acc.astype(np.float64) * sA.astype(np.float64)[:, None] * sB.astype(np.float64)[None, :]
    exact = prod + bias.astype(np.float64)[None, :]
    assert np.all(np.abs(got - exact) <= 2.0 ** -22 * (np.abs(prod) + np.abs(exact)))
    # no bias flag: no add at all; bias flag with NULL bias: adds zeros
    nb = oracle.epilogue(acc, sA, sB, None, has_bias=False)
    zb = oracle.epilogue(acc, sA, sB, None, has_bias=True)
    assert np.array_equal(nb, zb)


def test_activations_and_bf16_output():
    import torch

    case = W.dqip_random(8, 12, 40, seed=26, typeB="i8")
    base = oracle.dqip_forward(case)["C"]
    relu = oracle.dqip_forward(dict(case, act="relu"))["C"]
    leaky = oracle.dqip_forward(dict(case, act="leaky_relu", alpha=0.25))["C"]
    assert (base < 0).any() and (base > 0).any()
    assert np.array_equal(relu, np.where(base > 0, base, np.float32(0)))
    # alpha = 0.25 is a power of two, so v * alpha is exact
    assert np.array_equal(leaky, np.where(base < 0, base * np.float32(0.25), base))
    bf = oracle.dqip_forward(dict(case, typeC="bf16"))["C"]
    want = torch.from_numpy(base).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf, want)


def test_bf16_helpers_match_torch():
    import torch

    r = np.random.default_rng(27)
    x = r.normal(0, 10, 4000).astype(np.float32)
    # plant exact half-way cases: low 16 bits 0x8000 with odd and even upper
    bits = x.view(np.uint32)
    bits[:200] = (bits[:200] & 0xFFFF0000) | 0x8000
    x = bits.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f32_to_bf16(x), want)
    back = torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(oracle.bf16_to_f32(want), back)


def test_forward_rows_subset_matches_full():
    case = W.dqip_random(21, 10, 50, seed=28, typeB="f32", avoid=True)
    full = oracle.dqip_forward(case)
    rows = np.array([20, 0, 7, 7])
    part = oracle.dqip_forward(case, rows=rows)
    for key in ("uA", "scaleA", "zeroA", "acc", "C"):
        assert np.array_equal(part[key], full[key][rows])
    assert np.array_equal(part["iB"], full["iB"])


def test_forward_int8_b_uses_given_codes_and_scales():
    case = W.dqip_random(4, 6, 10, seed=29, typeB="i8")
    o = oracle.dqip_forward(case)
    assert np.array_equal(o["iB"], case["B"]) and np.array_equal(o["scaleB"], case["scaleB"])


# =============================================================== QLinearConv
# ONNX QLinearConv (opset 10): printed examples

@pytest.mark.parametrize("fname", ["qlinearconv_u8.json", "qlinearconv_i8.json"])
def test_qlinear_conv_printed_examples(fname):
    with open(os.path.join(GOLDEN, fname)) as f:
        g = json.load(f)
    x = np.array(g["x"], dtype=g["x_dtype"]).reshape(g["x_shape"])
    w = np.array(g["w"], dtype=g["w_dtype"]).reshape(g["w_shape"])
    y = oracle.qlinear_conv(x, np.float32(g["x_scale"]), g["x_zero_point"], w,
                            np.array(g["w_scale"], np.float32), np.array(g["w_zero_point"]),
                            np.float32(g["y_scale"]), g["y_zero_point"],
                            y_type="u8" if g["y_dtype"] == "uint8" else "i8")
    assert np.array_equal(y, np.array(g["y"], dtype=g["y_dtype"]).reshape(g["y_shape"]))


def test_qlinear_conv_1x1_brute_force_and_exact_requantization():
    r = np.random.default_rng(30)
    Nb, Cc, M, H, Wd = 2, 64, 8, 6, 7
    x = r.integers(0, 256, (Nb, Cc, H, Wd)).astype(np.uint8)
    w = r.integers(-127, 128, (M, Cc)).astype(np.int8)
    ws = r.uniform(0.0005, 0.002, M).astype(np.float32)
    bias = r.integers(-10000, 10001, M).astype(np.int32)
    xs, ys, yz = np.float32(0.01), np.float32(0.004), 128
    y = oracle.qlinear_conv(x, xs, 128, w, ws, np.zeros(M, np.int32), ys, yz, bias=bias)
    # integer part by brute force with Python ints on a few outputs
    for (n, m, h, q) in [(0, 0, 0, 0), (1, 7, 5, 6), (0, 3, 2, 4), (1, 1, 0, 3)]:
        acc = sum(int(w[m, c]) * (int(x[n, c, h, q]) - 128) for c in range(Cc)) + int(bias[m])
        exact = acc * float(xs) * float(ws[m]) / float(ys)
        if abs(exact - np.floor(exact) - 0.5) > 1e-3:
            assert int(y[n, m, h, q]) == min(255, max(0, int(np.floor(exact + 0.5)) + yz))
    # every output: the exact rational acc*x_scale*w_scale/y_scale (float64)
    # rounded to nearest, except within 1e-5 of a half-way point where the
    # fp32 roundings of the pages' formula may decide either way
    acc = np.einsum("mc,nchw->nmhw", w.astype(np.int64), x.astype(np.int64) - 128)
    acc = acc + bias.astype(np.int64)[None, :, None, None]
    exact = acc * np.float64(xs) * ws.astype(np.float64)[None, :, None, None] / np.float64(ys)
    frac = np.abs(exact - np.floor(exact) - 0.5)
    want = np.clip(np.floor(exact + 0.5) + yz, 0, 255)
    sure = frac > 1e-5
    assert sure.mean() > 0.99 and (want[sure] == 255).any() and (want[sure] == 0).any()
    assert np.array_equal(y[sure].astype(np.float64), want[sure])


# ================================================== QGemm family (R15-R19)
# onnxruntime quantization_defs.cc, schemas QGemm, MatMulIntegerToFloat and
# DynamicQuantizeMatMul: inputs A, B with scales and zero points (B's per
# tensor or per column), QGemm's int32 C, alpha, transA / transB and the
# optional 8-bit output; the readings are R15-R19 in oracle.c.

def _q8(r, shape, u8):
    return (r.integers(0, 256, shape).astype(np.uint8) if u8
            else r.integers(-128, 128, shape).astype(np.int8))


def test_qgemm_unit_scales_zero_points_is_the_integer_matmul():
    # a_scale = b_scale = alpha = 1 and zero points 0: Y is A @ B (numpy's
    # int64 matmul; every |sum| < 2^24, so exact in fp32)
    r = np.random.default_rng(40)
    for ua, ub in ((True, False), (False, True), (True, True), (False, False)):
        A, B = _q8(r, (9, 31), ua), _q8(r, (31, 5), ub)
        Y = oracle.qgemm(A, B, 1.0, 0, 1.0)
        assert np.array_equal(Y, (A.astype(np.int64) @ B.astype(np.int64)).astype(np.float32))


def test_qgemm_zero_point_shift_invariance():
    # (A + t) - (a_zp + t) = A - a_zp: moving a code range and its zero point
    # together leaves every sum and output unchanged; likewise per column of B
    r = np.random.default_rng(41)
    A = r.integers(20, 200, (6, 40)).astype(np.uint8)
    B = r.integers(-100, 100, (40, 7)).astype(np.int8)
    bz = r.integers(-20, 21, 7).astype(np.int32)
    bs = r.uniform(0.01, 0.02, 7).astype(np.float32)
    Y0, acc0 = oracle.qgemm(A, B, 0.05, 17, bs, bz, with_acc=True)
    Y1, acc1 = oracle.qgemm((A + 33).astype(np.uint8), B, 0.05, 50, bs, bz, with_acc=True)
    assert np.array_equal(acc0, acc1) and np.array_equal(Y0, Y1)
    tcol = np.arange(7, dtype=np.int32) - 3
    B2 = (B.astype(np.int32) + tcol[None, :]).astype(np.int8)
    Y2, acc2 = oracle.qgemm(A, B2, 0.05, 17, bs, bz + tcol, with_acc=True)
    assert np.array_equal(acc0, acc2) and np.array_equal(Y0, Y2)
    # and a non-zero a_zp really enters: sum changes by -a_zp * column sums
    _, acc3 = oracle.qgemm(A, B, 0.05, 18, bs, bz, with_acc=True)
    colsum = (B.astype(np.int64) - bz[None, :]).sum(axis=0)
    assert np.array_equal(acc0.astype(np.int64) - acc3, np.broadcast_to(colsum, acc0.shape))


def test_qgemm_transposed_operands():
    r = np.random.default_rng(42)
    A, B = _q8(r, (5, 12), True), _q8(r, (12, 4), False)
    args = dict(a_scale=0.1, a_zp=9, b_scale=np.float32([0.2, 0.3, 0.4, 0.5]),
                b_zp=np.int32([1, -2, 3, 0]))
    Y = oracle.qgemm(A, B, **args)
    assert np.array_equal(oracle.qgemm(np.ascontiguousarray(A.T), B, transA=True, **args), Y)
    assert np.array_equal(oracle.qgemm(A, np.ascontiguousarray(B.T), transB=True, **args), Y)
    assert np.array_equal(oracle.qgemm(np.ascontiguousarray(A.T), np.ascontiguousarray(B.T),
                                       transA=True, transB=True, **args), Y)


def test_qgemm_brute_force_with_c_broadcasts_alpha_and_bias():
    # Python integers for the sums, numpy fp32 scalars in R17's order
    r = np.random.default_rng(43)
    M, N, K = 4, 5, 9
    A, B = _q8(r, (M, K), False), _q8(r, (K, N), True)
    a_scale, a_zp, alpha = np.float32(0.03), -5, np.float32(1.5)
    bs = r.uniform(0.01, 0.05, N).astype(np.float32)
    bz = r.integers(100, 156, N).astype(np.int32)
    bias = r.uniform(-1, 1, N).astype(np.float32)
    Cs = {"MN": r.integers(-500, 500, (M, N)), "N": r.integers(-500, 500, N),
          "1N": r.integers(-500, 500, (1, N)), "M1": r.integers(-500, 500, (M, 1)),
          "scalar": np.int64(321)}
    for name, Cm in Cs.items():
        Cb = np.broadcast_to(np.asarray(Cm, np.int64), (M, N))
        Y, acc = oracle.qgemm(A, B, a_scale, a_zp, bs, bz, C=np.asarray(Cm, np.int32),
                              alpha=alpha, bias=bias, with_acc=True)
        sa = np.float32(alpha * a_scale)
        for m in range(M):
            for n in range(N):
                s = sum((int(A[m, k]) - a_zp) * (int(B[k, n]) - int(bz[n])) for k in range(K))
                s += int(Cb[m, n])
                assert acc[m, n] == s, (name, m, n)
                v = np.float32(np.float32(np.float32(s) * sa) * bs[n]) + bias[n]
                assert Y[m, n] == np.float32(v), (name, m, n)


def test_qgemm_requantized_output_ties_and_saturation():
    # unit scales, y_scale 2: real / y_scale = sum / 2, a tie at every odd
    # sum; K = 1 with B = 1 makes the sums the codes of A themselves
    A = np.int8([[1], [3], [5], [-1], [-3], [100], [-128], [127]])
    B = np.int8([[1]])
    y = oracle.qgemm(A, B, 1.0, 0, 1.0, y_scale=2.0, y_zp=10, y_type="i8")
    # sum/2 =      0.5  1.5  2.5  -0.5  -1.5  50   -64  63.5
    want = np.int8([0, 2, 2, 0, -2, 50, -64, 64]) + 10
    assert np.array_equal(y.ravel(), want.astype(np.int32).clip(-128, 127).astype(np.int8))
    # saturation at both ends of uint8
    y = oracle.qgemm(A, B, 1.0, 0, 1.0, y_scale=0.25, y_zp=128, y_type="u8")
    assert y.ravel()[5] == 255 and y.ravel()[6] == 0


def test_dynamic_quantize_matmul_per_tensor_hand_values():
    # lo = -1, hi = 127/128: scale = (255/128)/255 = 1/128 exactly and
    # zp = rne(128) = 128; q(x) = rne(128 x) + 128
    A = np.float32([[-1.0, 127 / 128], [0.5, 3 / 256], [5 / 256, 0.0]])
    sc, zp, q = oracle.quantize_tensor_u8(A)
    assert sc == np.float32(1 / 128) and zp == 128
    #                     -128+128  127+128  64+128  rne(1.5)=2  rne(2.5)=2  0+128
    assert np.array_equal(q, np.uint8([[0, 255], [192, 130], [130, 128]]))
    # all zeros: scale 1, zero point 0, codes 0 (R4 over the tensor)
    sc, zp, q = oracle.quantize_tensor_u8(np.zeros((2, 3), np.float32))
    assert sc == 1.0 and zp == 0 and not q.any()
    # the composition: DynamicQuantizeMatMul = MatMulIntegerToFloat of the
    # quantized tensor with its scale and zero point
    r = np.random.default_rng(44)
    A = r.normal(0, 1, (7, 33)).astype(np.float32)
    B = _q8(r, (33, 6), False)
    bs = r.uniform(0.01, 0.05, 6).astype(np.float32)
    bias = r.uniform(-1, 1, 6).astype(np.float32)
    sc, zp, q = oracle.quantize_tensor_u8(A)
    assert q.max() == 255 or q.min() == 0
    assert np.array_equal(oracle.dynamic_quantize_matmul(A, B, bs, bias=bias),
                          oracle.matmul_integer_to_float(q, B, sc, bs, a_zp=zp, bias=bias))
    # and it approximates the float product within the quantization error
    exact = A.astype(np.float64) @ (B.astype(np.float64) * bs[None, :]) + bias
    bound = 0.5 * float(sc) * np.abs(B.astype(np.float64) * bs[None, :]).sum(axis=0)
    Y = oracle.dynamic_quantize_matmul(A, B, bs, bias=bias)
    assert (np.abs(Y - exact) <= bound[None, :] * 1.001 + 1e-5).all()


# ------------------------------------------------ N-dimensional products (R29)
# MatMulIntegerToFloat / DynamicQuantizeMatMul take N-dimensional A and B and
# infer Y's shape as ONNX MatMul does, which follows numpy.matmul: numpy's own
# matmul fixes the shapes and the batch pairing here.

ND_SHAPES = [
    ((2, 3, 5, 7), (7, 4)),        # B 2-D: every A batch against the one B
    ((2, 1, 5, 7), (3, 7, 4)),     # both broadcast: Y batches (2, 3)
    ((5, 7), (2, 3, 7, 4)),        # A 2-D against B batches
    ((4, 5, 7), (4, 7, 3)),        # equal batches
    ((1, 5, 7), (4, 7, 3)),        # A batch of one, broadcast
    ((3, 1, 2, 5, 7), (2, 1, 7, 4)),
    ((7,), (2, 7, 4)),             # 1-D A: one row, dropped from Y
    ((2, 5, 7), (7,)),             # 1-D B: one column, dropped from Y
    ((7,), (7,)),                  # dot product: Y is a scalar
]


@pytest.mark.parametrize("sa,sb", ND_SHAPES)
def test_matmul_nd_shapes_and_pairing_are_numpy_matmul(sa, sb):
    M, N, K, yb, out, pairs = oracle.matmul_batches(sa, sb)
    assert out == np.matmul(np.zeros(sa), np.zeros(sb)).shape
    assert len(pairs) == int(np.prod(yb, dtype=np.int64))
    # unit scales and zero points 0: Y is numpy's integer matmul exactly
    # (every |sum| < 2^24)
    r = np.random.default_rng(sum(sa) * 13 + sum(sb))
    A, B = _q8(r, sa, True), _q8(r, sb, False)
    Y = oracle.matmul_integer_to_float_nd(A, B, 1.0, 1.0)
    want = np.matmul(A.astype(np.int64), B.astype(np.int64)).astype(np.float32)
    assert Y.shape == want.shape and np.array_equal(Y, want)


def test_matmul_nd_rejects_what_numpy_rejects():
    for sa, sb in (((2, 5, 7), (3, 7, 4)), ((5, 7), (6, 4)), ((2, 3, 5, 7), (4, 7, 2))):
        with pytest.raises(ValueError):
            np.matmul(np.zeros(sa), np.zeros(sb))
        with pytest.raises(ValueError):
            oracle.matmul_batches(sa, sb)


def test_matmul_integer_to_float_nd_zero_points_scales_and_bias():
    # sums from numpy's int64 matmul of the shifted codes; the fp32 steps in
    # R17's order, vectorized in numpy: ((float)sum * a_scale) * b_scale[n]
    # + bias[n], each product and the sum rounded to fp32 once
    r = np.random.default_rng(45)
    A = _q8(r, (2, 1, 6, 37), True)
    B = _q8(r, (3, 37, 5), False)
    a_scale, a_zp = np.float32(0.021), 131
    bs = r.uniform(0.01, 0.05, 5).astype(np.float32)
    bz = r.integers(-9, 10, 5).astype(np.int32)
    bias = r.uniform(-1, 1, 5).astype(np.float32)
    Y = oracle.matmul_integer_to_float_nd(A, B, a_scale, bs, a_zp, bz, bias)
    s = np.matmul(A.astype(np.int64) - a_zp, B.astype(np.int64) - bz.astype(np.int64))
    want = (s.astype(np.float32) * a_scale).astype(np.float32) * bs
    want = (want.astype(np.float32) + bias).astype(np.float32)
    assert Y.shape == (2, 3, 6, 5) and np.array_equal(Y, want)


def test_dynamic_quantize_matmul_nd_quantizes_the_whole_tensor():
    # the batches span different ranges, so one scale for the whole tensor
    # (R19) differs from a scale per batch; the result is MatMulIntegerToFloat
    # on the codes of the whole tensor, within the quantization error of the
    # float product
    r = np.random.default_rng(46)
    A = np.stack([r.normal(0, 1, (5, 33)), 4 * r.normal(0, 1, (5, 33))]).astype(np.float32)
    B = _q8(r, (2, 33, 6), False)
    bs = r.uniform(0.01, 0.05, 6).astype(np.float32)
    bias = r.uniform(-1, 1, 6).astype(np.float32)
    Y = oracle.dynamic_quantize_matmul_nd(A, B, bs, bias=bias)
    lo, hi = min(0.0, float(A.min())), max(0.0, float(A.max()))
    sc = np.float32(np.float32(hi) - np.float32(lo)) / np.float32(255)
    tsc, zp, q = oracle.quantize_tensor_u8(A)
    assert tsc == np.float32(sc)
    assert np.array_equal(Y, oracle.matmul_integer_to_float_nd(q, B, tsc, bs, zp, bias=bias))
    per_batch = oracle.dynamic_quantize_matmul(A[0], B[0], bs, bias=bias)
    assert not np.array_equal(Y[0], per_batch)
    exact = np.matmul(A.astype(np.float64), B.astype(np.float64) * bs) + bias
    bound = 0.5 * float(sc) * np.abs(B.astype(np.float64) * bs).sum(axis=1, keepdims=True)
    assert (np.abs(Y - exact) <= bound * 1.001 + 1e-5).all()
