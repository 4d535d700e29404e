"""Pins of the oracle's fp16 QuantizeLinear / DequantizeLinear (R24).

onnxruntime quantization_defs.cc lets QuantizeLinear's x and y_scale, and
DequantizeLinear's x_scale and y, be float16. The oracle's binary16 decoder
and round-to-nearest-even encoder are pinned against numpy's float16 casts
(every one of the 65536 patterns, and fp32 values on ties, in the subnormal
range and at overflow); the operators against the fp32 oracle (already
pinned) on the exactly converted values, and by hand.
"""
import numpy as np
import pytest

import oracle


def test_decoder_every_pattern_matches_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    assert np.isnan(got[nan]).all()


def test_encoder_matches_numpy_on_ties_subnormals_and_overflow():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = h.view(np.float16).astype(np.float32)
    vals = vals[np.isfinite(vals)]
    nxt = np.nextafter(vals.astype(np.float16), np.float16(np.inf)).astype(np.float32)
    ok = np.isfinite(nxt)
    mids = ((vals[ok].astype(np.float64) + nxt[ok]) / 2).astype(np.float32)  # exact ties
    r = np.random.default_rng(0)
    rand = (r.standard_normal(200000) * 10.0 ** r.integers(-9, 6, 200000)).astype(np.float32)
    edge = np.float32([65504, 65519.996, 65520, 65536, 1e10, -1e10, 6e-8, 5.96e-8, 2.98e-8, 2.9802322e-8,
                       np.inf, -np.inf, 0.0, -0.0, 6.1035156e-05, 6.1032e-05])
    x = np.concatenate([vals, mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf)), rand, edge])
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f32_to_f16(x), ref)
    assert oracle.f32_to_f16(np.float32([np.nan]))[0] & 0x7e00 == 0x7e00


def test_encoder_hand_values():
    # 1 + 2^-11 is the tie between 1 and 1 + 2^-10 -> even (1.0, 0x3c00);
    # 1 + 3 * 2^-11 -> 1 + 2^-9 (0x3c02); 2^-25 is half the smallest
    # subnormal -> 0; 3 * 2^-25 -> 2 * 2^-24 (0x0002); 65520 -> inf
    x = np.float32([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 2.0 ** -25, 3 * 2.0 ** -25, 65520.0, -2.0])
    assert oracle.f32_to_f16(x).tolist() == [0x3c00, 0x3c02, 0x0000, 0x0002, 0x7c00, 0xc000]


@pytest.mark.parametrize("axis", [None, 1])
def test_quantize_f16_is_the_fp32_rule_on_exact_values(axis):
    r = np.random.default_rng(1)
    x = (r.standard_normal((4, 6, 9)) * 3).astype(np.float16)
    s = r.uniform(0.01, 0.05, 1 if axis is None else 6).astype(np.float16)
    z = r.integers(-10, 10, s.size).astype(np.int32)
    got = oracle.quantize_linear_f16(x.view(np.uint16), s.view(np.uint16), z, axis=axis, y_type="i8")
    want = oracle.quantize_linear(x.astype(np.float32), s.astype(np.float32), z, axis=axis, y_type="i8")
    assert np.array_equal(got, want)


def test_quantize_f16_hand_ties():
    # s = 0.5 (exact in fp16): x / s for x = 0.25, 0.75, 1.25, -0.25 is 0.5,
    # 1.5, 2.5, -0.5 -> 0, 2, 2, 0 (ties to even); 100 / 0.5 = 200 -> 127
    x = np.float16([0.25, 0.75, 1.25, -0.25, 100.0])
    got = oracle.quantize_linear_f16(x.view(np.uint16), np.float16([0.5]).view(np.uint16), [0])
    assert got.tolist() == [0, 2, 2, 0, 127]


def test_dequantize_f16_is_one_rounding_of_the_exact_product():
    # the exact product in float64, rounded once by numpy's float16 cast
    r = np.random.default_rng(2)
    q = r.integers(0, 256, (3, 5, 7)).astype(np.uint8)
    s = r.uniform(1e-4, 3.0, 5).astype(np.float16)
    z = r.integers(0, 256, 5).astype(np.int32)
    got = oracle.dequantize_linear_f16(q, s.view(np.uint16), z, axis=1, y_type="f16")
    exact = (q.astype(np.float64) - z[None, :, None]) * s.astype(np.float64)[None, :, None]
    assert np.array_equal(got, exact.astype(np.float16).view(np.uint16))
    got32 = oracle.dequantize_linear_f16(q, s.view(np.uint16), z, axis=1, y_type="f32")
    assert np.array_equal(got32, exact.astype(np.float32))
