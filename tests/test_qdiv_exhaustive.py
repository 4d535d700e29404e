"""Exhaustive CPU check of the quantizers' division (no GPU).

Every quantizer of the library (the rows of A, the columns of B,
QuantizeLinear, the requantizing epilogues) needs rne(x / s) of the IEEE fp32
quotient, as the ONNX Runtime QuantizeLinear schema defines it (round to
nearest, ties to even, then the zero point and saturation). The gfx950
kernels do not divide per element: they take y = RN(1/s) once per scale and
correct q0 = RN(x*y) with one residual step, q = fma(fma(-q0, s, x), y, q0)
(P. Markstein, "Computation of elementary functions on the IBM RISC
System/6000 processor", IBM J. Res. Develop. 34(1), 1990). Markstein's
theorem gives the correctly rounded quotient when y is the correctly rounded
reciprocal and q0 is within one ulp of x/s, with no underflow in the
residual; q0 = RN(x*y) is only guaranteed within 1.5 ulp, so the theorem
alone does not cover every x. This test closes the gap by brute force:
`qdiv_exhaustive.c` restates the kernels' three operation sequences in C and
runs each over all 2^32 fp32 bit patterns x (NaNs excluded) for a committed
set of scales, against the definition computed with IEEE `/`.

Scale classes: powers of two, all-ones significands (1 - 2^-24, near 2^-7,
just below 2^-99), scales of the workloads (0.005, 0.0371, the usage
example's row and column scales 0.15/255 and 2.4/63, 1e-30, the 1x1
QLinearConv output scale 0.02 and a draw from the per-channel output scales'
range U(0.005, 0.05)), the boundary 2^-100 of the fast path and 1.5 * 2^-100,
and scales that must take the IEEE division (just below 2^-100, a subnormal
3e-39, and 2^127 and FLT_MAX, whose reciprocals are subnormal). Expected: no code mismatch anywhere, and
for every fast scale the corrected quotient equals the IEEE quotient bit for
bit whenever |x/s| >= 1/4 (below that both round to 0).
"""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qdiv_exhaustive.c")


def _bits(f):
    return "%08x" % struct.unpack("<I", struct.pack("<f", float(np.float32(f))))[0]


SCALES = {
    "1": _bits(1.0),
    "2^-7": _bits(2.0 ** -7),
    "2^-100 (fast-path boundary)": _bits(2.0 ** -100),
    "1.5*2^-100": _bits(1.5 * 2.0 ** -100),
    "all-ones significand below 1": "3f7fffff",
    "all-ones significand near 2^-7": "3c7fffff",
    "all-ones significand below 2^-99": "0dffffff",
    "0.005": _bits(0.005),
    "0.0371": _bits(0.0371),
    "0.15/255 (the usage example's row scale)": _bits(np.float32(0.15) / np.float32(255)),
    "2.4/63 (the usage example's column scale)": _bits(np.float32(2.4) / np.float32(63)),
    "1e-30": _bits(1e-30),
    "0.02 (1x1 QLinearConv y_scale)": _bits(0.02),
    "a draw from U(0.005,0.05)": _bits(0.00859234),
    "just below 2^-100 (IEEE path)": "0d7fffff",
    "3e-39 subnormal (IEEE path)": _bits(3e-39),
    "2^127 (subnormal reciprocal, IEEE path)": _bits(2.0 ** 127),
    "FLT_MAX (IEEE path)": "7f7fffff",
}


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    assert gcc, "gcc is needed to build the exhaustive checker"
    exe = str(tmp_path_factory.mktemp("qdiv") / "qdiv_exhaustive")
    subprocess.run([gcc, "-O3", "-ffp-contract=off", "-mfma", "-mavx2", "-fopenmp", SRC, "-o", exe, "-lm"],
                   check=True)
    return exe


def test_corrected_quotient_gives_ieee_codes_for_every_x(checker):
    names = list(SCALES)
    r = subprocess.run([checker, *[SCALES[n] for n in names]], capture_output=True, text=True,
                       check=True, timeout=1200)
    lines = r.stdout.strip().splitlines()
    assert len(lines) == len(names), r.stdout + r.stderr
    bad = []
    for name, line in zip(names, lines):
        f = dict(kv.split("=") for kv in line.split())
        assert f["s"] == SCALES[name]
        assert int(f["n"]) == 2 ** 32 - 2 * (2 ** 23 - 1), line  # every non-NaN pattern
        print(f"{name:45s} {line}", flush=True)
        fast = f["fast"] == "1"
        want_fast = "IEEE path" not in name
        if fast != want_fast:
            bad.append(f"{name}: fast path {'taken' if fast else 'not taken'}")
        for key in ("qmis", "f1", "f2", "f3"):
            if int(f[key]) != 0:
                bad.append(f"{name}: {key}={f[key]}")
    assert not bad, bad


def test_checker_catches_a_plain_reciprocal_multiply(tmp_path):
    """The checker itself is not vacuous: rounding x * RN(1/s) without the
    residual step must produce code mismatches for an ordinary scale."""
    gcc = shutil.which("gcc")
    src = open(SRC).read().replace("const float res = fmaf(fmaf(-q0, s, x), y, q0);",
                                   "const float res = q0;")
    assert "const float res = q0;" in src
    p = tmp_path / "planted.c"
    p.write_text(src)
    exe = str(tmp_path / "planted")
    subprocess.run([gcc, "-O3", "-ffp-contract=off", "-mfma", "-mavx2", "-fopenmp", str(p), "-o", exe, "-lm"],
                   check=True)
    out = subprocess.run([exe, _bits(0.0371)], capture_output=True, text=True, check=True).stdout
    f = dict(kv.split("=") for kv in out.split())
    assert int(f["qmis"]) > 0 and int(f["f1"]) > 0 and int(f["f3"]) > 0, out
