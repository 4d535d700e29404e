"""GPU parity of the quantized matrix products (QGemm, MatMulIntegerToFloat,
DynamicQuantizeMatMul) against the CPU oracle, through the C ABI.

The int32 sums (sum + C) must be bit-exact, and so must 8-bit outputs; an
fp32 Y must be within 1e-5 relative (reference magnitude |Y| + |bias|)."""
import numpy as np
import pytest

import oracle
from gpu_case import assert_close_c, log, tile_rows, to_dev

pytestmark = pytest.mark.gpu

_T = {"f32": 0, "i8": 2, "u8": 3}


def _q8(r, shape, u8):
    return (r.integers(0, 256, shape).astype(np.uint8) if u8
            else r.integers(-128, 128, shape).astype(np.int8))


def _zp_dev(v, u8, torch):
    if v is None:
        return None
    return to_dev(np.atleast_1d(np.asarray(v)).astype(np.uint8 if u8 else np.int8), torch)


def run_qgemm(dq, A, B, *, a_scale=None, a_zp=None, b_scale, b_zp=None, transA=False,
              transB=False, C=None, alpha=1.0, bias=None, y_type="f32", y_scale=None, y_zp=None,
              accumulators=False, repeat=1):
    """Init + set_b + forward on the GPU; returns Y (and the int32 sums)."""
    import torch

    M, K = (A.shape[1], A.shape[0]) if transA else A.shape
    N = B.shape[0] if transB else B.shape[1]
    a_t = "f32" if A.dtype == np.float32 else ("u8" if A.dtype == np.uint8 else "i8")
    b_u8 = B.dtype == np.uint8
    h = dq.dq_qgemm_init(M, N, K, _T[a_t], transA, _T["u8" if b_u8 else "i8"], transB,
                         _T[y_type], alpha)
    try:
        dq.dq_qgemm_set_b(h, to_dev(B, torch), to_dev(np.atleast_1d(np.float32(b_scale)), torch),
                          _zp_dev(b_zp, b_u8, torch))
        Ad = to_dev(A, torch)
        asd = None if a_scale is None else to_dev(np.float32([a_scale]), torch)
        azd = None if a_zp is None else _zp_dev(a_zp, a_t == "u8", torch)
        Cd = None if C is None else to_dev(np.asarray(C, np.int32), torch)
        bd = None if bias is None else to_dev(bias, torch)
        ysd = None if y_scale is None else to_dev(np.float32([y_scale]), torch)
        yzd = None if y_zp is None else _zp_dev(y_zp, y_type == "u8", torch)
        ydt = {"f32": torch.float32, "u8": torch.uint8, "i8": torch.int8}[y_type]
        Y = torch.empty((M, N), dtype=ydt, device="cuda")
        for _ in range(repeat):
            dq.dq_qgemm_forward(h, Ad, asd, azd, Cd, bd, ysd, yzd, Y)
        out = {"Y": Y.cpu().numpy(), "info": dq.dq_qgemm_info(h)}
        if accumulators:
            acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
            dq.dq_qgemm_forward_accumulators(h, Ad, asd, azd, Cd, acc)
            out["acc"] = acc.cpu().numpy()
        torch.cuda.synchronize()
    finally:
        dq.dq_qgemm_release(h)
    return out


def _want(A, B, **kw):
    """The oracle's Y and sums for the same arguments."""
    a_zp = kw.pop("a_zp", None)
    a_scale = kw.pop("a_scale", None)
    y_type = kw.pop("y_type", "f32")
    C = kw.pop("C", None)
    if A.dtype == np.float32:
        sc, zp, q = oracle.quantize_tensor_u8(A)
        return oracle.qgemm(q, B, sc, zp, kw.pop("b_scale"), kw.pop("b_zp", None), C=C,
                            y_type=None if y_type == "f32" else y_type, with_acc=True, **kw)
    return oracle.qgemm(A, B, a_scale, 0 if a_zp is None else a_zp, kw.pop("b_scale"),
                        kw.pop("b_zp", None), C=C, y_type=None if y_type == "f32" else y_type,
                        with_acc=True, **kw)


def _check(got, want, y_type, bias=None):
    Yw, accw = want
    if "acc" in got:
        assert np.array_equal(got["acc"], accw), "int32 sums"
    if y_type == "f32":
        return assert_close_c(got["Y"], Yw, "f32", bias)
    assert np.array_equal(got["Y"], Yw), "8-bit Y"
    return 100


# ------------------------------------------------- MatMulIntegerToFloat

MITF = [
    # (M, N, K, a_u8, b_u8, per_column_scale, b_zp, bias)
    (1, 1, 1, True, False, False, None, False),
    (37, 45, 70, True, False, True, None, True),
    (65, 33, 129, True, True, True, "col", True),
    (256, 256, 256, False, True, False, "tensor", False),
    (300, 130, 1000, True, False, True, "col", True),
    (129, 520, 33, False, False, True, "col", True),
]


@pytest.mark.parametrize("M,N,K,a_u8,b_u8,per_col,bzp,bias", MITF)
def test_matmul_integer_to_float(gpu, M, N, K, a_u8, b_u8, per_col, bzp, bias):
    log(f"matmul_integer_to_float {M}x{N}x{K} A:{'u8' if a_u8 else 'i8'} "
        f"B:{'u8' if b_u8 else 'i8'} per_col:{per_col} b_zp:{bzp} bias:{bias}")
    r = np.random.default_rng(M * 31 + N * 7 + K)
    A, B = _q8(r, (M, K), a_u8), _q8(r, (K, N), b_u8)
    bs = r.uniform(0.001, 0.01, N if per_col else 1).astype(np.float32)
    lo, hi = (100, 156) if b_u8 else (-20, 21)
    bz = None if bzp is None else r.integers(lo, hi, N if bzp == "col" else 1).astype(np.int32)
    bv = r.uniform(-1, 1, N).astype(np.float32) if bias else None
    a_zp = int(r.integers(100, 156)) if a_u8 else int(r.integers(-20, 21))
    kw = dict(a_scale=np.float32(0.02), a_zp=a_zp, b_scale=bs, b_zp=bz, bias=bv)
    got = run_qgemm(gpu, A, B, accumulators=True, **kw)
    _check(got, _want(A, B, **kw), "f32", bv)


# ----------------------------------------------------------------- QGemm

QGEMM = [
    # (M, N, K, transA, transB, C shape, alpha, y_type)
    (64, 96, 160, False, False, "MN", 1.0, "u8"),
    (100, 70, 300, True, False, "N", 0.5, "i8"),
    (70, 100, 256, False, True, "1N", 2.0, "f32"),
    (260, 130, 96, True, True, "M1", 1.0, "u8"),
    (33, 257, 1024, False, False, "scalar", 1.25, "i8"),
    (300, 300, 64, False, False, None, 1.0, "u8"),
]


@pytest.mark.parametrize("M,N,K,tA,tB,cshape,alpha,y_type", QGEMM)
def test_qgemm(gpu, M, N, K, tA, tB, cshape, alpha, y_type):
    log(f"qgemm {M}x{N}x{K} transA:{tA} transB:{tB} C:{cshape} alpha:{alpha} Y:{y_type}")
    r = np.random.default_rng(M + 3 * N + 5 * K)
    A = _q8(r, (K, M) if tA else (M, K), True)
    B = _q8(r, (N, K) if tB else (K, N), False)
    bs = r.uniform(0.0005, 0.002, N).astype(np.float32)
    bz = r.integers(-10, 11, N).astype(np.int32)
    Cm = None
    if cshape is not None:
        shp = {"MN": (M, N), "N": (N,), "1N": (1, N), "M1": (M, 1), "scalar": ()}[cshape]
        Cm = r.integers(-20000, 20000, shp).astype(np.int32)
    kw = dict(a_scale=np.float32(0.01), a_zp=128, b_scale=bs, b_zp=bz, transA=tA, transB=tB,
              C=Cm, alpha=alpha, y_type=y_type)
    if y_type != "f32":
        # real spans about +-(a few units) x 1e-3 .. : y_scale puts it on ~+-100 codes
        kw.update(y_scale=np.float32(0.002), y_zp=(128 if y_type == "u8" else 3))
    got = run_qgemm(gpu, A, B, accumulators=True, **kw)
    want = _want(A, B, **{k: v for k, v in kw.items() if k not in ("y_scale", "y_zp")},
                 **({"y_scale": kw["y_scale"], "y_zp": kw["y_zp"]} if y_type != "f32" else {}))
    _check(got, want, y_type)
    if y_type != "f32":
        # both saturation ends occur and the codes are not all equal
        assert len(np.unique(got["Y"])) > 50


# ---------------------------------------------------- DynamicQuantizeMatMul

DQMM = [
    # (M, N, K, b_u8, per_col, b_zp, bias)
    (64, 64, 128, False, True, None, True),
    (513, 257, 300, False, True, "col", True),
    (1000, 200, 512, True, False, "tensor", False),
    (7, 1000, 48, False, True, None, True),
]


@pytest.mark.parametrize("M,N,K,b_u8,per_col,bzp,bias", DQMM)
def test_dynamic_quantize_matmul(gpu, M, N, K, b_u8, per_col, bzp, bias):
    log(f"dynamic_quantize_matmul {M}x{N}x{K} B:{'u8' if b_u8 else 'i8'} b_zp:{bzp}")
    r = np.random.default_rng(M + N + K)
    A = r.normal(0.0, 1.0, (M, K)).astype(np.float32)
    A[r.random((M, K)) < 0.01] *= 20.0
    B = _q8(r, (K, N), b_u8)
    bs = r.uniform(0.001, 0.01, N if per_col else 1).astype(np.float32)
    lo, hi = (100, 156) if b_u8 else (-20, 21)
    bz = None if bzp is None else r.integers(lo, hi, N if bzp == "col" else 1).astype(np.int32)
    bv = r.uniform(-1, 1, N).astype(np.float32) if bias else None
    kw = dict(b_scale=bs, b_zp=bz, bias=bv)
    got = run_qgemm(gpu, A, B, accumulators=True, **kw)
    _check(got, _want(A, B, **kw), "f32", bv)


def test_dynamic_quantize_matmul_negative_only_and_zero_tensors(gpu):
    """A tensor without positive values (hi = 0) and an all-zero tensor
    (scale 1, zero point 0)."""
    log("dynamic_quantize_matmul edge tensors")
    r = np.random.default_rng(5)
    B = _q8(r, (40, 24), False)
    bs = np.float32([0.01])
    for A in (-np.abs(r.normal(0, 1, (16, 40))).astype(np.float32),
              np.zeros((16, 40), np.float32)):
        got = run_qgemm(gpu, A, B, b_scale=bs, accumulators=True)
        _check(got, _want(A, B, b_scale=bs), "f32")


# ----------------------------------------------------------- edge cases

def test_qgemm_extreme_sums_stay_exact(gpu):
    """K at its maximum (32768), A = 255 with zero point 0, B = -128 with
    zero point 127: every sum is 255 * -255 * 32768 = -2,130,739,200, next
    to the int32 limit, and the row-sum correction at its largest."""
    log("qgemm extreme sums")
    M, N, K = 64, 64, 32768
    A = np.full((M, K), 255, np.uint8)
    B = np.full((K, N), -128, np.int8)
    kw = dict(a_scale=np.float32(1e-3), a_zp=0, b_scale=np.float32([1e-3]),
              b_zp=np.int32([127]))
    got = run_qgemm(gpu, A, B, accumulators=True, **kw)
    assert (got["acc"] == -255 * 255 * K).all()
    _check(got, _want(A, B, **kw), "f32")


def test_qgemm_repeated_forwards_and_row_subset_at_4096(gpu):
    """4096^3 MatMulIntegerToFloat (u8 A with zero point, i8 B per column):
    three forwards in a row, every int32 sum of two rows from every 256-row
    tile (and the first and last rows) bit-exact."""
    log("matmul_integer_to_float 4096^3 sampled rows")
    r = np.random.default_rng(6)
    M = N = K = 4096
    A, B = _q8(r, (M, K), True), _q8(r, (K, N), False)
    bs = r.uniform(0.001, 0.01, N).astype(np.float32)
    bz = r.integers(-5, 6, N).astype(np.int32)
    bv = r.uniform(-1, 1, N).astype(np.float32)
    kw = dict(a_scale=np.float32(0.02), a_zp=117, b_scale=bs, b_zp=bz, bias=bv)
    got = run_qgemm(gpu, A, B, accumulators=True, repeat=3, **kw)
    rows = tile_rows(M, 6)
    Yw, accw = _want(np.ascontiguousarray(A[rows]), B, **kw)
    assert np.array_equal(got["acc"][rows], accw)
    assert_close_c(got["Y"][rows], Yw, "f32", bv)


def test_qgemm_argument_errors_on_device(gpu):
    import torch

    dq = gpu
    h = dq.dq_qgemm_init(8, 8, 16, _T["u8"], False, _T["i8"], False, _T["u8"], 1.0)
    try:
        A = torch.zeros((8, 16), dtype=torch.uint8, device="cuda")
        Y = torch.zeros((8, 8), dtype=torch.uint8, device="cuda")
        s = torch.ones(1, dtype=torch.float32, device="cuda")
        # forward before set_b
        with pytest.raises(dq.DQError) as e:
            dq.dq_qgemm_forward(h, A, s, None, None, None, s, None, Y)
        assert e.value.status == dq.DQ_ERR_STATE
        B = torch.zeros((16, 8), dtype=torch.int8, device="cuda")
        with pytest.raises(dq.DQError) as e:   # b_scale of 3 entries
            dq.dq_qgemm_set_b(h, B, torch.ones(3, device="cuda"))
        assert e.value.status == dq.DQ_ERR_ARG
        dq.dq_qgemm_set_b(h, B, s)
        with pytest.raises(dq.DQError) as e:   # 8-bit Y without y_scale
            dq.dq_qgemm_forward(h, A, s, None, None, None, None, None, Y)
        assert e.value.status == dq.DQ_ERR_ARG
        with pytest.raises(dq.DQError) as e:   # bias with an 8-bit Y
            dq.dq_qgemm_forward(h, A, s, None, None, torch.zeros(8, device="cuda"), s, None, Y)
        assert e.value.status == dq.DQ_ERR_ARG
        with pytest.raises(dq.DQError) as e:   # C that does not broadcast
            dq.dq_qgemm_forward(h, A, s, None, torch.zeros((3, 8), dtype=torch.int32,
                                                           device="cuda"), None, s, None, Y)
        assert e.value.status == dq.DQ_ERR_ARG
        dq.dq_qgemm_forward(h, A, s, None, None, None, s, None, Y)
        torch.cuda.synchronize()
    finally:
        dq.dq_qgemm_release(h)


@pytest.mark.parametrize("kind", ["mitf", "dqmm", "qgemm"])
def test_benchmark_products_full_size(gpu, kind):
    """The three timed 4096^3 products (MatMulIntegerToFloat, DynamicQuantizeMatMul,
    QGemm with uint8 Y) with their seed and arguments: the int32 sums and Y of
    two rows from every 256-row tile (and the first and last rows) against
    the oracle. A row of the result depends only on its
    row of A, once DynamicQuantizeMatMul's per-tensor quantization has been
    taken over the whole of A."""
    import workloads

    c = workloads.qgemm_case(kind)
    A, B, M = c["A"], c["B"], c["M"]
    kw = dict(b_scale=c["b_scale"], b_zp=c["b_zp"])
    if kind != "dqmm":
        kw.update(a_scale=c["a_scale"], a_zp=c["a_zp"])
    if kind == "qgemm":
        kw.update(C=c["C"], y_type="u8", y_scale=c["y_scale"], y_zp=c["y_zp"])
    else:
        kw["bias"] = c["bias"]
    log(f"{c['name']} sampled rows")
    got = run_qgemm(gpu, A, B, accumulators=True, **kw)
    rows = tile_rows(M, 11)
    if kind == "dqmm":
        sc, zp, q = oracle.quantize_tensor_u8(A)
        want = oracle.qgemm(np.ascontiguousarray(q[rows]), B, sc, zp, c["b_scale"], c["b_zp"],
                            bias=c["bias"], with_acc=True)
    else:
        want = _want(np.ascontiguousarray(A[rows]), B, **dict(kw))
    _check({"Y": got["Y"][rows], "acc": got["acc"][rows]}, want, kw.get("y_type", "f32"), kw.get("bias"))


# ------------------------------------------------------ seeded random cases

def _random_qgemm_cases(seed, n):
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dyn = r.integers(4) == 0  # DynamicQuantizeMatMul: fp32 A quantized per tensor
        p = dict(M=int(r.integers(1, 600)), N=int(r.integers(1, 600)), K=int(r.integers(1, 1500)),
                 a=("f32" if dyn else ["u8", "i8"][int(r.integers(2))]), b_u8=bool(r.integers(2)),
                 per_col=bool(r.integers(2)), bzp=[None, "tensor", "col"][int(r.integers(3))],
                 seed=int(r.integers(1 << 30)))
        if dyn:
            p.update(tA=False, tB=False, C=None, alpha=1.0, y="f32", bias=bool(r.integers(2)))
        else:
            p.update(tA=bool(r.integers(2)), tB=bool(r.integers(2)),
                     C=[None, "scalar", "N", "1N", "M1", "MN"][int(r.integers(6))],
                     alpha=float(r.choice([1.0, 0.5, 1.75])), y=["f32", "u8", "i8"][int(r.integers(3))])
            p["bias"] = p["y"] == "f32" and bool(r.integers(2))
        out.append(p)
    return out


@pytest.mark.parametrize("p", _random_qgemm_cases(2030, 24),
                         ids=lambda p: f"{p['M']}x{p['N']}x{p['K']}-{p['a']}-{p['y']}")
def test_random_quantized_products(gpu, p):
    """Seeded random cases of the three operators: the int32 sums and 8-bit
    outputs bit-exact, fp32 outputs within the bar. An 8-bit output's y_scale
    is set from the oracle's fp32 output, so the codes spread over the range
    and both ends saturate."""
    log(f"quantized product random {p}")
    M, N, K = p["M"], p["N"], p["K"]
    r = np.random.default_rng(p["seed"])
    if p["a"] == "f32":
        A = r.normal(0.0, 1.0, (M, K)).astype(np.float32)
        A[r.random((M, K)) < 0.01] *= 20.0
    else:
        A = _q8(r, (K, M) if p["tA"] else (M, K), p["a"] == "u8")
    B = _q8(r, (N, K) if p["tB"] else (K, N), p["b_u8"])
    bs = r.uniform(0.0005, 0.005, N if p["per_col"] else 1).astype(np.float32)
    lo, hi = (100, 156) if p["b_u8"] else (-20, 21)
    bz = None if p["bzp"] is None else r.integers(lo, hi, N if p["bzp"] == "col" else 1).astype(np.int32)
    kw = dict(b_scale=bs, b_zp=bz)
    if p["a"] != "f32":
        kw.update(a_scale=np.float32(0.01), a_zp=int(r.integers(100, 156)) if p["a"] == "u8" else int(r.integers(-20, 21)),
                  transA=p["tA"], transB=p["tB"], alpha=p["alpha"])
        if p["C"] is not None:
            shp = {"MN": (M, N), "N": (N,), "1N": (1, N), "M1": (M, 1), "scalar": ()}[p["C"]]
            kw["C"] = r.integers(-20000, 20000, shp).astype(np.int32)
    if p["bias"]:
        kw["bias"] = r.uniform(-1, 1, N).astype(np.float32)
    if p["y"] == "f32":
        got = run_qgemm(gpu, A, B, accumulators=True, **kw)
        _check(got, _want(A, B, **dict(kw)), "f32", kw.get("bias"))
        return
    yf, _ = _want(A, B, **dict(kw))
    y_scale = np.float32(max(float(np.std(yf)), 1e-6) / 40.0)
    y_zp = 128 if p["y"] == "u8" else 3
    got = run_qgemm(gpu, A, B, accumulators=True, y_type=p["y"], y_scale=y_scale, y_zp=y_zp, **kw)
    _check(got, _want(A, B, y_type=p["y"], y_scale=y_scale, y_zp=y_zp, **dict(kw)), p["y"])
