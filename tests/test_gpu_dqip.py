"""GPU parity of the dynamic quantized inner product against the CPU oracle.

Integer outputs (uA, zeroA, iB, column sums, int32 sums) must be bit-exact,
and so must scaleA / scaleB (IEEE division on both sides). C must be within
1e-5 relative (fp32; reference magnitude |C| + |bias|) or 1 ulp (bf16)."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_case import assert_close_c, log, run_dqip, tile_rows

pytestmark = pytest.mark.gpu


def _compare(case, got, want, rows=None, check_b=True):
    r = slice(None) if rows is None else rows
    for key in ("uA", "scaleA", "zeroA"):
        if key in got:
            g = got[key][r]
            w = want[key]
            assert np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                                  w.view(np.uint32) if w.dtype == np.float32 else w), key
    if check_b and "iB" in got:
        assert np.array_equal(got["iB"], want["iB"]), "iB"
        assert np.array_equal(got["scaleB"].view(np.uint32), want["scaleB"].view(np.uint32)), "scaleB"
        assert np.array_equal(got["colsumB"], want["colsumB"]), "colsumB"
    if "acc" in got:
        assert np.array_equal(got["acc"][r], want["acc"]), "int32 sums"
    return assert_close_c(got["C"][r], want["C"], case["typeC"], case.get("bias"))


def test_ramp_usage_example(gpu):
    log("dqip ramp 4x8x16")
    case = W.dqip_ramp()
    got = run_dqip(gpu, case)
    exact = _compare(case, got, oracle.dqip_forward(case))
    log(f"  {exact}% of C bit-identical; info: {got['info']}")


def test_small_64x64x128(gpu):
    log("dqip 64x64x128")
    case = W.dqip_small()
    _compare(case, run_dqip(gpu, case), oracle.dqip_forward(case))


SWEEP = [
    # (M, N, K, typeA, typeB, constB, typeC, act, avoid)
    (1, 1, 1, "f32", "f32", True, "f32", "identity", False),
    (7, 13, 29, "f32", "f32", True, "f32", "relu", True),
    (129, 130, 200, "bf16", "i8", True, "bf16", "relu", False),
    (257, 63, 513, "f32", "f32", False, "f32", "leaky_relu", True),
    (33, 300, 1000, "bf16", "bf16", False, "bf16", "identity", False),
    (128, 128, 128, "f32", "i8", True, "f32", "identity", False),
    (200, 77, 4100, "f32", "f32", False, "bf16", "relu", False),
    (64, 256, 333, "bf16", "f32", True, "f32", "leaky_relu", False),
    (5, 1, 70, "f32", "bf16", False, "f32", "identity", True),
    (300, 5, 16, "bf16", "i8", True, "f32", "relu", False),
    # small products in one launch (constant B, K % 16 == 0, K <= 1024): each
    # register depth of the kernel (K <= 128, 256, 512, 1024), bf16 output,
    # leaky ReLU, and a K that ends half way through a 32-deep fragment
    (32, 2048, 256, "f32", "i8", True, "bf16", "leaky_relu", False),
    (48, 100, 1024, "bf16", "f32", True, "f32", "relu", False),
    (7, 33, 272, "f32", "f32", True, "f32", "identity", True),
    (70, 40, 496, "bf16", "i8", True, "bf16", "identity", False),
    # constant B with a short K on the 128 x 128 tiles: ragged M, N ending
    # inside a 32-column block and (N % 4 != 0) inside a 4-column store,
    # K ending half way through a 32-deep fragment
    (1000, 1600, 512, "f32", "i8", True, "f32", "relu", False),
    (700, 2100, 48, "bf16", "f32", True, "bf16", "leaky_relu", True),
    (4100, 1030, 272, "f32", "f32", True, "f32", "identity", False),
    (2048, 1024, 160, "bf16", "i8", True, "f32", "relu", False),
    (1536, 1540, 96, "f32", "f32", True, "bf16", "identity", True),
]


@pytest.mark.parametrize("M,N,K,tA,tB,constB,tC,act,avoid", SWEEP)
def test_sweep_odd_shapes(gpu, M, N, K, tA, tB, constB, tC, act, avoid):
    log(f"dqip sweep {M}x{N}x{K} A:{tA} B:{tB} const:{constB} C:{tC} {act} avoid:{avoid}")
    case = W.dqip_random(M, N, K, seed=M * 7 + N * 3 + K, typeA=tA, typeB=tB, typeC=tC,
                         constB=constB, act=act, avoid=avoid, alpha=0.1, outliers=0.01,
                         zero_rows=(0,) if M > 2 else (), zero_cols=(N - 1,) if N > 2 else ())
    _compare(case, run_dqip(gpu, case, ext_buf=(M % 2 == 1)), oracle.dqip_forward(case))


DYNAMIC_B = [
    # (M, N, K, typeB, avoid): a non-constant B with N % 4 == 0 (the
    # vectorized maxima and packing kernels), K ragged against the 256-deep
    # padding and against the 64 x 64 packing tiles, N not a multiple of 8, bf16 B
    (40, 520, 1040, "f32", False),
    (24, 132, 4096, "bf16", True),
    (16, 260, 4097, "f32", True),
    (8, 64, 8192, "bf16", False),
    (33, 1028, 2000, "f32", False),
]


@pytest.mark.parametrize("M,N,K,tB,avoid", DYNAMIC_B)
def test_dynamic_b_column_quantizer(gpu, M, N, K, tB, avoid):
    """iB, scaleB and the column sums bit-exact (every column, every k) for
    a B quantized on every call, with all-zero columns and columns whose
    scales fall below 2^-100 (the IEEE division path); C against the oracle."""
    log(f"dqip dynamic B {M}x{N}x{K} B:{tB} avoid:{avoid}")
    case = W.dqip_random(M, N, K, seed=N + K, typeA="f32", typeB="f32", typeC="f32",
                         constB=False, act="relu", avoid=avoid, outliers=0.01,
                         zero_cols=(0, N - 1))
    B = case["B"]
    for j, f in ((3, 1e-33), (N // 2, 3e-38), (N - 5, 1e-36)):
        B[:, j] *= np.float32(f)
    if tB == "bf16":
        case["B"], case["typeB"] = W.to_bf16_bits(B), "bf16"
    _compare(case, run_dqip(gpu, case), oracle.dqip_forward(case))


ROW_PATHS = [
    # (M, K, typeA): register-resident rows of 1..8 groups of 16 per lane,
    # several rows per wave (M above the persistent grid), odd row counts
    (5000, 2048, "f32"),
    (2049, 4096, "f32"),
    (3000, 1024, "bf16"),
    (2100, 8192, "bf16"),
    (4099, 512, "f32"),
]


@pytest.mark.parametrize("M,K,tA", ROW_PATHS)
def test_row_quantizer_paths(gpu, M, K, tA):
    """Every uA / scaleA / zeroA bit-exact for the row-quantizer variants;
    C checked on sampled rows."""
    log(f"dqip row quantizer M={M} K={K} A:{tA}")
    case = W.dqip_random(M, 16, K, seed=M + K, typeA=tA, typeB="i8", typeC="f32", constB=True,
                         outliers=0.01, zero_rows=(0, M // 2, M - 1))
    got = run_dqip(gpu, case, accumulators=False)
    uA, sA, zA = oracle.quantize_rows(case["A"], tA)
    assert np.array_equal(got["zeroA"], zA)
    assert np.array_equal(got["scaleA"].view(np.uint32), sA.view(np.uint32))
    assert np.array_equal(got["uA"], uA)
    _compare_sampled(case, got, _sample_rows(M, 5))


@pytest.mark.parametrize("tA,tB,constB,K", [("f32", "f32", False, 300), ("bf16", "bf16", False, 300),
                                             ("f32", "f32", True, 288), ("bf16", "f32", True, 288)])
def test_tiny_scales_stay_exact(gpu, tA, tB, constB, K):
    """Rows of A and columns of B scaled down until their quantization scales
    fall below 2^-100 and into the subnormal range: there the quantizers'
    reciprocal-and-residual quotient is not exact and the IEEE division must
    be taken; every code, scale and zero point stays bit-exact. A constant B
    with K % 16 == 0 runs the one-launch small-product kernel."""
    log(f"dqip tiny scales A:{tA} B:{tB} const:{constB} K={K}")
    case = W.dqip_random(70, 68, K, seed=21, typeA="f32", typeB="f32", typeC="f32",
                         constB=constB, outliers=0.01)
    A, B = case["A"], case["B"]
    for i, f in ((1, 1e-33), (2, 1e-36), (3, 1e-38), (4, 3e-39)):
        A[i] *= np.float32(f)
    for j, f in ((1, 1e-33), (2, 1e-36), (5, 1e-37), (8, 3e-38)):
        B[:, j] *= np.float32(f)
    if tA == "bf16":
        case["A"], case["typeA"] = W.to_bf16_bits(A), "bf16"
    if tB == "bf16":
        case["B"], case["typeB"] = W.to_bf16_bits(B), "bf16"
    _compare(case, run_dqip(gpu, case), oracle.dqip_forward(case))


def test_tiny_scales_and_unaligned_a_on_128_tiles(gpu):
    """A product on the 128 x 128 GEMM tiles with rows whose scales fall
    below 2^-100 and into the subnormal range (the IEEE division path) and
    all-zero rows, with A 16-byte aligned and only 4-byte aligned (the row
    quantizer's unaligned loads): both bit-exact against the oracle."""
    log("dqip tiny scales + unaligned A, 128 x 128 tiles")
    case = W.dqip_random(1024, 1600, 288, seed=31, typeA="f32", typeB="i8", typeC="f32",
                         constB=True, act="relu", outliers=0.01, zero_rows=(5, 1023))
    A = case["A"]
    for i, f in ((1, 1e-33), (2, 1e-36), (3, 1e-38), (64, 3e-39), (130, 1e-35)):
        A[i] *= np.float32(f)
    want = oracle.dqip_forward(case)
    _compare(case, run_dqip(gpu, case), want)
    _compare(case, run_dqip(gpu, case, a_offset=4), want)


@pytest.mark.parametrize("tA", ["f32", "bf16"])
def test_unaligned_a_takes_the_two_launch_path(gpu, tA):
    """A small product whose A is only 4-byte aligned cannot use the one-
    launch kernel (16-byte loads): the row quantizer's unaligned path and the
    GEMM run instead, with the same results."""
    log(f"dqip unaligned A ({tA})")
    case = W.dqip_random(40, 24, 96, seed=4, typeA=tA, typeB="f32", constB=True, act="relu")
    want = oracle.dqip_forward(case)
    _compare(case, run_dqip(gpu, case, a_offset=4), want)
    _compare(case, run_dqip(gpu, case), want)


def test_no_bias_flag_and_null_bias(gpu):
    log("dqip bias handling")
    case = W.dqip_random(40, 24, 96, seed=3, bias=False)
    _compare(case, run_dqip(gpu, case), oracle.dqip_forward(case))
    # bias flag set but NULL bias pointer: zeros are added
    case2 = dict(case, has_bias=True)
    got = run_dqip(gpu, case2)
    want = oracle.dqip_forward(dict(case2, bias=None))
    _compare(case, got, want)


def test_internal_and_external_buffers_agree_and_repeat_bitwise(gpu):
    log("dqip buffers + determinism")
    case = W.dqip_random(300, 260, 700, seed=11, typeA="bf16", typeB="f32", constB=False,
                         typeC="bf16", act="relu", avoid=True)
    a = run_dqip(gpu, case, ext_buf=False, repeat=3)
    b = run_dqip(gpu, case, ext_buf=True, repeat=2)
    for key in ("C", "uA", "iB", "acc", "colsumB"):
        assert np.array_equal(a[key], b[key]), key


def test_reinit_keeps_or_recreates(gpu):
    import torch

    log("dqip re-init")
    case = W.dqip_random(16, 32, 64, seed=12, typeB="i8")
    got = run_dqip(gpu, case, keep_ctx=True)
    h = got["ctx"]
    try:
        # same parameters: the context and its set parameters are kept
        h2 = gpu.dqip_init(16, 32, 64, gpu.DQ_F32, gpu.DQ_I8, gpu.DQ_F32, True, True,
                           gpu.DQ_ACT_IDENTITY, False, ctx=h)
        assert h2 == h
        A = torch.from_numpy(case["A"]).cuda()
        C = torch.empty((16, 32), device="cuda")
        gpu.dqip_forward(h2, A, None, None, C)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), got["C"])
        # a change (activation): re-created, set_params needed again
        h3 = gpu.dqip_init(16, 32, 64, gpu.DQ_F32, gpu.DQ_I8, gpu.DQ_F32, True, True,
                           gpu.DQ_ACT_RELU, False, ctx=h2)
        with pytest.raises(gpu.DQError) as e:
            gpu.dqip_forward(h3, A, None, None, C)
        assert e.value.status == gpu.DQ_ERR_STATE
        h = h3
    finally:
        gpu.dqip_release(h)


def test_failed_reinit_keeps_the_old_context(gpu, monkeypatch):
    """A re-init whose allocations fail (forced from the host with
    DQIP_FAIL_ALLOC) returns DQ_ERR_ALLOC and leaves the old context valid:
    it still computes the same C and is released exactly once."""
    import torch

    log("dqip failed re-init")
    case = W.dqip_random(16, 32, 64, seed=13, typeB="i8")
    got = run_dqip(gpu, case, keep_ctx=True)
    h = got["ctx"]
    try:
        monkeypatch.setenv("DQIP_FAIL_ALLOC", "1")
        with pytest.raises(gpu.DQError) as e:
            gpu.dqip_init(16, 32, 64, gpu.DQ_F32, gpu.DQ_I8, gpu.DQ_F32, True, True,
                          gpu.DQ_ACT_RELU, False, ctx=h)
        assert e.value.status == gpu.DQ_ERR_ALLOC
        monkeypatch.delenv("DQIP_FAIL_ALLOC")
        A = torch.from_numpy(case["A"]).cuda()
        C = torch.empty((16, 32), device="cuda")
        gpu.dqip_forward(h, A, None, None, C)
        torch.cuda.synchronize()
        assert np.array_equal(C.cpu().numpy(), got["C"])
    finally:
        gpu.dqip_release(h)


def test_argument_errors_on_device(gpu):
    import torch

    log("dqip argument errors")
    h = gpu.dqip_init(8, 8, 8, gpu.DQ_F32, gpu.DQ_F32, gpu.DQ_F32, False, False,
                      gpu.DQ_ACT_IDENTITY, False)
    try:
        A = torch.zeros((8, 8), device="cuda")
        C = torch.empty((8, 8), device="cuda")
        with pytest.raises(gpu.DQError) as e:  # non-constant B missing
            gpu.dqip_forward(h, A, None, None, C)
        assert e.value.status == gpu.DQ_ERR_ARG
        buf = torch.empty(gpu.dqip_external_buffer_size(h) + 512, dtype=torch.uint8, device="cuda")
        with pytest.raises(gpu.DQError) as e:  # misaligned buf
            gpu.dqip_forward(h, A, A, buf.data_ptr() + 1, C)
        assert e.value.status == gpu.DQ_ERR_ARG
        with pytest.raises(gpu.DQError) as e:
            gpu.dqip_read_quantized_a(h, None, None)  # internal buffer never used
        assert e.value.status == gpu.DQ_ERR_STATE
    finally:
        gpu.dqip_release(h)
    h = gpu.dqip_init(8, 8, 8, gpu.DQ_F32, gpu.DQ_I8, gpu.DQ_F32, True, False,
                      gpu.DQ_ACT_IDENTITY, False)
    try:
        B = torch.zeros((8, 8), dtype=torch.int8, device="cuda")
        with pytest.raises(gpu.DQError) as e:  # int8 B without scales
            gpu.dqip_set_params(h, B, None, None, None)
        assert e.value.status == gpu.DQ_ERR_ARG
        with pytest.raises(gpu.DQError) as e:  # forward before set_params
            gpu.dqip_forward(h, torch.zeros((8, 8), device="cuda"), None, None,
                             torch.empty((8, 8), device="cuda"))
        assert e.value.status == gpu.DQ_ERR_STATE
    finally:
        gpu.dqip_release(h)


def test_extreme_sums_stay_exact(gpu):
    """K at its maximum (65536), every code of A at 255 with zero point 0 and
    B at -128 / 127: the int32 sums reach -255*128*65535 = -2,139,095,040 + ...
    next to the int32 limit, and must still be exact."""
    log("dqip extreme sums")
    M, N, K = 64, 64, 65536
    A = np.empty((M, K), np.float32)
    A[:, :] = 1.0
    A[:, 0] = -1e-30  # lo just below 0: zeroA = 0, every other code 255
    B = np.full((K, N), -128, np.int8)
    B[:, 1::2] = 127
    case = dict(name="extreme", M=M, N=N, K=K, A=A, B=B, typeA="f32", typeB="i8", typeC="f32",
                constB=True, bias=None, act="identity", alpha=0.01, avoid=False,
                scaleB=np.full(N, 1e-3, np.float32))
    want = oracle.dqip_forward(case)
    assert int(want["acc"].min()) == -255 * 128 * (K - 1)
    assert abs(int(want["acc"].min())) > 2 ** 30
    _compare(case, run_dqip(gpu, case), want)


# ------------------------------------------------------------ full sizes

def _sample_rows(M, seed, n=12):
    r = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, M - 1], r.integers(0, M, n)])).astype(np.int64)


def _compare_sampled(case, got, rows):
    want = oracle.dqip_forward(case, rows=rows)
    return _compare(case, got, want, rows=rows)


def test_full_4096_bf16_relu(gpu):
    log("dqip full 4096x4096x4096 bf16 A, int8 B, relu, bf16 out")
    case = W.dqip_large()
    got = run_dqip(gpu, case, accumulators=True)
    # quantized A: every row bit-exact
    uA, sA, zA = oracle.quantize_rows(case["A"], "bf16")
    assert np.array_equal(got["uA"], uA) and np.array_equal(got["zeroA"], zA)
    assert np.array_equal(got["scaleA"].view(np.uint32), sA.view(np.uint32))
    assert np.array_equal(got["iB"], case["B"])
    assert np.array_equal(got["colsumB"], oracle.colsum(case["B"]))
    # C and the int32 sums: two rows from every 256-row tile, first and last
    rows = tile_rows(case["M"], 1)
    log(f"  {len(rows)} rows against the oracle")
    _compare_sampled(case, got, rows)


@pytest.mark.parametrize("recurrent", [False, True])
def test_full_lstm_gates(gpu, recurrent):
    log(f"dqip lstm gates recurrent={recurrent}")
    case = W.dqip_lstm(recurrent=recurrent)
    got = run_dqip(gpu, case)
    if recurrent:
        _compare(case, got, oracle.dqip_forward(case))
    else:
        _compare_sampled(case, got, tile_rows(case["M"], 2))


def test_full_8192_dynamic_b(gpu):
    log("dqip full 8192^3 dynamic fp32 B, avoidOverflow")
    case = W.dqip_dynamic_b()
    got = run_dqip(gpu, case, accumulators=False)
    rows = tile_rows(case["M"], 3)
    log(f"  {len(rows)} rows against the oracle")
    want = oracle.dqip_forward(case, rows=rows)
    _compare(case, got, want, rows=rows, check_b=True)


# ------------------------------------------------------------ seeded random shapes

def _random_cases(seed, n, big):
    """n cases drawn from one seeded generator: shapes with ragged edges against
    every tile (32, 128, 256) and the 256-deep K padding, both A types, a
    constant B (fp32 or int8) or one quantized on every call (fp32 or bf16),
    every activation and output type, bias on or off, avoidOverflow, planted
    zero rows and columns, and A 16-byte aligned or not. big: shapes on the
    256 x 256 tiles (checked on sampled rows)."""
    r = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        if big:
            M, N = int(r.integers(3000, 5200)), int(r.integers(3000, 5200))
            K = int(r.integers(16, 1600))
        else:
            M, N = int(r.integers(1, 700)), int(r.integers(1, 700))
            K = int(r.integers(1, 2100))
        tA = ["f32", "bf16"][int(r.integers(2))]
        constB = bool(r.integers(2))
        tB = ["f32", "i8"][int(r.integers(2))] if constB else ["f32", "bf16"][int(r.integers(2))]
        tC = ["f32", "bf16"][int(r.integers(2))]
        act = ["identity", "relu", "leaky_relu"][int(r.integers(3))]
        avoid = bool(r.integers(2)) and tB != "i8"
        bias = bool(r.integers(4))  # three in four with a bias
        a_offset = 0 if r.integers(4) else (4 if tA == "f32" else 2)
        cases.append(dict(M=M, N=N, K=K, tA=tA, tB=tB, constB=constB, tC=tC, act=act, avoid=avoid,
                          bias=bias, a_offset=a_offset, seed=int(r.integers(1 << 30))))
    return cases


def _run_random(gpu, p, rows=None):
    M, N = p["M"], p["N"]
    log(f"dqip random {M}x{N}x{p['K']} A:{p['tA']} B:{p['tB']} const:{p['constB']} C:{p['tC']} "
        f"{p['act']} avoid:{p['avoid']} bias:{p['bias']} A offset:{p['a_offset']} seed:{p['seed']}")
    case = W.dqip_random(M, N, p["K"], seed=p["seed"], typeA=p["tA"], typeB=p["tB"], typeC=p["tC"],
                         constB=p["constB"], bias=p["bias"], act=p["act"], avoid=p["avoid"], alpha=0.2,
                         outliers=0.01, zero_rows=(M // 2,) if M > 3 else (),
                         zero_cols=(N // 3,) if N > 3 else ())
    got = run_dqip(gpu, case, ext_buf=bool(p["seed"] & 1), a_offset=p["a_offset"])
    if rows is None:
        _compare(case, got, oracle.dqip_forward(case))
    else:
        _compare_sampled(case, got, rows)


@pytest.mark.parametrize("p", _random_cases(2026, 28, big=False), ids=lambda p: f"{p['M']}x{p['N']}x{p['K']}")
def test_random_shapes(gpu, p):
    """Every output of the forward against the oracle, on seeded random cases."""
    _run_random(gpu, p)


@pytest.mark.parametrize("p", _random_cases(2027, 6, big=True), ids=lambda p: f"{p['M']}x{p['N']}x{p['K']}")
def test_random_shapes_large_tiles(gpu, p):
    """Seeded random cases on the 256 x 256 tiles: C and the int32 sums on two
    rows of every 256-row tile plus the first and last, the quantized A, B,
    scales and column sums whole."""
    _run_random(gpu, p, rows=tile_rows(p["M"], p["seed"] % 97))
