"""GPU parity of the element-wise quantized operators against the CPU oracle.

Every output is an integer (8-bit codes, int32 products and sums), so the
bar is bit-exact equality on every element. Cases cover each kernel variant:
16-, 4- and 1-byte vectors, each broadcast pattern, unaligned pointers,
ragged tails, tiny scales (the IEEE-division path), row, column and general
reductions, split sums, and concat with empty and misaligned inputs.
"""
import zlib

import numpy as np
import pytest

import oracle
from gpu_case import log

pytestmark = pytest.mark.gpu


def _seed(*key):
    """A seed that names the case (stable across processes, unlike hash())."""
    return zlib.crc32(repr(key).encode())


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _scal(v, dt=np.float32):
    return _dev(np.asarray([v], dt))


def _zp(v, t):
    return _scal(v, np.uint8 if t == "u8" else np.int8)


def _codes(r, shape, t):
    return (r.integers(0, 256, shape).astype(np.uint8) if t == "u8"
            else r.integers(-128, 128, shape).astype(np.int8))


def _type(dq, t):
    return dq.DQ_U8 if t == "u8" else dq.DQ_I8


def _tdt(t):
    import torch

    return torch.uint8 if t == "u8" else torch.int8


# ================================================================= binary

BIN_SHAPES = [
    ((64, 1024), (64, 1024)),     # flat, 16-byte vectors
    ((64, 1024), (1024,)),        # row vector B
    ((64, 1024), (64, 1)),        # column vector B (broadcast byte)
    ((1, 512), (300, 512)),       # A broadcast along rows
    ((4096, 33), ()),             # scalar B, merged to one flat dim
    ((3, 5, 36), (5, 1)),         # inner 36: 4-byte vectors
    ((2, 3, 4, 5), (3, 1, 5)),    # inner 5: one element per lane
    ((1000003,), (1000003,)),     # ragged flat
    ((7,), (7,)),
    ((2, 1, 3, 16), (4, 1, 16)),  # broadcast on both sides
    ((0, 16), (16,)),             # empty
]


def _run_binary(dq, op, t, A, B, sa, za, sb, zb, sc, zc, offset=0):
    import torch

    shape = np.broadcast_shapes(A.shape, B.shape)
    Ad, Bd = _dev(A), _dev(B)
    if op == "mulint":
        C = torch.empty(int(np.prod(shape)) + offset, dtype=torch.int32, device="cuda")[offset:]
        dq.dq_mul_integer(Ad, _zp(za, t), Bd, _zp(zb, t), _type(dq, t), C, a_shape=A.shape,
                          b_shape=B.shape)
    else:
        C = torch.empty(int(np.prod(shape)) + offset, dtype=_tdt(t), device="cuda")[offset:]
        fn = dq.qlinear_add if op == "add" else dq.qlinear_mul
        fn(Ad, _scal(sa), _zp(za, t), Bd, _scal(sb), _zp(zb, t), _scal(sc), _zp(zc, t),
           _type(dq, t), C, a_shape=A.shape, b_shape=B.shape)
    torch.cuda.synchronize()
    return C.cpu().numpy().reshape(shape)


def _want_binary(op, A, B, sa, za, sb, zb, sc, zc):
    if op == "add":
        return oracle.qlinear_add(A, sa, za, B, sb, zb, sc, zc)
    if op == "mul":
        return oracle.qlinear_mul(A, sa, za, B, sb, zb, sc, zc)
    return oracle.mul_integer(A, za, B, zb)


def _params(r, op, t):
    lo, hi = (0, 256) if t == "u8" else (-128, 128)
    za, zb, zc = (int(v) for v in r.integers(lo, hi, 3))
    sa, sb = np.float32(r.uniform(0.002, 0.05)), np.float32(r.uniform(0.002, 0.05))
    sc = np.float32(r.uniform(0.01, 0.1)) if op == "add" else np.float32(r.uniform(0.5, 5.0))
    return sa, za, sb, zb, sc, zc


@pytest.mark.parametrize("sa_,sb_", BIN_SHAPES)
@pytest.mark.parametrize("t", ["u8", "i8"])
@pytest.mark.parametrize("op", ["add", "mul", "mulint"])
def test_binary_matches_oracle(gpu, op, t, sa_, sb_):
    r = np.random.default_rng(_seed(op, t, sa_, sb_))
    A, B = _codes(r, sa_, t), _codes(r, sb_, t)
    p = _params(r, op, t)
    log(f"binary {op} {t} {sa_} x {sb_}")
    got = _run_binary(gpu, op, t, A, B, *p)
    want = _want_binary(op, A, B, *p)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ"


@pytest.mark.parametrize("op", ["add", "mul", "mulint"])
def test_binary_swapped_operands_and_unaligned_output(gpu, op):
    # B broadcast into A's place (the (0, 1) operand pattern) and an output
    # one element past an aligned address (forces the one-element lanes)
    r = np.random.default_rng(11)
    A, B = _codes(r, (1024,), "u8"), _codes(r, (96, 1024), "u8")
    p = _params(r, op, "u8")
    want = _want_binary(op, A, B, *p)
    assert np.array_equal(_run_binary(gpu, op, "u8", A, B, *p), want)
    assert np.array_equal(_run_binary(gpu, op, "u8", A, B, *p, offset=1), want)


@pytest.mark.parametrize("op", ["add", "mul"])
@pytest.mark.parametrize("t", ["u8", "i8"])
def test_binary_ties_saturation_and_tiny_scales(gpu, op, t):
    # every (a, b) pair; power-of-two scales put many quotients exactly on
    # .5 ties; a C_scale below 2^-100 takes the IEEE-division path
    lo, hi = (0, 256) if t == "u8" else (-128, 128)
    codes = np.arange(lo, hi).astype(np.uint8 if t == "u8" else np.int8)
    A = np.repeat(codes, 256).reshape(256, 256)
    B = np.tile(codes, 256).reshape(256, 256)
    for sa, sb, sc in ((0.5, 0.25, 1.0), (0.125, 2.0, 4.0), (1e-20, 1e-20, 1e-33),
                       (np.float32(0.0371), np.float32(0.0113), np.float32(0.0517))):
        if op == "mul" and sc == 1e-33:
            sc = 1e-38
        za, zb, zc = (3, -2, 1) if t == "i8" else (131, 120, 128)
        got = _run_binary(gpu, op, t, A, B, sa, za, sb, zb, sc, zc)
        want = _want_binary(op, A, B, sa, za, sb, zb, sc, zc)
        assert np.array_equal(got, want), f"scales {sa} {sb} {sc}: {(got != want).sum()} differ"


def test_binary_bench_size(gpu):
    # the size the benchmark times: [8192, 8192] uint8 plus a row vector
    r = np.random.default_rng(12)
    A, B = _codes(r, (8192, 8192), "u8"), _codes(r, (8192,), "u8")
    p = _params(r, "add", "u8")
    log("binary add at [8192, 8192] + [8192]")
    got = _run_binary(gpu, "add", "u8", A, B, *p)
    # 256 sampled rows: each output row depends only on its row of A and B
    rows = np.sort(r.choice(8192, 256, replace=False))
    want = oracle.qlinear_add(A[rows], p[0], p[1], B, p[2], p[3], p[4], p[5])
    assert np.array_equal(got[rows], want)


# ======================================================= one-code functions

def _run_unary(dq, fn, t, X, xs, xz, ys, yz, alpha=0.01, offset=0):
    import torch

    n = X.size
    xd = torch.empty(n + offset, dtype=_tdt(t), device="cuda")
    xd[offset:] = _dev(X.reshape(-1))
    y = torch.empty(n + offset, dtype=_tdt(t), device="cuda")
    if fn == "leaky":
        dq.qlinear_leaky_relu(xd[offset:], _scal(xs), _zp(xz, t), _scal(ys), _zp(yz, t),
                              _type(dq, t), y[offset:], alpha=alpha)
    else:
        dq.qlinear_sigmoid(xd[offset:], _scal(xs), _zp(xz, t), _scal(ys), _zp(yz, t),
                           _type(dq, t), y[offset:])
    torch.cuda.synchronize()
    return y[offset:].cpu().numpy().reshape(X.shape)


def _want_unary(fn, X, xs, xz, ys, yz, alpha=0.01):
    if fn == "leaky":
        return oracle.qlinear_leaky_relu(X, xs, xz, ys, yz, alpha)
    return oracle.qlinear_sigmoid(X, xs, xz, ys, yz)


UNARY_PARAMS = [
    (0.0625, 0, 1 / 256, -128, 0.01),
    (0.05, 7, 0.02, 3, 0.2),
    (np.float32(0.0371), -5, np.float32(0.0093), 11, 0.01),
    (1e-30, 0, 1e-39, 0, 0.5),      # tiny output scale: IEEE division in the table
    (0.5, 100, 0.25, 50, 1.0),
]


@pytest.mark.parametrize("fn", ["leaky", "sigmoid"])
@pytest.mark.parametrize("t", ["u8", "i8"])
@pytest.mark.parametrize("prm", UNARY_PARAMS)
def test_unary_every_code(gpu, fn, t, prm):
    xs, xz, ys, yz, alpha = prm
    if t == "u8":
        xz, yz = abs(xz) + 100, abs(yz) + 20
        if fn == "sigmoid":
            yz = 0
    lo = 0 if t == "u8" else -128
    X = np.arange(lo, lo + 256).astype(np.uint8 if t == "u8" else np.int8)
    got = _run_unary(gpu, fn, t, X, xs, xz, ys, yz, alpha)
    want = _want_unary(fn, X, xs, xz, ys, yz, alpha)
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"


@pytest.mark.parametrize("fn", ["leaky", "sigmoid"])
@pytest.mark.parametrize("n,offset", [(1000003, 0), (4096 * 1024, 0), (65537, 1), (15, 0), (1, 3)])
def test_unary_streams(gpu, fn, n, offset):
    r = np.random.default_rng(n + offset)
    X = _codes(r, (n,), "i8")
    got = _run_unary(gpu, fn, "i8", X, 0.04, -3, 0.01, 2, 0.1, offset=offset)
    assert np.array_equal(got, _want_unary(fn, X, 0.04, -3, 0.01, 2, 0.1))


# ============================================================== reductions

REDUCE_GPU = [
    ((3, 4, 5), [1]), ((3, 4, 5), [0, 2]), ((3, 4, 5), None), ((3, 4, 5), [-1]),
    ((2, 3, 4, 5), [1, 2]), ((2, 3, 4, 5), [0, 3]), ((7,), [0]), ((6, 1, 4), [1]),
    ((64, 512, 7, 7), [2, 3]),     # global average pool: rows of 49
    ((256, 4096), [1]),            # rows, 16-byte chunks, 64 lanes a row
    ((4096, 256), [0]),            # columns, split over workgroups for the sum
    ((8, 49, 2048), [1]),          # columns of an NHWC pool
    ((3, 1000, 5), [1]),           # columns, one byte a lane
    ((2, 1 << 20), [1]),           # two long rows
    ((1 << 18, 3), [0]),           # three long columns
    ((70000, 2, 16), [1]),         # many column groups (more than 65535)
    ((4, 6, 8), [0, 1, 2]),        # everything
    ((5, 1, 7), [1]),              # only a size-1 dim reduced: count 1
    ((37, 4095), [1]),             # the longest rows staged through LDS
    ((37, 4097), [1]),             # one past it: one byte a lane
    ((1000, 13), [1]),             # short rows, many per block, ragged end
]


def _run_reduce(dq, mode, t, X, axes, prm=None):
    import torch

    mask = oracle._axes_mask(X.ndim, axes)
    kept = [n for d, n in enumerate(X.shape) if not mask >> d & 1]
    nout = int(np.prod(kept)) if kept else 1
    xd = _dev(X)
    if mode == "sum":
        y = torch.empty(nout, dtype=torch.int32, device="cuda")
        dq.dq_reduce_sum_integer(xd, _type(dq, t), axes, y)
    else:
        xs, xz, ys, yz = prm
        y = torch.empty(nout, dtype=_tdt(t), device="cuda")
        dq.qlinear_reduce_mean(xd, _type(dq, t), axes, _scal(xs), _zp(xz, t), _scal(ys), _zp(yz, t),
                               y)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("shape,axes", REDUCE_GPU)
@pytest.mark.parametrize("t", ["u8", "i8"])
def test_reduce_sum_integer_matches_oracle(gpu, shape, axes, t):
    r = np.random.default_rng(_seed(shape, str(axes), t))
    X = _codes(r, shape, t)
    log(f"reduce_sum {t} {shape} axes {axes}")
    got = _run_reduce(gpu, "sum", t, X, axes)
    want = oracle.reduce_sum_integer(X, axes, keepdims=False).reshape(-1)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{(got != want.view(np.int32)).sum()} differ"


@pytest.mark.parametrize("shape,axes", REDUCE_GPU)
@pytest.mark.parametrize("t", ["u8", "i8"])
def test_qlinear_reduce_mean_matches_oracle(gpu, shape, axes, t):
    r = np.random.default_rng(_seed(shape, str(axes), t, 1))
    X = _codes(r, shape, t)
    prm = (np.float32(0.0213), 5 if t == "i8" else 121, np.float32(0.0041), -7 if t == "i8" else 119)
    log(f"reduce_mean {t} {shape} axes {axes}")
    got = _run_reduce(gpu, "mean", t, X, axes, prm)
    want = oracle.qlinear_reduce_mean(X, *prm, axes=axes, keepdims=False).reshape(-1)
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ"


def test_reduce_mean_ties(gpu):
    # power-of-two scales: means like 1.5 and 2.5 land exactly on ties
    X = np.array([[1, 2], [2, 3], [3, 4], [0, 5], [255, 255]], np.uint8)
    got = _run_reduce(gpu, "mean", "u8", X, [1], (1.0, 0, 1.0, 0))
    assert got.tolist() == oracle.qlinear_reduce_mean(X, 1.0, 0, 1.0, 0, [1], False).tolist()
    assert got.tolist() == [2, 2, 4, 2, 255]


def test_reduce_sum_wraps_like_int32(gpu):
    # 2^24 codes of 255 sum to 255 * 2^24 >= 2^31: the int32 accumulation
    # wraps, and its bit pattern is the exact uint32 sum
    X = np.full((2, 1 << 24), 255, np.uint8)
    got = _run_reduce(gpu, "sum", "u8", X, [1])
    assert got.view(np.uint32).tolist() == [255 << 24] * 2


def test_reduce_sum_over_an_empty_axis_is_zero(gpu):
    import torch

    y = torch.full((6,), 7, dtype=torch.int32, device="cuda")
    x = torch.empty(0, dtype=torch.uint8, device="cuda")
    gpu.dq_reduce_sum_integer(x, gpu.DQ_U8, [1], y, shape=(6, 0))
    torch.cuda.synchronize()
    assert y.cpu().tolist() == [0] * 6


# ================================================================= concat

CONCAT_CASES = [
    (((2, 16, 8), (2, 32, 8), (2, 16, 8)), 1),     # 16-byte rows
    (((4, 5, 7), (4, 3, 7)), 1),                   # ragged rows
    (((3, 4), (5, 4), (1, 4)), 0),
    (((6, 10), (6, 6)), -1),
    (((2, 3, 49), (2, 0, 49), (2, 5, 49)), 1),     # an empty input
    (((1, 64, 56, 56), (1, 32, 56, 56)), 1),       # NCHW channel concat
    (((128, 256), (128, 512), (128, 256), (128, 1024)), 1),
    (tuple((3, 16 * k + 16, 4) for k in range(10)), 1),   # ten inputs: two launches
    (tuple((2, k + 1, 3) for k in range(9)), 1),          # nine ragged inputs
]


@pytest.mark.parametrize("shapes,axis", CONCAT_CASES)
@pytest.mark.parametrize("t", ["u8", "i8"])
def test_qlinear_concat_matches_oracle(gpu, shapes, axis, t):
    import torch

    r = np.random.default_rng(_seed(shapes, axis, t))
    lo, hi = (0, 256) if t == "u8" else (-128, 128)
    ins = []
    for i, s in enumerate(shapes):
        x = _codes(r, s, t)
        sc = np.float32(r.uniform(0.01, 0.05)) if i != 1 else np.float32(0.02)
        ins.append((x, sc, int(r.integers(lo, hi))))
    ys, yz = np.float32(0.02), int(r.integers(lo, hi))
    want = oracle.qlinear_concat(ins, ys, yz, axis)
    dev = [(_dev(x), _scal(s), _zp(z, t)) for x, s, z in ins]
    y = torch.empty(want.shape, dtype=_tdt(t), device="cuda")
    gpu.qlinear_concat(dev, axis, _scal(ys), _zp(yz, t), _type(gpu, t), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert np.array_equal(got, want), f"{(got != want).sum()} differ"


@pytest.mark.parametrize("kind", ["add", "add_rowvec", "mul", "mul_integer", "sigmoid", "leaky_relu",
                                  "sum_rows", "sum_cols", "mean_rows", "mean_pool_nchw", "mean_pool_nhwc",
                                  "concat"])
def test_benchmark_workloads_full_size(gpu, kind):
    """Every timed element-wise workload at its full size with its seed and
    parameters. The oracle computes a sample of the outputs exactly: the
    outputs of one row (batch entry, column) depend only on that row of
    the inputs, and a one-code function only on its code."""
    import torch
    import workloads

    c = workloads.elementwise_case(kind)
    t, xs, sc, zp = c["type"], c["xs"], c["scales"], c["zps"]
    r = np.random.default_rng(_seed("bench", kind))
    log(f"element-wise benchmark workload {kind}: {[x.shape for x in xs]}")
    if kind in ("add", "add_rowvec", "mul", "mul_integer"):
        op = {"add": "add", "add_rowvec": "add", "mul": "mul", "mul_integer": "mulint"}[kind]
        A, B = xs
        got = _run_binary(gpu, op, t, A, B, sc[0], zp[0], sc[1], zp[1], sc[2], zp[2])
        rows = np.sort(r.choice(A.shape[0], 256, replace=False))
        Bs = B[rows] if B.ndim == A.ndim else B
        want = _want_binary(op, A[rows], Bs, sc[0], zp[0], sc[1], zp[1], sc[2], zp[2])
        part = got[rows]
    elif kind in ("sigmoid", "leaky_relu"):
        fn = "leaky" if kind == "leaky_relu" else "sigmoid"
        X = xs[0]
        got = _run_unary(gpu, fn, t, X, sc[0], zp[0], sc[1], zp[1], alpha=c.get("alpha", 0.01))
        idx = np.unique(r.integers(0, X.size, 1 << 20))
        want = _want_unary(fn, X[idx], sc[0], zp[0], sc[1], zp[1], alpha=c.get("alpha", 0.01))
        part = got[idx]
    elif kind == "concat":
        ax = c["axis"]
        shape = list(xs[0].shape)
        shape[ax] = sum(x.shape[ax] for x in xs)
        y = torch.empty(shape, dtype=_tdt(t), device="cuda")
        gpu.qlinear_concat([(_dev(x), _scal(s), _zp(z, t)) for x, s, z in zip(xs, sc, zp)], ax,
                           _scal(sc[len(xs)]), _zp(zp[len(xs)], t), _type(gpu, t), y)
        torch.cuda.synchronize()
        ns = np.sort(r.choice(shape[0], 4, replace=False))
        want = oracle.qlinear_concat([(x[ns], s, z) for x, s, z in zip(xs, sc, zp)], sc[len(xs)],
                                     zp[len(xs)], ax)
        part = y.cpu().numpy()[ns]
    else:
        X, axes = xs[0], c["axes"]
        mode = "sum" if kind.startswith("sum_") else "mean"
        got = _run_reduce(gpu, mode, t, X, axes, None if mode == "sum" else (sc[0], zp[0], sc[1], zp[1]))
        kept = [n for d, n in enumerate(X.shape) if d not in axes]
        got = got.reshape(kept)
        if axes == [0]:  # columns: each output is one column of X
            cols = np.sort(r.choice(X.shape[1], 256, replace=False))
            Xs, part = X[:, cols], got[cols]
        else:  # the leading axis is kept: each output row reads one leading entry of X
            ns = np.sort(r.choice(X.shape[0], min(64, X.shape[0]), replace=False))
            Xs, part = X[ns], got[ns]
        want = (oracle.reduce_sum_integer(Xs, axes=axes) if mode == "sum"
                else oracle.qlinear_reduce_mean(Xs, sc[0], zp[0], sc[1], zp[1], axes=axes))
        want = want.reshape(part.shape)
    assert part.shape == want.shape, (part.shape, want.shape)
    assert np.array_equal(part, want), f"{(part != want).sum()} of {part.size} differ"


def _random_broadcast_cases(seed, n):
    """Seeded random numpy-broadcast pairs: an output of rank 1-6 (dims 1-24,
    at most ~300K elements); each operand drops some leading dims and sets
    others to 1, on one side, the other or both."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        rank = int(r.integers(1, 7))
        shape = [int(v) for v in r.integers(1, 25, rank)]
        if np.prod(shape) > 300_000:
            continue

        def operand():
            keep = int(r.integers(0, rank + 1)) if r.integers(3) == 0 else rank
            s = shape[rank - keep:]
            return tuple(1 if r.integers(3) == 0 else d for d in s)

        out.append(dict(a=operand(), b=operand(), op=["add", "mul", "mulint"][int(r.integers(3))],
                        t=["u8", "i8"][int(r.integers(2))], seed=int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("p", _random_broadcast_cases(2033, 30), ids=lambda p: f"{p['op']}-{p['a']}x{p['b']}")
def test_binary_random_broadcasts(gpu, p):
    """Every output code bit-exact against the oracle on seeded random
    broadcast shapes (the operands' canonical form: size-1 dims dropped,
    neighbours merged)."""
    r = np.random.default_rng(p["seed"])
    A, B = _codes(r, p["a"], p["t"]), _codes(r, p["b"], p["t"])
    prm = _params(r, p["op"], p["t"])
    log(f"binary random {p['op']} {p['t']} {p['a']} x {p['b']}")
    got = _run_binary(gpu, p["op"], p["t"], A, B, *prm)
    want = _want_binary(p["op"], A, B, *prm)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ"


def _random_reduce_cases(seed, n):
    """Seeded random reductions: rank 1-5 (dims 1-40, up to ~500K elements),
    a random non-empty set of axes (negative indices allowed) or all of them,
    sum or mean, int8 or uint8."""
    r = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        rank = int(r.integers(1, 6))
        shape = tuple(int(v) for v in r.integers(1, 41, rank))
        if np.prod(shape) > 500_000:
            continue
        if r.integers(6) == 0:
            axes = None
        else:
            ax = sorted(set(int(v) for v in r.integers(0, rank, int(r.integers(1, rank + 1)))))
            axes = [a - rank if r.integers(2) else a for a in ax]
        out.append(dict(shape=shape, axes=axes, mode=["sum", "mean"][int(r.integers(2))],
                        t=["u8", "i8"][int(r.integers(2))], seed=int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("p", _random_reduce_cases(2034, 30), ids=lambda p: f"{p['mode']}-{p['shape']}-{p['axes']}")
def test_reduce_random_axes(gpu, p):
    """ReduceSumInteger and QLinearReduceMean bit-exact against the oracle on
    seeded random shapes and axis sets (rows, columns or the general kernel
    by the canonical form)."""
    r = np.random.default_rng(p["seed"])
    t = p["t"]
    X = _codes(r, p["shape"], t)
    log(f"reduce random {p['mode']} {t} {p['shape']} axes {p['axes']}")
    if p["mode"] == "sum":
        got = _run_reduce(gpu, "sum", t, X, p["axes"])
        want = oracle.reduce_sum_integer(X, p["axes"], keepdims=False).reshape(-1)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    else:
        prm = (np.float32(0.0213), 5 if t == "i8" else 121, np.float32(0.0041), -7 if t == "i8" else 119)
        got = _run_reduce(gpu, "mean", t, X, p["axes"], prm)
        want = oracle.qlinear_reduce_mean(X, *prm, axes=p["axes"], keepdims=False).reshape(-1)
        assert np.array_equal(got, want), f"{(got != want).sum()} of {got.size} differ"
