"""GPU parity of the N-dimensional MatMulIntegerToFloat and
DynamicQuantizeMatMul (numpy.matmul's batch broadcasting, 1-D operands)
against the CPU oracle, through the C ABI (dq_qgemm_init_batched).

The int32 sums must be bit-exact; the fp32 Y within 1e-5 relative
(reference magnitude |Y| + |bias|), as for the 2-D products."""
import numpy as np
import pytest

import oracle
from gpu_case import assert_close_c, log, to_dev

pytestmark = pytest.mark.gpu

_T = {"f32": 0, "i8": 2, "u8": 3}


def _q8(r, shape, u8):
    return (r.integers(0, 256, shape).astype(np.uint8) if u8
            else r.integers(-128, 128, shape).astype(np.int8))


def _shapes(sa, sb):
    """M, N, K, the two batch shapes and Y's shape, by numpy.matmul's rules
    (a 1-D A is one row, a 1-D B one column, dropped from Y)."""
    a_vec, b_vec = len(sa) == 1, len(sb) == 1
    a2 = (1,) + tuple(sa) if a_vec else tuple(sa)
    b2 = tuple(sb) + (1,) if b_vec else tuple(sb)
    M, K, N = a2[-2], a2[-1], b2[-1]
    out = np.matmul(np.zeros(sa, np.int8), np.zeros(sb, np.int8)).shape
    return M, N, K, a2[:-2], b2[:-2], out


def run_nd(dq, A, B, *, a_scale=None, a_zp=None, b_scale, b_zp=None, bias=None,
           accumulators=False, forwards=1):
    """init_batched + set_b + forward on the GPU; returns Y (and the sums).
    forwards > 1 runs the context again on other A's (returned too)."""
    import torch

    As = A if isinstance(A, list) else [A]
    M, N, K, ab, bb, out = _shapes(As[0].shape, B.shape)
    a_t = "f32" if As[0].dtype == np.float32 else ("u8" if As[0].dtype == np.uint8 else "i8")
    b_u8 = B.dtype == np.uint8
    h = dq.dq_qgemm_init_batched(ab, bb, M, N, K, _T[a_t], _T["u8" if b_u8 else "i8"])
    res = {"info": dq.dq_qgemm_info(h)}
    try:
        bz = None if b_zp is None else to_dev(np.atleast_1d(b_zp).astype(np.uint8 if b_u8 else np.int8),
                                              torch)
        dq.dq_qgemm_set_b(h, to_dev(B, torch), to_dev(np.atleast_1d(np.float32(b_scale)), torch), bz)
        asd = None if a_scale is None else to_dev(np.float32([a_scale]), torch)
        azd = None if a_zp is None else to_dev(
            np.atleast_1d(a_zp).astype(np.uint8 if a_t == "u8" else np.int8), torch)
        bd = None if bias is None else to_dev(bias, torch)
        Ys = []
        for Ai in As[:forwards]:
            Y = torch.empty(out, dtype=torch.float32, device="cuda")
            dq.dq_qgemm_forward(h, to_dev(Ai, torch), asd, azd, None, bd, None, None, Y)
            Ys.append(Y.cpu().numpy())
        res["Y"] = Ys[0]
        res["Ys"] = Ys
        if accumulators:
            acc = torch.empty(out, dtype=torch.int32, device="cuda")
            dq.dq_qgemm_forward_accumulators(h, to_dev(As[0], torch), asd, azd, None, acc)
            res["acc"] = acc.cpu().numpy()
        torch.cuda.synchronize()
    finally:
        dq.dq_qgemm_release(h)
    return res


def _want_acc(A, B, a_zp, b_zp):
    """The oracle's int32 sums, batch by batch (oracle.matmul_batches pairs)."""
    M, N, K, yb, out, pairs = oracle.matmul_batches(A.shape, B.shape)
    Ab = np.ascontiguousarray(A).reshape(-1, M, K)
    Bb = np.ascontiguousarray(B).reshape(-1, K, N)
    acc = np.empty((len(pairs), M, N), np.int32)
    for z, (ia, ib) in enumerate(pairs):
        _, acc[z] = oracle.qgemm(Ab[ia], Bb[ib], 1.0, a_zp, 1.0, b_zp, with_acc=True)
    return acc.reshape(out)


MITF_ND = [
    # (A shape, B shape, a_u8, b_u8, per-column scale, b_zp, bias)
    ((2, 3, 37, 70), (70, 45), True, False, True, "col", True),       # one B: batches folded into rows
    ((2, 1, 33, 129), (3, 129, 65), False, True, False, "tensor", False),
    ((65, 40), (4, 40, 33), True, True, True, "col", True),          # A broadcast over B's batches
    ((4, 20, 64), (4, 64, 20), True, False, True, None, True),
    ((1, 6, 64), (5, 64, 7), False, False, False, "col", False),
    ((3, 1, 2, 9, 48), (2, 1, 48, 17), True, False, True, "col", True),
    ((70,), (2, 70, 20), True, False, True, "col", True),              # 1-D A
    ((3, 9, 70), (70,), False, True, False, "tensor", True),           # 1-D B
    ((2, 256, 512), (2, 512, 384), True, False, True, "col", True),   # whole tiles per batch
    ((8, 12, 20, 64), (8, 12, 64, 20), True, False, True, None, False),  # 96 small products
]


@pytest.mark.parametrize("sa,sb,a_u8,b_u8,per_col,bzp,bias", MITF_ND)
def test_matmul_integer_to_float_nd(gpu, sa, sb, a_u8, b_u8, per_col, bzp, bias):
    log(f"matmul_integer_to_float_nd A{sa} B{sb} A:{'u8' if a_u8 else 'i8'} "
        f"B:{'u8' if b_u8 else 'i8'} per_col:{per_col} b_zp:{bzp} bias:{bias}")
    r = np.random.default_rng(sum(sa) * 131 + sum(sb) * 7 + len(sa))
    M, N, K, _, _, out = _shapes(sa, sb)
    A, B = _q8(r, sa, a_u8), _q8(r, sb, b_u8)
    bs = r.uniform(0.001, 0.01, N if per_col else 1).astype(np.float32)
    lo, hi = (100, 156) if b_u8 else (-20, 21)
    bz = None if bzp is None else r.integers(lo, hi, N if bzp == "col" else 1).astype(np.int32)
    bv = r.uniform(-1, 1, N).astype(np.float32) if bias else None
    a_zp = int(r.integers(100, 156)) if a_u8 else int(r.integers(-20, 21))
    a_scale = np.float32(0.02)
    got = run_nd(gpu, A, B, a_scale=a_scale, a_zp=a_zp, b_scale=bs, b_zp=bz, bias=bv,
                 accumulators=True)
    want = oracle.matmul_integer_to_float_nd(A, B, a_scale, bs, a_zp, bz, bv)
    assert got["Y"].shape == want.shape == out
    assert np.array_equal(got["acc"], _want_acc(A, B, a_zp, bz)), "int32 sums"
    assert_close_c(got["Y"], want, "f32", bv)


DQMM_ND = [
    # (A shape, B shape, b_u8, per-column scale, b_zp, bias)
    ((4, 2, 16, 64), (64, 32), False, True, None, True),        # one B: folded
    ((3, 50, 300), (3, 300, 130), False, True, "col", True),
    ((2, 1, 7, 33), (1, 3, 33, 5), True, False, "tensor", False),
    ((40,), (3, 40, 24), False, True, None, True),               # 1-D A
]


@pytest.mark.parametrize("sa,sb,b_u8,per_col,bzp,bias", DQMM_ND)
def test_dynamic_quantize_matmul_nd(gpu, sa, sb, b_u8, per_col, bzp, bias):
    log(f"dynamic_quantize_matmul_nd A{sa} B{sb} B:{'u8' if b_u8 else 'i8'} per_col:{per_col} "
        f"b_zp:{bzp} bias:{bias}")
    r = np.random.default_rng(sum(sa) * 17 + sum(sb))
    M, N, K, _, _, out = _shapes(sa, sb)
    # batches over different ranges: one scale for the whole tensor matters
    A = r.normal(0, 1, sa).astype(np.float32)
    if len(sa) > 2:
        A[0] *= 5
    B = _q8(r, sb, b_u8)
    bs = r.uniform(0.001, 0.01, N if per_col else 1).astype(np.float32)
    lo, hi = (100, 156) if b_u8 else (-20, 21)
    bz = None if bzp is None else r.integers(lo, hi, N if bzp == "col" else 1).astype(np.int32)
    bv = r.uniform(-1, 1, N).astype(np.float32) if bias else None
    got = run_nd(gpu, A, B, b_scale=bs, b_zp=bz, bias=bv, accumulators=True)
    want = oracle.dynamic_quantize_matmul_nd(A, B, bs, bz, bv)
    assert got["Y"].shape == want.shape == out
    sc, zp, q = oracle.quantize_tensor_u8(A)
    assert np.array_equal(got["acc"], _want_acc(q, B, zp, bz)), "int32 sums"
    assert_close_c(got["Y"], want, "f32", bv)


def test_nd_context_runs_again_on_new_inputs(gpu):
    # the packed A buffers of one context are refilled on every forward: a
    # second forward on other values (the fp32 A's range changing) must not
    # keep anything of the first
    r = np.random.default_rng(77)
    sa, sb = (3, 24, 96), (3, 96, 40)
    B = _q8(r, sb, False)
    bs = r.uniform(0.001, 0.01, 40).astype(np.float32)
    A1 = r.normal(0, 1, sa).astype(np.float32)
    A2 = (3 * r.normal(0, 1, sa) + 1).astype(np.float32)
    log("nd context, two forwards A(3,24,96) B(3,96,40)")
    got = run_nd(gpu, [A1, A2], B, b_scale=bs, forwards=2)
    for Ai, Yi in zip((A1, A2), got["Ys"]):
        assert_close_c(Yi, oracle.dynamic_quantize_matmul_nd(Ai, B, bs), "f32")


def test_nd_binding_checks_the_batch_extents(gpu):
    # the binding sizes A, B and Y by the batch counts: tensors of one batch
    # too few are refused before the call
    import torch

    dq = gpu
    h = dq.dq_qgemm_init_batched((2, 3), (1, 3), 8, 16, 32, _T["u8"], _T["i8"])
    try:
        bs = torch.ones(1, dtype=torch.float32, device="cuda")
        with pytest.raises(dq.DQError):
            dq.dq_qgemm_set_b(h, torch.zeros((2, 32, 16), dtype=torch.int8, device="cuda"), bs)
        dq.dq_qgemm_set_b(h, torch.zeros((3, 32, 16), dtype=torch.int8, device="cuda"), bs)
        a_s = torch.ones(1, dtype=torch.float32, device="cuda")
        with pytest.raises(dq.DQError):
            dq.dq_qgemm_forward(h, torch.zeros((5, 8, 32), dtype=torch.uint8, device="cuda"), a_s, None,
                                None, None, None, None,
                                torch.empty((6, 8, 16), dtype=torch.float32, device="cuda"))
        with pytest.raises(dq.DQError):
            dq.dq_qgemm_forward(h, torch.zeros((6, 8, 32), dtype=torch.uint8, device="cuda"), a_s, None,
                                None, None, None, None,
                                torch.empty((5, 8, 16), dtype=torch.float32, device="cuda"))
        # C is not an input of these operators
        with pytest.raises(dq.DQError) as e:
            dq.dq_qgemm_forward(h, torch.zeros((6, 8, 32), dtype=torch.uint8, device="cuda"), a_s, None,
                                torch.zeros((8, 16), dtype=torch.int32, device="cuda"), None, None, None,
                                torch.empty((6, 8, 16), dtype=torch.float32, device="cuda"))
        assert e.value.status == dq.DQ_ERR_ARG
        torch.cuda.synchronize()
    finally:
        dq.dq_qgemm_release(h)
