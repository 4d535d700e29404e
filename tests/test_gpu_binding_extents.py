"""The binding's host-side extent checks: a device tensor too small for the
shape a call implies is refused with DQ_ERR_ARG before anything is launched
(a short buffer would otherwise be read or written out of bounds on the
device). Every call here fails on the host; no kernel runs."""
import pytest

pytestmark = pytest.mark.gpu


def _refused(gpu, fn, *args, **kw):
    with pytest.raises(gpu.DQError) as e:
        fn(*args, **kw)
    assert e.value.status == gpu.DQ_ERR_ARG
    assert "needed" in str(e.value)


def test_qgemm_short_output_and_bias(gpu):
    import torch

    M, N, K = 40, 24, 64
    h = gpu.dq_qgemm_init(M, N, K, gpu.DQ_U8, False, gpu.DQ_I8, False, gpu.DQ_F32)
    try:
        B = torch.zeros((K, N), dtype=torch.int8, device="cuda")
        gpu.dq_qgemm_set_b(h, B, torch.ones(1, device="cuda"))
        A = torch.zeros((M, K), dtype=torch.uint8, device="cuda")
        sa = torch.ones(1, device="cuda")
        _refused(gpu, gpu.dq_qgemm_forward, h, A, sa, None, None, None, None, None,
                 torch.empty(M * N - 1, device="cuda"))
        _refused(gpu, gpu.dq_qgemm_forward, h, A, sa, None, None, torch.zeros(N - 1, device="cuda"),
                 None, None, torch.empty((M, N), device="cuda"))
        _refused(gpu, gpu.dq_qgemm_forward, h, A[:-1], sa, None, None, None, None, None,
                 torch.empty((M, N), device="cuda"))
        _refused(gpu, gpu.dq_qgemm_set_b, h, B[:-1], torch.ones(1, device="cuda"))
    finally:
        gpu.dq_qgemm_release(h)


def test_elementwise_short_outputs(gpu):
    import torch

    u8 = dict(dtype=torch.uint8, device="cuda")
    s = torch.ones(1, device="cuda")
    z = torch.zeros(1, **u8)
    A = torch.zeros((8, 16), **u8)
    Brow = torch.zeros(16, **u8)
    _refused(gpu, gpu.qlinear_add, A, s, z, Brow, s, z, s, z, gpu.DQ_U8, torch.empty(127, **u8))
    _refused(gpu, gpu.dq_mul_integer, A, z, Brow, z, gpu.DQ_U8,
             torch.empty(128, dtype=torch.uint8, device="cuda"))  # int32 output: 512 bytes needed
    _refused(gpu, gpu.qlinear_sigmoid, A, s, z, s, z, gpu.DQ_U8, torch.empty(100, **u8))
    _refused(gpu, gpu.dq_reduce_sum_integer, A, gpu.DQ_U8, [0],
             torch.empty(15, dtype=torch.int32, device="cuda"))
    _refused(gpu, gpu.qlinear_reduce_mean, A, gpu.DQ_U8, [1], s, z, s, z, torch.empty(7, **u8))
    _refused(gpu, gpu.qlinear_concat, [(A, s, z), (A, s, z)], 0, s, z, gpu.DQ_U8,
             torch.empty(255, **u8))


def test_quantize_per_axis_short_scales(gpu):
    import torch

    x = torch.zeros((2, 6, 5), device="cuda")
    y = torch.empty((2, 6, 5), dtype=torch.int8, device="cuda")
    _refused(gpu, gpu.qlinear_quantize, x, torch.ones(5, device="cuda"),
             torch.zeros(6, dtype=torch.int8, device="cuda"), gpu.DQ_I8, y, axis=1)
    _refused(gpu, gpu.qlinear_dequantize, y, gpu.DQ_I8, torch.ones(6, device="cuda"),
             torch.zeros(5, dtype=torch.int8, device="cuda"), x, axis=-2)


def test_qconv_and_lstm_short_outputs(gpu):
    import torch

    h = gpu.dq_qconv_init(8, 9, 9, 16, 3, 3, gpu.DQ_U8, gpu.DQ_I8, gpu.DQ_U8, pads=(1, 1, 1, 1))
    try:
        oh, ow = gpu.dq_qconv_output_shape(h)
        x = torch.zeros((2, 8, 9, 9), dtype=torch.uint8, device="cuda")
        s = torch.ones(1, device="cuda")
        _refused(gpu, gpu.dq_qconv_set_w, h, torch.zeros((16, 8, 3, 2), dtype=torch.int8, device="cuda"), s)
        _refused(gpu, gpu.dq_qconv_forward, h, x, s, None, s, None,
                 torch.empty((2, 16, oh, ow - 1), dtype=torch.uint8, device="cuda"))
    finally:
        gpu.dq_qconv_release(h)
    h = gpu.dq_lstm_init(5, 3, 16, 8, "forward", gpu.DQ_I8, gpu.DQ_I8)
    try:
        X = torch.zeros((5, 3, 16), device="cuda")
        _refused(gpu, gpu.dq_lstm_forward, h, X, Y=torch.empty((5, 1, 3, 7), device="cuda"))
        _refused(gpu, gpu.dq_lstm_forward, h, X[:4])
    finally:
        gpu.dq_lstm_release(h)
