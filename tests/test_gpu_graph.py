"""The operators under stream capture (HIP graphs, through torch.cuda.graph):
each call is captured once after an eager warm-up and replayed for several
input sets, with eager calls between the replays; every replay must equal
the eager result on the same inputs bit for bit. A call that allocates on
first use (the internal work buffer, the prepared convolution input) does
so in the warm-up, and the library's own clears are kernels, not memsets,
so nothing in a forward is an allocation or a memset node."""
import numpy as np
import pytest

import workloads as W
from gpu_case import log, to_dev

pytestmark = pytest.mark.gpu


def _graph_matches_eager(torch, static_inputs, input_sets, run, outputs, replays=2):
    eager = []
    for vals in input_sets:
        for t, v in zip(static_inputs, vals):
            t.copy_(torch.from_numpy(np.ascontiguousarray(v)))
        run()
        torch.cuda.synchronize()
        eager.append([o.clone() for o in outputs])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for _ in range(replays):
        for i, vals in enumerate(input_sets):
            for o in outputs:
                o.zero_()
            for t, v in zip(static_inputs, vals):
                t.copy_(torch.from_numpy(np.ascontiguousarray(v)))
            g.replay()
            torch.cuda.synchronize()
            for k, (o, e) in enumerate(zip(outputs, eager[i])):
                assert torch.equal(o, e), f"replay of input set {i}, output {k}"
            run()  # eager work between the replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K,constB", [(64, 64, 128, True), (1536, 1536, 512, True),
                                          (300, 260, 1100, False)])
def test_dqip_forward_replays(gpu, M, N, K, constB):
    """One-launch small product; row quantizer + 128x128 GEMM; a B quantized
    on every call (fill kernel, column maxima with atomics, packing)."""
    import torch

    log(f"graph dqip {M}x{N}x{K} const:{constB}")
    case = W.dqip_random(M, N, K, seed=M + K, typeA="f32", typeB="f32", typeC="f32",
                         constB=constB, act="relu")
    h = gpu.dqip_init(M, N, K, gpu.DQ_F32, gpu.DQ_F32, gpu.DQ_F32, constB, True,
                      gpu.DQ_ACT_RELU, False)
    try:
        B = to_dev(case["B"], torch)
        bias = to_dev(case["bias"], torch)
        gpu.dqip_set_params(h, B if constB else None, None, bias, None)
        A = to_dev(case["A"], torch)
        C = torch.empty((M, N), device="cuda")
        buf = torch.empty(gpu.dqip_external_buffer_size(h), dtype=torch.uint8, device="cuda")
        r = np.random.default_rng(M)
        sets = [[r.normal(0, 1, (M, K)).astype(np.float32)] for _ in range(3)]
        if not constB:
            sets = [s + [r.normal(0, 0.05, (K, N)).astype(np.float32)] for s in sets]
        statics = [A] if constB else [A, B]
        _graph_matches_eager(torch, statics, sets,
                             lambda: gpu.dqip_forward(h, A, None if constB else B, buf, C), [C])
    finally:
        gpu.dqip_release(h)


def test_quantize_dequantize_replays(gpu):
    import torch

    log("graph Q/DQ per axis")
    r = np.random.default_rng(1)
    shape = (4, 16, 9, 7)
    x = torch.empty(shape, device="cuda")
    ys = to_dev(r.uniform(0.005, 0.05, 16).astype(np.float32), torch)
    yz = to_dev(r.integers(-10, 11, 16).astype(np.int8), torch)
    q = torch.empty(shape, dtype=torch.int8, device="cuda")
    d = torch.empty(shape, device="cuda")

    def run():
        gpu.qlinear_quantize(x, ys, yz, gpu.DQ_I8, q, axis=1)
        gpu.qlinear_dequantize(q, gpu.DQ_I8, ys, yz, d, axis=1)

    sets = [[r.normal(0, 1, shape).astype(np.float32)] for _ in range(3)]
    _graph_matches_eager(torch, [x], sets, run, [q, d])


def test_dynamic_quantize_matmul_replays(gpu):
    """fp32 A quantized per tensor on every call (extremes by atomics after
    a clearing kernel), then the product with per-column B zero points."""
    import torch

    log("graph DynamicQuantizeMatMul")
    M, N, K = 200, 96, 160
    r = np.random.default_rng(2)
    h = gpu.dq_qgemm_init(M, N, K, gpu.DQ_F32, False, gpu.DQ_U8, False, gpu.DQ_F32)
    try:
        gpu.dq_qgemm_set_b(h, to_dev(r.integers(0, 256, (K, N)).astype(np.uint8), torch),
                           to_dev(r.uniform(0.001, 0.01, N).astype(np.float32), torch),
                           to_dev(r.integers(100, 156, N).astype(np.uint8), torch))
        A = torch.empty((M, K), device="cuda")
        bias = to_dev(r.uniform(-1, 1, N).astype(np.float32), torch)
        Y = torch.empty((M, N), device="cuda")
        sets = [[r.normal(0, 1, (M, K)).astype(np.float32)] for _ in range(3)]
        _graph_matches_eager(torch, [A], sets,
                             lambda: gpu.dq_qgemm_forward(h, A, None, None, None, bias, None, None, Y),
                             [Y])
    finally:
        gpu.dq_qgemm_release(h)


def test_qlinear_conv_replays(gpu):
    """The prepared input and the implicit GEMM of a 3x3 layer (the prepared
    input's buffer is grown by the eager warm-up)."""
    import torch

    log("graph QLinearConv 3x3")
    r = np.random.default_rng(3)
    N, C, H, Wd, M = 2, 32, 14, 14, 64
    h = gpu.dq_qconv_init(C, H, Wd, M, 3, 3, gpu.DQ_U8, gpu.DQ_I8, gpu.DQ_U8, pads=(1, 1, 1, 1))
    try:
        oh, ow = gpu.dq_qconv_output_shape(h)
        gpu.dq_qconv_set_w(h, to_dev(r.integers(-128, 128, (M, C, 3, 3)).astype(np.int8), torch),
                           to_dev(r.uniform(0.001, 0.01, M).astype(np.float32), torch), None,
                           to_dev(r.integers(-500, 500, M).astype(np.int32), torch))
        x = torch.empty((N, C, H, Wd), dtype=torch.uint8, device="cuda")
        xs = to_dev(np.float32([0.02]), torch)
        ys = to_dev(np.float32([0.05]), torch)
        z = to_dev(np.uint8([128]), torch)
        y = torch.empty((N, M, oh, ow), dtype=torch.uint8, device="cuda")
        sets = [[r.integers(0, 256, (N, C, H, Wd)).astype(np.uint8)] for _ in range(3)]
        _graph_matches_eager(torch, [x], sets, lambda: gpu.dq_qconv_forward(h, x, xs, z, ys, z, y), [y])
    finally:
        gpu.dq_qconv_release(h)


def test_lstm_forward_replays(gpu):
    """The whole recurrence (the input projection, then one launch a step)."""
    import torch

    log("graph DynamicQuantizeLSTM")
    r = np.random.default_rng(4)
    seq, batch, ni, hd = 6, 3, 16, 8
    h = gpu.dq_lstm_init(seq, batch, ni, hd, "forward", gpu.DQ_I8, gpu.DQ_I8)
    try:
        gpu.dq_lstm_set_weights(h, to_dev(r.integers(-128, 128, (1, ni, 4 * hd)).astype(np.int8), torch),
                                to_dev(np.float32([0.01]), torch), None,
                                to_dev(r.integers(-128, 128, (1, hd, 4 * hd)).astype(np.int8), torch),
                                to_dev(np.float32([0.02]), torch), None)
        X = torch.empty((seq, batch, ni), device="cuda")
        Y = torch.empty((seq, 1, batch, hd), device="cuda")
        Yh = torch.empty((1, batch, hd), device="cuda")
        Yc = torch.empty((1, batch, hd), device="cuda")
        sets = [[r.uniform(-1, 1, (seq, batch, ni)).astype(np.float32)] for _ in range(3)]
        _graph_matches_eager(torch, [X], sets, lambda: gpu.dq_lstm_forward(h, X, Y=Y, Y_h=Yh, Y_c=Yc),
                             [Y, Yh, Yc])
    finally:
        gpu.dq_lstm_release(h)


def test_elementwise_replays(gpu):
    """QLinearAdd with a broadcast row and ReduceSumInteger over axis 0 (its
    output cleared by a kernel, then atomics)."""
    import torch

    log("graph element-wise")
    r = np.random.default_rng(5)
    u8 = dict(dtype=torch.uint8, device="cuda")
    A = torch.empty((64, 96), **u8)
    Brow = torch.empty(96, **u8)
    s = to_dev(np.float32([0.03]), torch)
    z = to_dev(np.uint8([128]), torch)
    Cout = torch.empty((64, 96), **u8)
    S = torch.empty(96, dtype=torch.int32, device="cuda")

    def run():
        gpu.qlinear_add(A, s, z, Brow, s, z, s, z, gpu.DQ_U8, Cout)
        gpu.dq_reduce_sum_integer(A, gpu.DQ_U8, [0], S)

    sets = [[r.integers(0, 256, (64, 96)).astype(np.uint8), r.integers(0, 256, 96).astype(np.uint8)]
            for _ in range(3)]
    _graph_matches_eager(torch, [A, Brow], sets, run, [Cout, S])
