"""GPU test of dqip_forward_noalloc, the forward that allocates nothing (its
work buffer is the library's static device scratch), against dqip_forward
with its own buffer: the same kernels on the same inputs, so C must be bit
for bit the same, on two calls in a row (the second with a smaller
problem, which reuses the scratch the first left behind), and a context
whose work buffer does not fit the scratch is refused before anything is
launched."""
import numpy as np
import pytest

import workloads as W
from gpu_case import _ACT, _DT, log, to_dev

pytestmark = pytest.mark.gpu


def _both(dq, case):
    import torch

    M, N, K = case["M"], case["N"], case["K"]
    h = dq.dqip_init(M, N, K, _DT[case["typeA"]], _DT[case["typeB"]], _DT[case["typeC"]],
                     case["constB"], case.get("bias") is not None, _ACT[case["act"]], case["avoid"])
    try:
        A = to_dev(case["A"], torch)
        B = to_dev(case["B"], torch)
        sB = to_dev(case.get("scaleB"), torch)
        bias = to_dev(case.get("bias"), torch)
        if case["constB"]:
            dq.dqip_set_params(h, B, sB, bias, None)
            Bf = None
        else:
            dq.dqip_set_params(h, None, None, bias, None)
            Bf = B
        assert dq.dqip_external_buffer_size(h) <= dq.DQIP_NOALLOC_SCRATCH_BYTES
        cdt = torch.float32 if case["typeC"] == "f32" else torch.int16
        C1 = torch.full((M, N), 7, dtype=cdt, device="cuda")
        C2 = torch.full((M, N), 9, dtype=cdt, device="cuda")
        dq.dqip_forward(h, A, Bf, None, C1)
        dq.dqip_forward_noalloc(h, A, Bf, C2)
        torch.cuda.synchronize()
        return C1.cpu().numpy(), C2.cpu().numpy()
    finally:
        dq.dqip_release(h)


def test_noalloc_matches_forward_twice_second_smaller(gpu):
    # 4096 x 3072: the 256 x 256 GEMM tile; then a non-constant B on 32 x 32 tiles
    big = W.dqip_random(4096, 3072, 512, seed=31, typeA="bf16", typeB="i8", typeC="bf16",
                        constB=True, act="relu", outliers=0.01)
    small = W.dqip_random(300, 70, 520, seed=32, typeA="f32", typeB="f32", typeC="f32",
                          constB=False, act="leaky_relu", avoid=True)
    for case in (big, small):
        log(f"dqip_forward_noalloc {case['M']}x{case['N']}x{case['K']} const:{case['constB']}")
        want, got = _both(gpu, case)
        assert np.array_equal(got, want)


def test_noalloc_refuses_a_work_buffer_beyond_the_scratch(gpu):
    import torch

    log("dqip_forward_noalloc: too large")
    h = gpu.dqip_init(4096, 64, 8192, gpu.DQ_F32, gpu.DQ_F32, gpu.DQ_F32, False, False,
                      gpu.DQ_ACT_IDENTITY, False)
    try:
        assert gpu.dqip_external_buffer_size(h) > gpu.DQIP_NOALLOC_SCRATCH_BYTES
        A = torch.zeros((4096, 8192), device="cuda")
        B = torch.zeros((8192, 64), device="cuda")
        C = torch.full((4096, 64), 5.0, device="cuda")
        with pytest.raises(gpu.DQError) as e:
            gpu.dqip_forward_noalloc(h, A, B, C)
        assert e.value.status == gpu.DQ_ERR_RANGE
        torch.cuda.synchronize()
        assert bool((C == 5.0).all())  # nothing was launched
    finally:
        gpu.dqip_release(h)
