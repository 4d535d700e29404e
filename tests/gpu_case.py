"""Helpers of the GPU parity tests: run a workload case (a dict made by
``workloads``) through the C ABI and read back every intermediate, and
compare float outputs to the oracle's at the stated tolerances."""
from __future__ import annotations

import numpy as np

_DT = {"f32": 0, "bf16": 1, "i8": 2, "u8": 3}
_ACT = {"identity": 0, "relu": 1, "leaky_relu": 2}


def log(msg):
    print(msg, flush=True)


def to_dev(a, torch):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def run_dqip(dq, case, *, ext_buf=False, accumulators=True, inspect=True, ctx=None,
             keep_ctx=False, repeat=1, a_offset=0):
    """Init + set_params + forward (and accumulators / inspection).
    a_offset: A placed that many bytes past a 256-byte aligned allocation
    (a multiple of its element size), to reach the paths for unaligned A.
    Returns a dict of numpy arrays."""
    import torch

    M, N, K = case["M"], case["N"], case["K"]
    h = dq.dqip_init(M, N, K, _DT[case["typeA"]], _DT[case["typeB"]], _DT[case["typeC"]],
                     case["constB"], case.get("bias") is not None or case.get("has_bias", False),
                     _ACT[case["act"]], case["avoid"], ctx=ctx)
    out = {}
    try:
        A = to_dev(case["A"], torch)
        if a_offset:
            es = A.element_size()
            assert a_offset % es == 0
            flat = torch.zeros(A.numel() + a_offset // es, dtype=A.dtype, device="cuda")
            flat[a_offset // es:] = A.reshape(-1)
            A = flat[a_offset // es:].view(A.shape)
            assert A.data_ptr() % 16 == a_offset % 16
        B = to_dev(case["B"], torch)
        sB = to_dev(case.get("scaleB"), torch)
        bias = to_dev(case.get("bias"), torch)
        params = [float(case.get("alpha", 0.01))] if case["act"] == "leaky_relu" else None
        if case["constB"]:
            dq.dqip_set_params(h, B, sB, bias, params)
            Bfwd = None
        else:
            dq.dqip_set_params(h, None, None, bias, params)
            Bfwd = B
        buf = None
        if ext_buf:
            nbytes = dq.dqip_external_buffer_size(h)
            buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        cdt = torch.float32 if case["typeC"] == "f32" else torch.int16
        Cg = torch.empty((M, N), dtype=cdt, device="cuda")
        for _ in range(repeat):
            dq.dqip_forward(h, A, Bfwd, buf, Cg)
        torch.cuda.synchronize()
        out["C"] = Cg.cpu().numpy()
        if case["typeC"] == "bf16":
            out["C"] = out["C"].view(np.uint16)
        if inspect:
            uA = torch.empty((M, K), dtype=torch.uint8, device="cuda")
            sA = torch.empty(M, dtype=torch.float32, device="cuda")
            zA = torch.empty(M, dtype=torch.int32, device="cuda")
            dq.dqip_read_quantized_a(h, buf, uA, sA, zA)
            iB = torch.empty((K, N), dtype=torch.int8, device="cuda")
            sBo = torch.empty(N, dtype=torch.float32, device="cuda")
            cs = torch.empty(N, dtype=torch.int32, device="cuda")
            dq.dqip_read_quantized_b(h, buf, iB, sBo, cs)
            torch.cuda.synchronize()
            out.update(uA=uA.cpu().numpy(), scaleA=sA.cpu().numpy(), zeroA=zA.cpu().numpy(),
                       iB=iB.cpu().numpy(), scaleB=sBo.cpu().numpy(), colsumB=cs.cpu().numpy())
        if accumulators:
            acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
            dq.dqip_forward_accumulators(h, A, Bfwd, buf, acc)
            torch.cuda.synchronize()
            out["acc"] = acc.cpu().numpy()
        out["info"] = dq.dqip_info(h)
        out["internal_bytes"] = dq.dqip_internal_buffer_size(h)
    finally:
        if keep_ctx:
            out["ctx"] = h
        else:
            dq.dqip_release(h)
    return out


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in units in the last place between two bf16 bit arrays (the
    bit patterns mapped onto a monotone integer line)."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, 0x8000 - (b & 0x7FFF), 0x8000 + (b & 0x7FFF))
    return np.abs(ordered(a_bits) - ordered(b_bits))


def assert_close_c(got, want, typeC, bias=None, rtol=1e-5):
    """fp32: |got - want| <= rtol * (|want| + |bias|); bf16: <= 1 ulp."""
    if typeC == "bf16":
        d = bf16_ulp_diff(got, want)
        assert d.max() <= 1, f"bf16 outputs differ by {d.max()} ulp at {np.argmax(d)}"
        return int((d == 0).mean() * 100)
    ref = np.abs(want.astype(np.float64))
    if bias is not None:
        ref = ref + np.abs(bias.astype(np.float64))[None, :]
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    ok = err <= rtol * ref + 1e-30
    assert ok.all(), (f"{(~ok).sum()} fp32 outputs beyond {rtol} relative; worst "
                      f"{(err / np.maximum(ref, 1e-30)).max():.3g}")
    return int((got == want).mean() * 100)


def tile_rows(M, seed, tile=256):
    """Rows to check at full size: two from every `tile`-row block (one at a
    position that moves through the block from block to block, so that
    successive blocks hit different waves, 32-row strips and lanes of a
    256-row GEMM tile, and one drawn at random), plus the first and last
    row. A row of C depends only on its row of A, so the oracle can compute
    exactly these rows."""
    r = np.random.default_rng(seed)
    rows = [0, M - 1]
    for t in range((M + tile - 1) // tile):
        lo, hi = t * tile, min(M, (t + 1) * tile)
        rows.append(lo + (37 * t + 11 * seed) % (hi - lo))
        rows.append(int(r.integers(lo, hi)))
    return np.unique(np.array(rows, np.int64))
