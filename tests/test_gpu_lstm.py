"""GPU parity of DynamicQuantizeLSTM against the CPU oracle (readings R26-R28).

Both sides quantize X and every H_{s-1} per tensor with the same fp32 rule,
sum integers exactly and round each fp32 operation once in the same order;
each activation is evaluated in fp64 and rounded once (the library's fp64
exp and its tanh, accurate to a few fp64 units, differ from the host's in
the last bits, which can move an fp32 result by one unit only when the exact
value lies within a few 2^-52 of an fp32 rounding midpoint). So the outputs
agree to fp32 rounding: |got - want| <= 1e-6 + 1e-5 |want| (the fp32 bar),
and in practice bit for bit (the test reports how many values differ).

Cases: the gate-projection workload at full size (seq 128, batch 32, input
and hidden 512), forward / reverse / bidirectional, int8 and uint8 W and R
with per-tensor or per-column scales and zero points, sequence_lens with
zeros and ragged lengths, batch over one 32-entry tile, hidden sizes that
are not a multiple of 8 or 16 (ragged unit tiles, the scalar H loader), a
hidden size whose K runs over several fragment chunks, the largest hidden
size (4096, 128 KiB of LDS), peepholes, clip, input_forget, every
non-default activation with alpha / beta, missing optional inputs,
degenerate sizes (one hidden unit and one input feature, one entry and one
step, a lone entry of length 0), an empty sequence and an empty batch, and
a context run twice.
"""
import zlib

import numpy as np
import pytest

import workloads
from gpu_case import log
from oracle import lstm as L

pytestmark = pytest.mark.gpu


def _seed(*key):
    return zlib.crc32(repr(key).encode())


def _gpu_lstm(dq, c, *, activations=None, alpha=None, beta=None, clip=None, input_forget=0, repeat=1):
    import torch

    X = c["X"]
    seq, batch, nin = X.shape
    h = c["hidden"]
    dirs = 2 if c["direction"] == "bidirectional" else 1
    T = {np.dtype(np.uint8): dq.DQ_U8, np.dtype(np.int8): dq.DQ_I8}
    dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    ctx = dq.dq_lstm_init(seq, batch, nin, h, c["direction"], T[c["W"].dtype], T[c["R"].dtype],
                          activations, alpha, beta, clip or 0.0, input_forget)
    try:
        dq.dq_lstm_set_weights(ctx, dev(c["W"]), dev(c["W_scale"]), dev(c["W_zp"]), dev(c["R"]),
                               dev(c["R_scale"]), dev(c["R_zp"]), dev(c["B"]), dev(c["P"]))
        Xd, lens = dev(X), dev(c["sequence_lens"])
        h0, c0 = dev(c["initial_h"]), dev(c["initial_c"])
        outs = []
        for _ in range(repeat):
            Y = torch.full((seq, dirs, batch, h), float("nan"), device="cuda")
            Yh = torch.full((dirs, batch, h), float("nan"), device="cuda")
            Yc = torch.full((dirs, batch, h), float("nan"), device="cuda")
            dq.dq_lstm_forward(ctx, Xd, lens, h0, c0, Y, Yh, Yc)
            torch.cuda.synchronize()
            outs.append((Y.cpu().numpy(), Yh.cpu().numpy(), Yc.cpu().numpy()))
        return outs, dq.dq_lstm_info(ctx)
    finally:
        dq.dq_lstm_release(ctx)


def _oracle(c, **kw):
    return L.lstm(c["X"], c["W"], c["R"], c["W_scale"], c["W_zp"], c["R_scale"], c["R_zp"],
                  hidden_size=c["hidden"], B=c["B"], sequence_lens=c["sequence_lens"],
                  initial_h=c["initial_h"], initial_c=c["initial_c"], P=c["P"],
                  direction=c["direction"], **kw)


def _compare(got, want, info):
    for name, g, w in zip(("Y", "Y_h", "Y_c"), got, want):
        assert g.shape == w.shape, (name, g.shape, w.shape)
        assert np.isfinite(g).all(), f"{name}: values left unwritten ({info})"
        err = np.abs(g.astype(np.float64) - w)
        bound = 1e-6 + 1e-5 * np.abs(w)
        log(f"  {name}: {int((g != w).sum())} of {g.size} differ, max |err| {err.max():.3g}")
        assert (err <= bound).all(), f"{name}: {(err > bound).sum()} beyond the fp32 bar ({info})"


def _check(dq, c):
    want = _oracle(c)
    (got,), info = _gpu_lstm(dq, c)
    log(f"  {info}")
    _compare(got, want, info)


CASES = {
    # name: (seq, batch, input, hidden, generator options, attributes)
    "tiny": (5, 3, 12, 8, {}, {}),
    "ragged_units_reverse_u8": (7, 5, 20, 13, dict(direction="reverse", w_type="u8", r_type="u8",
                                                   zero_points=True, lens=[7, 0, 3, 7, 1]), {}),
    "bidirectional_two_batch_tiles": (6, 40, 33, 24, dict(direction="bidirectional", peepholes=True,
                                                          lens=[6, 2, 0, 5] * 10), dict(clip=1.5)),
    "per_tensor_mixed_types": (9, 7, 64, 48, dict(w_type="u8", r_type="i8", per_channel=False,
                                                  zero_points=True), {}),
    "no_optional_inputs": (4, 6, 10, 20, dict(bias=False, initial=False), {}),
    "scalar_loader_h20": (5, 33, 17, 20, dict(peepholes=True, w_type="i8", r_type="u8"), {}),
    "k_chunks_h1100": (3, 4, 16, 1100, dict(zero_points=True), {}),
    "activations_input_forget": (6, 4, 16, 32, dict(peepholes=True),
                                 dict(activations=["HardSigmoid", "Softsign", "Elu"], alpha=[0.3, 0.7],
                                      beta=[0.45], input_forget=1)),
    "activations_bidirectional": (5, 3, 12, 16, dict(direction="bidirectional"),
                                  dict(activations=["Sigmoid", "ScaledTanh", "Softplus", "Affine", "Tanh",
                                                    "LeakyRelu"],
                                       alpha=[0.8, 0.9, 0.05], beta=[1.3, -0.1])),
    "activations_relu_thresholded": (4, 2, 8, 16, {}, dict(activations=["Sigmoid", "Relu", "ThresholdedRelu"],
                                                           alpha=[0.2], clip=3.0)),
    # degenerate sizes: one unit, one input feature, one batch entry, one step
    "hidden_1_input_1": (4, 3, 1, 1, dict(direction="bidirectional", peepholes=True), {}),
    "batch_1_seq_1": (1, 1, 5, 7, dict(w_type="u8", r_type="u8", zero_points=True), {}),
    "one_entry_length_0": (3, 1, 6, 9, dict(direction="reverse", lens=[0]), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_lstm_matches_oracle(gpu, name):
    seq, batch, nin, h, opts, attrs = CASES[name]
    c = workloads.lstm_case(seq, batch, nin, h, seed=_seed(name), **opts)
    log(f"lstm {name}: seq {seq} batch {batch} input {nin} hidden {h} {opts} {attrs}")
    kw = dict(attrs)
    # the ONNX attribute names of the oracle
    okw = {"activations": kw.get("activations"), "activation_alpha": kw.get("alpha"),
           "activation_beta": kw.get("beta"), "clip": kw.get("clip"),
           "input_forget": kw.get("input_forget", 0)}
    want = _oracle(c, **okw)
    outs, info = _gpu_lstm(gpu, c, repeat=2, **kw)
    log(f"  {info}")
    for got in outs:
        _compare(got, want, info)
    for a, b in zip(outs[1], outs[0]):
        assert np.array_equal(a, b), "a second forward on one context differs"


@pytest.mark.parametrize("direction", ["forward", "bidirectional"])
def test_lstm_gate_projection_workload_full_size(gpu, direction):
    """seq 128, batch 32, input 512, hidden 512, per-column int8 W and R:
    the timed workload in both directions, with its seed and arguments."""
    c = workloads.lstm_case(direction=direction)
    log(f"lstm full size {direction}: seq 128 batch 32 input 512 hidden 512")
    _check(gpu, c)


def test_lstm_largest_hidden_size(gpu):
    c = workloads.lstm_case(2, 3, 8, gpu.DQ_LSTM_HIDDEN_MAX, seed=_seed("hmax"), zero_points=True)
    log("lstm hidden 4096")
    _check(gpu, c)


def test_lstm_empty_sequence_returns_the_initial_state(gpu):
    import torch

    c = workloads.lstm_case(1, 3, 8, 16, seed=_seed("empty"), direction="bidirectional")
    h0 = torch.from_numpy(c["initial_h"]).cuda()
    c0 = torch.from_numpy(c["initial_c"]).cuda()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    ctx = gpu.dq_lstm_init(0, 3, 8, 16, "bidirectional", gpu.DQ_I8, gpu.DQ_I8)
    try:
        gpu.dq_lstm_set_weights(ctx, dev(c["W"]), dev(c["W_scale"]), None, dev(c["R"]), dev(c["R_scale"]),
                                None)
        Yh = torch.full_like(h0, float("nan"))
        Yc = torch.full_like(c0, float("nan"))
        gpu.dq_lstm_forward(ctx, None, None, h0, c0, None, Yh, Yc)
        torch.cuda.synchronize()
        assert torch.equal(Yh, h0) and torch.equal(Yc, c0)
    finally:
        gpu.dq_lstm_release(ctx)
    ctx = gpu.dq_lstm_init(4, 0, 8, 16, "forward", gpu.DQ_I8, gpu.DQ_I8)  # empty batch: nothing to do
    try:
        gpu.dq_lstm_set_weights(ctx, dev(c["W"][:1]), dev(c["W_scale"][:1]), None, dev(c["R"][:1]),
                                dev(c["R_scale"][:1]), None)
        gpu.dq_lstm_forward(ctx, None, None, None, None, None, None, None)
        torch.cuda.synchronize()
    finally:
        gpu.dq_lstm_release(ctx)


def test_lstm_lengths_beyond_the_sequence_are_clamped(gpu):
    """A length above seq acts as seq and a negative one as 0 (the library
    clamps device-side lengths instead of reading outside X or Y)."""
    c = workloads.lstm_case(4, 3, 8, 16, seed=_seed("clamp"), direction="reverse", lens=[9, -2, 4])
    okw = dict(c)
    okw["sequence_lens"] = np.array([4, 0, 4], np.int32)
    want = _oracle(okw)
    (got,), info = _gpu_lstm(gpu, c)
    _compare(got, want, info)


_PLAIN_ACTS = ["Sigmoid", "Tanh", "Relu", "Softsign", "Softplus"]


def _random_lstm_cases(seed, n):
    """Seeded random cases: sequence 1-12, batch 1-70 (over the 32-entry
    tiles), input 1-200, hidden 1-300 (ragged against the 8-unit tiles),
    every direction, int8 or uint8 W and R, per-direction or per-column
    scales, zero points, bias, peepholes, initial state and sequence_lens
    (zero and ragged lengths) each on or off, clip, input_forget, and the
    activations drawn from those without alpha / beta."""
    r = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        seq, batch = int(r.integers(1, 13)), int(r.integers(1, 71))
        direction = ["forward", "reverse", "bidirectional"][int(r.integers(3))]
        opts = dict(direction=direction, w_type=["i8", "u8"][int(r.integers(2))],
                    r_type=["i8", "u8"][int(r.integers(2))], per_channel=bool(r.integers(2)),
                    zero_points=bool(r.integers(2)), bias=bool(r.integers(4)), peepholes=bool(r.integers(2)),
                    initial=bool(r.integers(2)),
                    lens=(None if r.integers(2) else [int(v) for v in r.integers(0, seq + 1, batch)]))
        attrs = {}
        if r.integers(3) == 0:
            nact = 6 if direction == "bidirectional" else 3
            attrs["activations"] = [_PLAIN_ACTS[int(i)] for i in r.integers(0, len(_PLAIN_ACTS), nact)]
        if r.integers(3) == 0:
            attrs["clip"] = float(r.uniform(0.5, 3.0))
        if r.integers(4) == 0:
            attrs["input_forget"] = 1
        out.append(dict(seq=seq, batch=batch, nin=int(r.integers(1, 201)), h=int(r.integers(1, 301)),
                        opts=opts, attrs=attrs, seed=int(r.integers(1 << 30))))
    return out


@pytest.mark.parametrize("p", _random_lstm_cases(2032, 20),
                         ids=lambda p: f"s{p['seq']}b{p['batch']}i{p['nin']}h{p['h']}-{p['opts']['direction']}")
def test_lstm_random_cases(gpu, p):
    """Y, Y_h and Y_c within the fp32 bar of the oracle on seeded random cases."""
    c = workloads.lstm_case(p["seq"], p["batch"], p["nin"], p["h"], seed=p["seed"], **p["opts"])
    log(f"lstm random seq {p['seq']} batch {p['batch']} input {p['nin']} hidden {p['h']} {p['opts']} {p['attrs']}")
    kw = dict(p["attrs"])
    want = _oracle(c, activations=kw.get("activations"), activation_alpha=None, activation_beta=None,
                   clip=kw.get("clip"), input_forget=kw.get("input_forget", 0))
    (got,), info = _gpu_lstm(gpu, c, **kw)
    log(f"  {info}")
    _compare(got, want, info)
