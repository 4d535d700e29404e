"""Pins of the DynamicQuantizeLSTM oracle (readings R26-R28).

The oracle is held against things it does not compute itself: torch's LSTM
in float64 (a library routine; inputs chosen so that every dynamic
quantization is exact, else a tolerance from the quantization step with a
control that the tolerance separates a swapped gate), closed forms of tiny
cases (clip, each peephole alone), invariants that hold bit for bit
(reverse = forward on time-reversed input, bidirectional = the two
directions, a sequence = its steps chained through Y_h / Y_c, sequence_lens
= the truncated sequence, input_forget = a forget gate with negated
weights), and every activation against library functions."""
import math

import numpy as np
import pytest
import torch

from oracle import lstm as L

# gate block of i, o, f, c in the 4h axis; torch orders its blocks i, f, g(c), o
_TORCH_ORDER = (0, 2, 3, 1)


def _grid(rng, shape, z, step=2.0 ** -7):
    """fp32 values (q - z) * step whose per-tensor uint8 quantization is exact:
    the extremes q = 0 and q = 255 are present, so the scale is step and the
    zero point z."""
    q = rng.integers(0, 256, size=shape)
    flat = q.reshape(-1)
    flat[0], flat[-1] = 0, 255
    return ((q - z) * step).astype(np.float32)


def _weights(rng, dirs, rows, h, wtype, per_channel):
    if wtype == "u8":
        w = rng.integers(0, 256, size=(dirs, rows, 4 * h)).astype(np.uint8)
        zp = (rng.integers(100, 156, size=(dirs, 4 * h)) if per_channel
              else rng.integers(100, 156, size=dirs)).astype(np.uint8)
    else:
        w = rng.integers(-127, 128, size=(dirs, rows, 4 * h)).astype(np.int8)
        zp = (rng.integers(-8, 9, size=(dirs, 4 * h)) if per_channel
              else rng.integers(-8, 9, size=dirs)).astype(np.int8)
    sc = (rng.uniform(0.5, 1.5, size=(dirs, 4 * h) if per_channel else dirs)
          / (4.0 * 127 * math.sqrt(rows))).astype(np.float32)
    return w, sc, zp


def _real(w, sc, zp, d):
    """Dequantized [rows, 4h] weights of direction d in float64."""
    s = np.asarray(sc, np.float64)
    z = np.asarray(zp, np.float64)
    s, z = s[d], z[d]          # a row of [dirs, 4h], or the value of [dirs]
    return (w[d].astype(np.float64) - z) * s


def _torch_lstm(X, Wf, Rf, Wb, Rb, h, h0, c0):
    """torch.nn.LSTM in float64 with (i, o, f, c) blocks reordered to torch's."""
    nin = X.shape[2]
    m = torch.nn.LSTM(nin, h).double()
    idx = np.concatenate([np.arange(g * h, (g + 1) * h) for g in _TORCH_ORDER])
    with torch.no_grad():
        m.weight_ih_l0.copy_(torch.from_numpy(Wf[:, idx].T.copy()))
        m.weight_hh_l0.copy_(torch.from_numpy(Rf[:, idx].T.copy()))
        m.bias_ih_l0.copy_(torch.from_numpy(Wb[idx].astype(np.float64)))
        m.bias_hh_l0.copy_(torch.from_numpy(Rb[idx].astype(np.float64)))
        y, (yh, yc) = m(torch.from_numpy(X.astype(np.float64)),
                        (torch.from_numpy(h0[None].astype(np.float64)),
                         torch.from_numpy(c0[None].astype(np.float64))))
    return y.numpy(), yh[0].numpy(), yc[0].numpy()


def _case(seed, seq, batch, nin, h, wtype="i8", per_channel=True, zero_r=False, h0_grid=True):
    rng = np.random.default_rng(seed)
    X = _grid(rng, (seq, batch, nin), z=int(rng.integers(60, 200)))
    W, ws, wz = _weights(rng, 1, nin, h, wtype, per_channel)
    R, rs, rz = _weights(rng, 1, h, h, wtype, per_channel)
    if zero_r:
        R[...] = np.broadcast_to(np.asarray(rz).reshape(1, 1, -1) if np.asarray(rz).ndim == 2
                                 else np.asarray(rz).reshape(1, 1, 1), R.shape)
    B = rng.uniform(-0.5, 0.5, size=(1, 8 * h)).astype(np.float32)
    h0 = (_grid(rng, (1, batch, h), z=int(rng.integers(60, 200))) if h0_grid
          else rng.uniform(-1, 1, size=(1, batch, h)).astype(np.float32))
    c0 = rng.uniform(-1, 1, size=(1, batch, h)).astype(np.float32)
    return dict(X=X, W=W, R=R, W_scale=ws, W_zp=wz, R_scale=rs, R_zp=rz, B=B, h0=h0, c0=c0, h=h)


def _run(c, **kw):
    return L.lstm(c["X"], c["W"], c["R"], c["W_scale"], c["W_zp"], c["R_scale"], c["R_zp"],
                  hidden_size=c["h"], B=c["B"], initial_h=c["h0"], initial_c=c["c0"], **kw)


def _torch_of(c, swap_of=False):
    Wf, Rf = _real(c["W"], c["W_scale"], c["W_zp"], 0), _real(c["R"], c["R_scale"], c["R_zp"], 0)
    Wb, Rb = c["B"][0, :4 * c["h"]], c["B"][0, 4 * c["h"]:]
    if swap_of:   # a plausible mistake: the o and f blocks exchanged
        h = c["h"]
        idx = np.r_[0:h, 2 * h:3 * h, h:2 * h, 3 * h:4 * h]
        Wf, Rf, Wb, Rb = Wf[:, idx], Rf[:, idx], Wb[idx], Rb[idx]
    return _torch_lstm(c["X"], Wf, Rf, Wb, Rb, c["h"], c["h0"][0], c["c0"][0])


# ---------------------------------------------------------------- torch LSTM

@pytest.mark.parametrize("wtype", ["i8", "u8"])
@pytest.mark.parametrize("per_channel", [False, True])
def test_one_step_matches_torch_lstm(wtype, per_channel):
    """X and initial_h on an exact uint8 grid: the only differences left are
    fp32 roundings of the epilogue and the cell (a few ulps of values <= 2)."""
    c = _case(11, 1, 5, 24, 8, wtype, per_channel)
    Y, Yh, Yc = _run(c)
    ty, th, tc = _torch_of(c)
    assert np.abs(Y[:, 0] - ty).max() < 2e-6
    assert np.abs(Yh[0] - th).max() < 2e-6
    assert np.abs(Yc[0] - tc).max() < 2e-6


def test_zero_recurrent_weights_match_torch_over_many_steps():
    """R codes equal to R's zero point: H R is exactly 0 + Rb at every step, so
    a long sequence stays within fp32 rounding of torch's float64 LSTM."""
    c = _case(12, 9, 4, 16, 6, "u8", True, zero_r=True)
    Y, Yh, Yc = _run(c)
    ty, th, tc = _torch_of(c)
    assert np.abs(Y[:, 0] - ty).max() < 1e-5
    assert np.abs(Yc[0] - tc).max() < 1e-5


def test_quantized_recurrence_tracks_torch_and_separates_a_gate_swap():
    """With H quantized every step the oracle departs from float64 by about
    sqrt(h) times the rounding error of one H code (step / sqrt(12), step <=
    2/255) times |R| (~0.05), some 1e-3 at most (2.4e-4 seen); the same 2e-3
    bound fails for a plausible mistake (o and f swapped: 0.13)."""
    c = _case(13, 8, 6, 32, 16, "i8", True, h0_grid=False)
    Y, _, Yc = _run(c)
    ty, _, tc = _torch_of(c)
    err = np.abs(Y[:, 0] - ty).max()
    assert err < 2e-3
    sy, _, _ = _torch_of(c, swap_of=True)
    assert np.abs(Y[:, 0] - sy).max() > 5e-2


# ---------------------------------------------------------- closed forms

def _trivial(batch=3, h=4, seq=1, Wb=None, P=None, c0=None, clip=None, seed=3):
    """W and R codes at their zero points: X W = Wb and H R = Rb exactly."""
    rng = np.random.default_rng(seed)
    X = rng.uniform(-1, 1, size=(seq, batch, 5)).astype(np.float32)
    W = np.full((1, 5, 4 * h), 3, np.int8)
    R = np.full((1, h, 4 * h), 3, np.int8)
    sc = np.array([0.01], np.float32)
    zp = np.array([3], np.int8)
    B = np.zeros((1, 8 * h), np.float32)
    if Wb is not None:
        B[0, :4 * h] = Wb
    if c0 is None:
        c0 = rng.uniform(0.25, 1.0, size=(1, batch, h)).astype(np.float32)
    return L.lstm(X, W, R, sc, zp, sc, zp, hidden_size=h, B=B, initial_c=c0,
                  P=None if P is None else P[None], clip=clip), c0[0]


def test_tiny_clip_closed_form():
    """clip -> 0+ forces every gate input to ~0: i = f = o = 1/2, g ~ 0, so
    C_t = C_0 / 2^t exactly and H_t = 1/2 tanh(C_t) (C_t itself unclipped)."""
    rng = np.random.default_rng(4)
    h, seq = 4, 5
    Wb = rng.uniform(-3, 3, size=4 * h).astype(np.float32)
    (Y, Yh, Yc), c0 = _trivial(h=h, seq=seq, Wb=Wb, clip=1e-30)
    for t in range(seq):
        ct = c0 * np.float32(2.0 ** -(t + 1))
        ht = np.float32(0.5) * np.tanh(ct.astype(np.float64)).astype(np.float32)
        assert np.array_equal(Y[t, 0], ht)
    assert np.array_equal(Yc[0], c0 * np.float32(2.0 ** -seq))


def _sig(v):
    return 1.0 / (1.0 + math.exp(-v))


@pytest.mark.parametrize("which", ["i", "o", "f"])
def test_single_peephole_closed_form(which):
    """Zero gate products, g's bias beta, one peephole p: with C_0 = k,
    P_i: C_1 = k/2 + sig(p k) tanh(beta), H = tanh(C_1)/2;
    P_f: C_1 = sig(p k) k + tanh(beta)/2, H = tanh(C_1)/2;
    P_o: C_1 = k/2 + tanh(beta)/2, H = sig(p C_1) tanh(C_1)."""
    h = 4
    beta = 0.7
    Wb = np.zeros(4 * h, np.float32)
    Wb[3 * h:] = beta
    p = np.float32(1.3)
    P = np.zeros(3 * h, np.float32)
    P[{"i": 0, "o": 1, "f": 2}[which] * h:][:h] = p
    (Y, Yh, Yc), c0 = _trivial(h=h, Wb=Wb, P=P)
    tb = math.tanh(float(np.float32(beta)))
    for b in range(c0.shape[0]):
        for j in range(h):
            k = float(c0[b, j])
            if which == "i":
                c1 = k / 2 + _sig(float(p) * k) * tb
                h1 = 0.5 * math.tanh(c1)
            elif which == "f":
                c1 = _sig(float(p) * k) * k + tb / 2
                h1 = 0.5 * math.tanh(c1)
            else:
                c1 = k / 2 + tb / 2
                h1 = _sig(float(p) * c1) * math.tanh(c1)
            assert abs(Yc[0, b, j] - c1) < 1e-6
            assert abs(Yh[0, b, j] - h1) < 1e-6


# ---------------------------------------------------------- invariants

def _sym_case(seed, seq=6, batch=3, nin=10, h=5, dirs=1):
    """Each time slice of X holds the grid extremes, so the whole tensor and
    any run of time slices quantize with the same scale and zero point."""
    rng = np.random.default_rng(seed)
    z = 100
    q = rng.integers(0, 256, size=(seq, batch, nin))
    q[:, 0, 0], q[:, 0, 1] = 0, 255
    X = ((q - z) * 2.0 ** -7).astype(np.float32)
    W, ws, wz = _weights(rng, dirs, nin, h, "i8", True)
    R, rs, rz = _weights(rng, dirs, h, h, "i8", True)
    B = rng.uniform(-0.5, 0.5, size=(dirs, 8 * h)).astype(np.float32)
    P = rng.uniform(-0.5, 0.5, size=(dirs, 3 * h)).astype(np.float32)
    h0 = rng.uniform(-1, 1, size=(dirs, batch, h)).astype(np.float32)
    c0 = rng.uniform(-1, 1, size=(dirs, batch, h)).astype(np.float32)
    return dict(X=X, W=W, R=R, W_scale=ws, W_zp=wz, R_scale=rs, R_zp=rz, B=B, P=P, h0=h0,
                c0=c0, h=h)


def _run2(c, X=None, d=None, h0=None, c0=None, **kw):
    sl = slice(None) if d is None else slice(d, d + 1)
    return L.lstm(c["X"] if X is None else X, c["W"][sl], c["R"][sl], c["W_scale"][sl],
                  c["W_zp"][sl], c["R_scale"][sl], c["R_zp"][sl], hidden_size=c["h"],
                  B=c["B"][sl], P=c["P"][sl],
                  initial_h=c["h0"][sl] if h0 is None else h0,
                  initial_c=c["c0"][sl] if c0 is None else c0, **kw)


def test_reverse_is_forward_on_reversed_time():
    c = _sym_case(21)
    Yr, hr, cr = _run2(c, direction="reverse", clip=2.0)
    Yf, hf, cf = _run2(c, X=c["X"][::-1].copy(), clip=2.0)
    assert np.array_equal(Yr, Yf[::-1])
    assert np.array_equal(hr, hf) and np.array_equal(cr, cf)


def test_bidirectional_is_both_directions():
    c = _sym_case(22, dirs=2)
    acts = ["Sigmoid", "Tanh", "Tanh", "HardSigmoid", "Softsign", "Elu"]
    Y, Yh, Yc = _run2(c, direction="bidirectional", activations=acts,
                      activation_alpha=[0.25, 0.5], activation_beta=[0.4])
    Y0, h0, c0 = _run2(c, d=0)
    Y1, h1, c1 = _run2(c, d=1, direction="reverse", activations=acts[3:],
                       activation_alpha=[0.25, 0.5], activation_beta=[0.4])
    assert np.array_equal(Y[:, 0], Y0[:, 0]) and np.array_equal(Y[:, 1], Y1[:, 0])
    assert np.array_equal(Yh, np.concatenate([h0, h1])) and np.array_equal(Yc,
                                                                            np.concatenate([c0, c1]))


def test_sequence_is_its_steps_chained():
    c = _sym_case(23, seq=5)
    Y, Yh, Yc = _run2(c, input_forget=1)
    h, cc = c["h0"], c["c0"]
    for t in range(5):
        y1, h, cc = _run2(c, X=c["X"][t:t + 1], h0=h, c0=cc, input_forget=1)
        assert np.array_equal(Y[t], y1[0])
    assert np.array_equal(Yh, h) and np.array_equal(Yc, cc)


@pytest.mark.parametrize("direction", ["forward", "reverse"])
def test_sequence_lens_is_the_truncated_sequence(direction):
    """One entry of length Lb: its Y at times < Lb and its final state are those
    of the sequence cut to Lb; Y at later times is 0. Length 0 keeps the
    initial state."""
    c = _sym_case(24, seq=7, batch=1)
    for lb in (0, 1, 4, 7):
        Y, Yh, Yc = _run2(c, direction=direction, sequence_lens=np.array([lb], np.int32))
        assert not Y[lb:].any()
        if lb == 0:
            assert np.array_equal(Yh, c["h0"]) and np.array_equal(Yc, c["c0"])
            continue
        Yt, ht, ct = _run2(c, X=c["X"][:lb].copy(), direction=direction)
        assert np.array_equal(Y[:lb], Yt)
        assert np.array_equal(Yh, ht) and np.array_equal(Yc, ct)


def test_sequence_lens_in_a_batch_is_the_truncated_batch():
    """A batch with lengths (6, 3, 0, 5) agrees over its first three times with
    the batch cut to three times and lengths (3, 3, 0, 3) (the entries share
    H's quantization, so held rows must be held in both); finished entries
    hold their state and leave zeros in Y; length 0 keeps the initial state."""
    c = _sym_case(25, seq=6, batch=4)
    lens = np.array([6, 3, 0, 5], np.int32)
    Y, Yh, Yc = _run2(c, sequence_lens=lens)
    Yt, ht, ct = _run2(c, X=c["X"][:3].copy(), sequence_lens=np.array([3, 3, 0, 3], np.int32))
    assert np.array_equal(Y[:3], Yt)
    assert np.array_equal(Yh[:, 1], ht[:, 1]) and np.array_equal(Yc[:, 1], ct[:, 1])
    assert np.array_equal(Yh[:, 2], c["h0"][:, 2]) and np.array_equal(Yc[:, 2], c["c0"][:, 2])
    for b, lb in enumerate(lens):
        assert not Y[lb:, :, b].any()
        if lb:
            assert np.array_equal(Yh[:, b], Y[lb - 1, :, b])


def test_per_channel_with_equal_columns_is_per_tensor():
    c = _sym_case(26)
    c2 = dict(c)
    h = c["h"]
    for k in ("W", "R"):
        c2[k + "_scale"] = np.full((1, 4 * h), c[k + "_scale"][0, 0], np.float32)
        c2[k + "_zp"] = np.full((1, 4 * h), c[k + "_zp"][0, 0], np.int8)
    c1 = dict(c2)
    c1["W_scale"], c1["W_zp"] = c2["W_scale"][:, 0], c2["W_zp"][:, 0]
    c1["R_scale"], c1["R_zp"] = c2["R_scale"][:, 0], c2["R_zp"][:, 0]
    a = _run2(c2)
    b = _run2(c1)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_input_forget_is_a_negated_input_gate():
    """sigmoid(-x) = 1 - sigmoid(x): a forget gate whose codes, biases and
    peephole are the input gate's negated gives f = 1 - i up to rounding."""
    c = _sym_case(27)
    h = c["h"]
    for k in ("W", "R"):            # codes lie in [-127, 127]: negation is exact
        w = c[k].copy()
        w[..., 2 * h:3 * h] = -w[..., 0:h]
        c[k] = w
        c[k + "_scale"][:, 2 * h:3 * h] = c[k + "_scale"][:, 0:h]
        c[k + "_zp"][:, 2 * h:3 * h] = -c[k + "_zp"][:, 0:h]
    c["B"][:, 2 * h:3 * h] = -c["B"][:, 0:h]
    c["B"][:, 6 * h:7 * h] = -c["B"][:, 4 * h:5 * h]
    c["P"][:, 2 * h:3 * h] = -c["P"][:, 0:h]
    Y0, h0, c0 = _run2(c, input_forget=0, sequence_lens=np.array([1, 1, 1], np.int32))
    Y1, h1, c1 = _run2(c, input_forget=1, sequence_lens=np.array([1, 1, 1], np.int32))
    assert np.abs(Y0 - Y1).max() < 1e-6 and np.abs(c0 - c1).max() < 1e-6


# ---------------------------------------------------------- activations

def _f32(v):
    """An fp32 attribute value, as the operator receives it."""
    return float(np.float32(v))


_X = np.array([-30, -5.5, -1, -0.25, -1e-8, 0, 1e-8, 0.3, 1, 2.5, 7, 30], np.float32)


@pytest.mark.parametrize("name,lib", [
    ("sigmoid", lambda x: torch.sigmoid(x)),
    ("tanh", lambda x: torch.tanh(x)),
    ("relu", lambda x: torch.relu(x)),
    ("leakyrelu", lambda x: torch.nn.functional.leaky_relu(x, _f32(0.01))),
    ("elu", lambda x: torch.nn.functional.elu(x, 1.0)),
    ("softsign", lambda x: torch.nn.functional.softsign(x)),
    ("softplus", lambda x: torch.nn.functional.softplus(x, threshold=1e9)),
    ("hardsigmoid", lambda x: torch.clamp(_f32(0.2) * x + 0.5, 0, 1)),
    ("thresholdedrelu", lambda x: torch.where(x > 1.0, x, torch.zeros_like(x))),
    ("scaledtanh", lambda x: torch.tanh(x)),
    ("affine", lambda x: x),
])
def test_activation_defaults_against_library(name, lib):
    ref = lib(torch.from_numpy(_X.astype(np.float64))).numpy().astype(np.float32)
    got = L.activation(name, _X)
    assert np.array_equal(got, ref), (name, got, ref)


def test_activation_parameters_are_consumed_in_order():
    r = L.resolve_activations(["LeakyRelu", "Tanh", "HardSigmoid"], [0.1, 0.3], [0.4], 1)
    assert r == [("leakyrelu", 0.1, None), ("tanh", None, None), ("hardsigmoid", 0.3, 0.4)]
    r = L.resolve_activations(["Affine", "ScaledTanh", "Elu"], [2.0], None, 1)
    assert r == [("affine", 2.0, None), ("scaledtanh", None, None), ("elu", None, None)]
    x = np.float32(0.75)
    assert L.activation("scaledtanh", x, 2.0, 0.5) == np.float32(2.0 * math.tanh(0.375))
    assert L.activation("hardsigmoid", np.float32(-4), 0.3, 0.4) == 0


def test_rejects_bad_arguments():
    c = _sym_case(28)
    with pytest.raises(ValueError):
        _run2(c, direction="sideways")
    with pytest.raises(ValueError):
        _run2(c, sequence_lens=np.array([7, 1, 1], np.int32))
    with pytest.raises(ValueError):
        _run2(c, activations=["Sigmoid", "Tanh"])
    with pytest.raises(ValueError):
        _run2(c, activations=["Sigmoid", "Tanh", "Gelu"])
