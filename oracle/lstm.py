"""Reference DynamicQuantizeLSTM (CPU oracle).

TEST INFRASTRUCTURE: only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use it.

onnxruntime quantization_defs.cc, schema DynamicQuantizeLSTM (restated on the
graiphic.io DynamicQuantizeLSTM page), gives the tensors: X [seq, batch,
input] fp32; W [dirs, input, 4h] and R [dirs, hidden, 4h], 8-bit, gate blocks
in the order i, o, f, c, with scale / zero point per direction ([dirs]) or per
4h column ([dirs, 4h]); B [dirs, 8h] = (Wb, Rb); sequence_lens [batch]
int32; initial_h / initial_c [dirs, batch, h]; peepholes P [dirs, 3h] in the
order i, o, f; outputs Y [seq, dirs, batch, h], Y_h and Y_c [dirs, batch, h];
and the attributes direction, hidden_size, activations (f, g, h), their
alpha / beta, clip and input_forget. The cell equations are those of the
ONNX LSTM the schema follows. The readings this oracle takes:

R26  X W and H R are DynamicQuantizeMatMul products (R19): the fp32 operand is
     quantized per tensor to uint8, X once over the whole [seq * batch, input]
     matrix, H_{t-1} anew at every step over the whole [batch, h] matrix; the
     product is ((float)sum * a_scale) * w_scale[col] + bias[col] with bias
     Wb, resp. Rb.
R27  Per step, fp32 with one rounding per operation and no fused multiply-add:
       pre = xw[t] + hr;  pre_i += P_i * C_{t-1};  pre_f += P_f * C_{t-1}
       i = f(clip(pre_i));  f_t = 1 - i if input_forget else f(clip(pre_f))
       g = g(clip(pre_c));  C_t = f_t * C_{t-1} + i * g
       pre_o += P_o * C_t;  o = f(clip(pre_o));  H_t = o * h(C_t)
     clip(v) = min(max(v, -clip), clip) when clip > 0 (unset or <= 0 means no
     clip; the schema and the graiphic page differ on its default, both mean
     none); only the four gate inputs are clipped, not C_t. Every activation
     is evaluated in fp64 from its fp32 argument and rounded to fp32 once.
     activation_alpha / activation_beta are consumed in order by the
     activations that take the parameter; missing ones take the ONNX
     operator's default.
R28  sequence_lens: entry b with length L (0 <= L <= seq) takes steps
     s < L; at later steps its H and C are held and Y[s, d, b] is 0. The
     reverse direction feeds entry b the times t = L-1, ..., 0 (Y is written
     at time t). Y_h / Y_c are the state after the last step. A
     bidirectional LSTM runs the two directions independently, each with
     its own W, R, B, P, initial state and activations.
"""
from __future__ import annotations

import numpy as np

from . import dynamic_quantize_matmul

F32 = np.float32
F64 = np.float64

# name: (takes alpha, default alpha, takes beta, default beta), from the ONNX
# operators of the same name
ACTIVATIONS = {
    "relu": (False, None, False, None),
    "tanh": (False, None, False, None),
    "sigmoid": (False, None, False, None),
    "affine": (True, 1.0, True, 0.0),
    "leakyrelu": (True, 0.01, False, None),
    "thresholdedrelu": (True, 1.0, False, None),
    "scaledtanh": (True, 1.0, True, 1.0),
    "hardsigmoid": (True, 0.2, True, 0.5),
    "elu": (True, 1.0, False, None),
    "softsign": (False, None, False, None),
    "softplus": (False, None, False, None),
}


def activation(name, x, alpha=None, beta=None):
    """One ONNX RNN activation of an fp32 array, in fp64, rounded once (R27)."""
    n = name.lower()
    if n not in ACTIVATIONS:
        raise ValueError(f"activation {name} is not supported")
    x = np.asarray(x, F32).astype(F64)
    _, da, _, db = ACTIVATIONS[n]
    a = F64(F32(da if alpha is None else alpha)) if da is not None else None
    b = F64(F32(db if beta is None else beta)) if db is not None else None
    if n == "sigmoid":
        r = 1.0 / (1.0 + np.exp(-x))
    elif n == "tanh":
        r = np.tanh(x)
    elif n == "relu":
        r = np.maximum(x, 0.0)
    elif n == "affine":
        r = a * x + b
    elif n == "leakyrelu":
        r = np.where(x < 0, a * x, x)
    elif n == "thresholdedrelu":
        r = np.where(x > a, x, 0.0)
    elif n == "scaledtanh":
        r = a * np.tanh(b * x)
    elif n == "hardsigmoid":
        r = np.minimum(np.maximum(a * x + b, 0.0), 1.0)
    elif n == "elu":
        r = np.where(x >= 0, x, a * np.expm1(x))
    elif n == "softsign":
        r = x / (1.0 + np.abs(x))
    else:  # softplus: log(1 + exp(x)), evaluated without overflow
        r = np.logaddexp(0.0, x)
    return r.astype(F32)


def resolve_activations(activations, alphas, betas, dirs):
    """(name, alpha, beta) for f, g, h of every direction (R27)."""
    acts = ["Sigmoid", "Tanh", "Tanh"] * dirs if activations is None else list(activations)
    if len(acts) != 3 * dirs:
        raise ValueError(f"{3 * dirs} activations expected")
    al = list(alphas or [])
    be = list(betas or [])
    out = []
    for name in acts:
        n = name.lower()
        if n not in ACTIVATIONS:
            raise ValueError(f"activation {name} is not supported")
        ta, _, tb, _ = ACTIVATIONS[n]
        a = al.pop(0) if ta and al else None
        b = be.pop(0) if tb and be else None
        out.append((n, a, b))
    return out


def _per_col(v, d, n, dtype):
    a = np.asarray(v)
    row = a[d] if a.ndim == 2 else np.asarray(a[d]).reshape(1)
    return np.broadcast_to(row.astype(dtype), (n,)).copy()


def lstm(X, W, R, W_scale, W_zp, R_scale, R_zp, *, hidden_size, B=None, sequence_lens=None,
         initial_h=None, initial_c=None, P=None, direction="forward", activations=None,
         activation_alpha=None, activation_beta=None, clip=None, input_forget=0):
    """DynamicQuantizeLSTM (R26-R28). W / R: [dirs, input, 4h] / [dirs, h, 4h]
    uint8 or int8; scales fp32 and zero points of W's / R's type, [dirs] or
    [dirs, 4h]. Returns (Y, Y_h, Y_c)."""
    X = np.asarray(X, F32)
    seq, batch, nin = X.shape
    h = int(hidden_size)
    if direction not in ("forward", "reverse", "bidirectional"):
        raise ValueError("direction must be forward, reverse or bidirectional")
    dirs = 2 if direction == "bidirectional" else 1
    W = np.asarray(W)
    R = np.asarray(R)
    if W.shape != (dirs, nin, 4 * h) or R.shape != (dirs, h, 4 * h):
        raise ValueError("W or R has the wrong shape")
    lens = (np.full(batch, seq, np.int64) if sequence_lens is None
            else np.asarray(sequence_lens, np.int64))
    if lens.shape != (batch,) or (lens < 0).any() or (lens > seq).any():
        raise ValueError("sequence_lens must hold batch values in [0, seq]")
    acts = resolve_activations(activations, activation_alpha, activation_beta, dirs)
    use_clip = clip is not None and clip > 0
    cl = F32(clip) if use_clip else None
    Y = np.zeros((seq, dirs, batch, h), F32)
    Yh = np.zeros((dirs, batch, h), F32)
    Yc = np.zeros((dirs, batch, h), F32)
    for d in range(dirs):
        reverse = direction == "reverse" or d == 1
        fa, ga, ha = acts[3 * d:3 * d + 3]
        ws = _per_col(W_scale, d, 4 * h, F32)
        wz = _per_col(W_zp, d, 4 * h, np.int32)
        rs = _per_col(R_scale, d, 4 * h, F32)
        rz = _per_col(R_zp, d, 4 * h, np.int32)
        Wb = np.zeros(4 * h, F32) if B is None else np.asarray(B[d][:4 * h], F32)
        Rb = np.zeros(4 * h, F32) if B is None else np.asarray(B[d][4 * h:], F32)
        Pd = np.zeros(3 * h, F32) if P is None else np.asarray(P[d], F32)
        Pi, Po, Pf = Pd[0:h], Pd[h:2 * h], Pd[2 * h:3 * h]
        # input projection of all times at once (R26)
        xw = dynamic_quantize_matmul(X.reshape(seq * batch, nin), W[d], ws, wz, bias=Wb)
        xw = xw.reshape(seq, batch, 4 * h)
        H = np.zeros((batch, h), F32) if initial_h is None else np.array(initial_h[d], F32)
        C = np.zeros((batch, h), F32) if initial_c is None else np.array(initial_c[d], F32)
        for s in range(seq):
            hr = dynamic_quantize_matmul(H, R[d], rs, rz, bias=Rb)   # H_{t-1} R (R26)
            Hn, Cn = H.copy(), C.copy()
            for b in range(batch):
                if s >= lens[b]:
                    continue                      # held state, Y stays 0 (R28)
                t = lens[b] - 1 - s if reverse else s
                pre = xw[t, b] + hr[b]
                pi, po, pf, pc = pre[0:h], pre[h:2 * h], pre[2 * h:3 * h], pre[3 * h:]
                c0 = C[b]
                pi = pi + Pi * c0
                pf = pf + Pf * c0
                if use_clip:
                    pi, pf, pc = (np.minimum(np.maximum(v, -cl), cl) for v in (pi, pf, pc))
                ig = activation(fa[0], pi, fa[1], fa[2])
                fg = F32(1) - ig if input_forget else activation(fa[0], pf, fa[1], fa[2])
                gg = activation(ga[0], pc, ga[1], ga[2])
                c1 = fg * c0 + ig * gg
                po = po + Po * c1
                if use_clip:
                    po = np.minimum(np.maximum(po, -cl), cl)
                og = activation(fa[0], po, fa[1], fa[2])
                h1 = og * activation(ha[0], c1, ha[1], ha[2])
                Hn[b], Cn[b] = h1, c1
                Y[t, d, b] = h1
            H, C = Hn, Cn
        Yh[d], Yc[d] = H, C
    return Y, Yh, Yc
