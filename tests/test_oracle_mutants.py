"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them.  This is what makes the pins worth trusting:
a dropped term, a wrong sign or index, or a transposed operand anywhere in the
oracle fails at least one pin."""
import importlib.util
import os
import sys
import types

import pytest

import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "retention.py")

# (name, original text, planted mistake)
MUTANTS = [
    ("rotation sign", "out[..., 0::2] = xe * c - xo * s", "out[..., 0::2] = xe * c + xo * s"),
    ("rotation pair swap", "out[..., 1::2] = xe * s + xo * c", "out[..., 1::2] = xo * s + xe * c * 0.999"),
    ("dropped chunk carry", "+ gB * R\n", "+ R\n"),
    ("xi off by one", "(j[None, :] + 1.0)", "(j[None, :] + 0.0)"),
    ("zeta off by one", "(Bc - j[None, :] - 1.0)", "(Bc - j[None, :])"),
    ("transposed scores", "P = (Qc @ np.swapaxes(Kc, -1, -2))", "P = (Kc @ np.swapaxes(Qc, -1, -2))"),
    ("drow missing sqrt", "s = s * np.sqrt((1.0 - gamma[:, None]) / (1.0 - gamma[:, None] ** n[None, :]))",
     "s = s * ((1.0 - gamma[:, None]) / (1.0 - gamma[:, None] ** n[None, :]))"),
    ("drow count off by one", "n_prev + c0 + j + 1)", "n_prev + c0 + j)"),
    ("score norm without abs", "np.maximum(np.abs(den * s[None, :, :]), 1.0)", "np.maximum(den * s[None, :, :], 1.0)"),
    ("dropped key-sum term", "z = g3 * z + kp", "z = g3 * z"),
    ("chunk key-sum no decay", "+ gB[..., 0] * z", "+ z"),
    ("unbiased GN variance", "var = ((yt - mu) ** 2).mean(axis=-1, keepdims=True)",
     "var = ((yt - mu) ** 2).sum(axis=-1, keepdims=True) / (dv - 1)"),
    ("swish sign", "x / (1.0 + np.exp(-x))", "x / (1.0 + np.exp(x))"),
    ("scale by d_k", "s = s / np.sqrt(d_k)", "s = s / d_k"),
    ("anti-causal mask", "diff = n[:, None] - n[None, :]", "diff = n[None, :] - n[:, None]"),
    ("decode without decay", "S = gamma[None, :, None, None] * S + k[:, :, :, None]", "S = S + k[:, :, :, None]"),
    ("gamma exponent", "2.0 ** (-5.0 - np.arange", "2.0 ** (-4.0 - np.arange"),
    ("recurrent reads state before update", "        num = np.einsum('bhd,bhde->bhe', qp, S)\n",
     "        num = np.einsum('bhd,bhde->bhe', qp, S - kp[:, :, :, None] * v[:, :, p, None, :])\n"),
    ("heads interleaved", "np.transpose(x.reshape(b, L, h, hd // h), (0, 2, 1, 3))",
     "np.transpose(x.reshape(b, L, hd // h, h), (0, 3, 1, 2))"),
    ("block W_Q and W_K swapped", "    Q = split_heads(X @ _f64(WQ), h)\n    K = split_heads(X @ _f64(WK), h)\n",
     "    Q = split_heads(X @ _f64(WK), h)\n    K = split_heads(X @ _f64(WQ), h)\n"),
    ("gate after W_O", "out = gate_norm(Y, G, eps) @ _f64(WO)",
     "out = (group_norm_heads(Y, eps) @ _f64(WO)) * swish(G[..., :WO.shape[1]])"),
    ("unbiased LN variance", "var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)",
     "var = ((x - mu) ** 2).sum(axis=-1, keepdims=True) / (x.shape[-1] - 1)"),
    ("gelu tanh approximation", "return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))",
     "return 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))"),
    ("FFN without gelu", "return gelu(_f64(X) @ _f64(W1)) @ _f64(W2)", "return (_f64(X) @ _f64(W1)) @ _f64(W2)"),
    ("layer without the first LN", "m, st = msr_forward(layer_norm(X, ln_eps, *ln1),", "m, st = msr_forward(X,"),
    ("layer drops the MSR residual", "    Y = m + X\n", "    Y = m\n"),
    ("layer drops the FFN residual", "out = ffn(layer_norm(Y, ln_eps, *ln2), W1, W2) + Y",
     "out = ffn(layer_norm(Y, ln_eps, *ln2), W1, W2) + X"),
    ("decode heads transposed", "Q.reshape(b, h, dk), K.reshape(b, h, dk)",
     "Q.reshape(b, dk, h).transpose(0, 2, 1), K.reshape(b, dk, h).transpose(0, 2, 1)"),
    ("decode second LN on the layer input", "x = ffn(layer_norm(y, ln_eps, *ln2), W1, W2) + y",
     "x = ffn(layer_norm(x, ln_eps, *ln2), W1, W2) + y"),
    ("decode shares one state across layers", "zip(layers, states)", "zip(layers, [states[0]] * len(states))"),
    ("backward clamp gradient sign", "gden = np.where(active, -(s ** 2)", "gden = np.where(active, (s ** 2)"),
    ("backward clamp gradient missing a scale", "gden = np.where(active, -(s ** 2)", "gden = np.where(active, -(s ** 1)"),
    ("backward dk from the untransposed scores", "dkr = np.swapaxes(dS, -1, -2) @ q", "dkr = dS @ q"),
    ("backward without the inverse rotation", "dkr = xpos_rotate(dkr, -pos, theta)", "dkr = xpos_rotate(dkr, pos, theta)"),
    ("backward dv ignores the normaliser", "gnum = (s / nrm)[..., None] * g", "gnum = s[..., None] * g"),
    ("stack drops the carried state", "n_prev=n_prev, state=None if states is None else states[i]",
     "n_prev=n_prev, state=None"),
]


def _load_mutant(name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor for '{name}' not found in the oracle"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new):
    mod = _load_mutant(name, old, new)
    pins = [P.quick_forms] + [p for p in P.ALL_PINS if p is not P.pin_forms_agree]
    caught = []
    for pin in pins:
        try:
            pin(mod)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake '{name}'"
