"""Parity of a stack of RetNet layers (reading notes §三.4) with the fp64
oracle: the chunkwise forward of the stack with its per-layer states handed to
the token-by-token decode (recurrent form, §2.2), and one decode step of a
layer at the decode workload's shape (batch 128, d_model 4096, 16 heads of
256 / 512, FFN 16384) on sampled sequences."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, announce, check, check_bf16_out, dev, f64, host64
from linear_attention_sequence_retention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from linear_attention_sequence_retention_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return binding


def _vec(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _layers(cfg, n_layers, seed):
    """Per layer: device weights for the binding and fp64 copies for the oracle."""
    dev_layers, ref_layers = [], []
    for i in range(n_layers):
        msr_w, W1, W2, ln1, ln2 = W.layer_inputs(**cfg, seed=seed + i)
        dT = lambda w: dev(np.ascontiguousarray(w.T), "bf16")
        dev_layers.append((tuple(dT(w) for w in msr_w[1:]), dT(W1), dT(W2), (_vec(ln1[0]), _vec(ln1[1])),
                           (_vec(ln2[0]), _vec(ln2[1]))))
        ref_layers.append((tuple(f64(w, "bf16") for w in msr_w[1:]), f64(W1, "bf16"), f64(W2, "bf16"), ln1, ln2))
    return dev_layers, ref_layers


SMALL = dict(b=2, L=40, d_model=256, h=2, dk=128, dv=256, d_ff=512, x_sigma=1.0, w_sigma=0.05, ln_sigma=0.1,
             ln_eps=1e-5, chunk=16)


@pytest.mark.parametrize("flags,x_dtype", [(W.XPOS | W.NORM_ALL, "f32"), (W.XPOS, "f32"), (W.XPOS | W.NORM_ALL, "bf16")])
def test_stack_prefill_then_decode(R, flags, x_dtype):
    cfg, n_layers, P = SMALL, 2, 32
    b, T, h, dk, dv = cfg["b"], cfg["L"], cfg["h"], cfg["dk"], cfg["dv"]
    dl, rl = _layers(cfg, n_layers, seed=11)
    rng = np.random.default_rng(5)
    Xb = W.draw(rng, (b, T, cfg["d_model"]), 1.0, "bf16")
    X = W.as_f32(Xb, "bf16")
    xin = (lambda a: dev(np.ascontiguousarray(a), "bf16")) if x_dtype == "bf16" else (lambda a: dev(a, "f32"))
    src = Xb if x_dtype == "bf16" else X
    th, g = W.theta_vector(dk), W.gamma_vector(h)
    announce(f"stack {n_layers} layers prefill {P} then decode {T - P} flags {flags} x {x_dtype}")
    ref = oracle.retnet_stack(X.astype(np.float64), rl, h, th, flags, cfg["chunk"], 1e-5, 1e-5)
    states = R.new_states(n_layers, b, h, dk, dv)
    pre = R.retnet_stack_fwd(xin(src[:, :P]), dl, g, th, cfg["chunk"], flags, 1e-5, 1e-5, states_out=states)
    outs = []
    for t in range(P, T):
        outs.append(R.retnet_decode_step(xin(src[:, t]), dl, states, g, th, t, t + 1, flags, 1e-5, 1e-5))
    torch.cuda.synchronize()
    chk = check_bf16_out if x_dtype == "bf16" else check
    chk(f"stack prefill {P} tokens x {x_dtype}", host64(pre), ref[:, :P], TOL["bf16"])
    dec = np.stack([host64(o) for o in outs], axis=1)
    chk(f"stack decode tokens {P}..{T - 1} after prefill x {x_dtype}", dec, ref[:, P:], TOL["bf16"])


def test_stack_decode_from_empty(R):
    cfg, n_layers, T = SMALL, 2, 6
    b, h, dk, dv = cfg["b"], cfg["h"], cfg["dk"], cfg["dv"]
    flags = W.XPOS | W.NORM_ALL
    dl, rl = _layers(cfg, n_layers, seed=21)
    rng = np.random.default_rng(6)
    X = W.draw(rng, (b, T, cfg["d_model"]), 1.0, "bf16")
    th, g = W.theta_vector(dk), W.gamma_vector(h)
    announce(f"stack {n_layers} layers decode {T} tokens from an empty state, bf16 x")
    ref = oracle.retnet_stack(f64(X, "bf16"), rl, h, th, flags, 4, 1e-5, 1e-5)
    states = R.new_states(n_layers, b, h, dk, dv)
    outs = [R.retnet_decode_step(dev(np.ascontiguousarray(X[:, t]), "bf16"), dl, states, g, th, t, t + 1, flags,
                                 1e-5, 1e-5) for t in range(T)]
    torch.cuda.synchronize()
    assert outs[0].dtype == torch.bfloat16
    dec = np.stack([host64(o) for o in outs], axis=1)
    check_bf16_out("stack decode from empty (bf16 out)", dec, ref, TOL["bf16"])


def test_decode_layer_full_shape_sampled(R):
    """One layer's decode step at the decode workload's shape, from a random
    mid-sequence state (position 8192); the oracle recomputes 3 of the 128
    sequences (sequences are independent)."""
    cfg = dict(W.LAYER, b=128, L=1)
    b, h, dk, dv, dm = cfg["b"], cfg["h"], cfg["dk"], cfg["dv"], cfg["d_model"]
    flags = W.XPOS | W.NORM_ALL
    dl, rl = _layers(cfg, 1, seed=31)
    rng = np.random.default_rng(7)
    x = W.as_f32(W.draw(rng, (b, dm), 1.0, "bf16"), "bf16")
    S0 = W.draw(rng, (b, h, dk, dv), 0.1, "f32")
    # a key-sum of the size a long sequence builds (sum of gamma^j k~, |k~| ~ 1)
    z0 = W.draw(rng, (b, h, dk), 1.0, "f32")
    th, g = W.theta_vector(dk), W.gamma_vector(h)
    pos = 8192
    announce("decode layer b128 dm4096 h16 dk256 dv512 dff16384 at position 8192")
    states = [(torch.from_numpy(S0).cuda(), torch.from_numpy(z0).cuda())]
    out = R.retnet_decode_step(dev(x, "f32"), dl, states, g, th, pos, pos + 1, flags, 1e-5, 1e-5)
    torch.cuda.synchronize()
    rows = np.array([0, 77, 127])
    ref, rst = oracle.retnet_decode_step(x[rows].astype(np.float64), rl, h, th, flags, 1e-5, 1e-5,
                                         [(S0[rows].astype(np.float64), z0[rows].astype(np.float64))], pos, pos + 1)
    check("decode layer full shape, sampled sequences", host64(out)[rows], ref, TOL["bf16"])
    # the state takes k~ and v from the fp16-stored projections: fp16 operand bar
    check("decode layer state S after the step", host64(states[0][0])[rows], rst[0][0], TOL["bf16"])
    check("decode layer key-sum z after the step", host64(states[0][1])[rows], rst[0][1], TOL["bf16"])
