"""Parity of retention_recurrent_step and msr_gate_norm (HIP, through the C
ABI) with the fp64 oracle, and the prefill -> decode hand-off."""
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


def _decode(R, b, h, dk, dv, steps, flags, use_z, seed, sample=None, out_dtype=torch.float32, in_f16=False):
    S0, qs, ks, vs = W.decode_inputs(b, h, dk, dv, 0.1, 1 / np.sqrt(dk), steps, seed=seed)
    if in_f16:
        # fp16 inputs: the bf16 draws rounded to fp16; both sides see those values
        qs, ks, vs = (f64(a, "bf16").astype(np.float16) for a in (qs, ks, vs))
        ind = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        inf = lambda a: a.astype(np.float64)
    else:
        ind = lambda a: dev(a, "bf16")
        inf = lambda a: f64(a, "bf16")
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    pos0 = 8192
    announce(f"decode b{b} h{h} dk{dk} dv{dv} steps{steps} flags{flags} z={use_z} f16 in={in_f16} out={out_dtype}")
    S = torch.from_numpy(S0).cuda()
    z = torch.zeros((b, h, dk), dtype=torch.float32, device="cuda") if use_z else None
    outs = []
    for t in range(steps):
        o = R.recurrent_step(ind(qs[t]), ind(ks[t]), ind(vs[t]), S, g, th, pos0 + t,
                             pos0 + t + 1, flags, z=z, out_dtype=out_dtype)
        outs.append(o)
    torch.cuda.synchronize()
    # oracle on all or on sampled (batch, head) pairs
    pairs = [(bb, hh) for bb in range(b) for hh in range(h)] if sample is None else sample
    bi = np.array([p[0] for p in pairs])
    hi = np.array([p[1] for p in pairs])
    S_ref = S0[bi, hi].astype(np.float64)[None]
    z_ref = np.zeros((1, len(pairs), dk)) if use_z else None
    gs = g[hi]
    o_ref, o_got = [], []
    for t in range(steps):
        o_t, S_ref, z_ref = oracle.recurrent_step(inf(qs[t][bi, hi])[None], inf(ks[t][bi, hi])[None],
                                                  inf(vs[t][bi, hi])[None], S_ref, gs, th, flags,
                                                  pos0 + t, pos0 + t + 1, z=z_ref)
        o_ref.append(o_t[0])
        o_got.append(host64(outs[t])[bi, hi])
    name = f"decode b{b}h{h} steps{steps} f{flags}"
    if out_dtype == torch.float16:
        # fp16 output: half an fp16 ulp of the exact value on top of the fp32 bar
        got, ref = np.stack(o_got), np.stack(o_ref)
        half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -14))) - 11)
        ex = np.max(np.maximum(np.abs(got - ref) - half_ulp, 0.0)) / np.sqrt(np.mean(ref ** 2))
        print(f"[parity] {name} o f16: beyond output rounding = {ex:.3e}", flush=True)
        assert ex <= TOL["f32"]
    else:
        chk = check_bf16_out if out_dtype == torch.bfloat16 else check
        chk(name + " o (all steps)", np.stack(o_got), np.stack(o_ref), TOL["bf16"])
    S_got = host64(S)[bi, hi]
    check(name + " final S", S_got, S_ref[0], TOL["f32"])
    if use_z:
        check(name + " final z", host64(z)[bi, hi], z_ref[0], TOL["f32"])


def test_decode_small(R):
    _decode(R, 2, 16, 256, 512, 8, W.XPOS, False, seed=1)


def test_decode_all_norms(R):
    _decode(R, 3, 4, 256, 512, 6, W.XPOS | W.NORM_ALL, True, seed=2)


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 128), (128, 1024), (6, 12)])
def test_decode_shapes(R, dk, dv):
    _decode(R, 2, 3, dk, dv, 3, W.XPOS | W.NORM_ALL, True, seed=3, out_dtype=torch.bfloat16)


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float32])
def test_decode_f16_inputs(R, out_dtype):
    _decode(R, 2, 4, 128, 256, 5, W.XPOS | W.NORM_ALL, True, seed=4, out_dtype=out_dtype, in_f16=True)


def test_decode_full_sampled(R):
    """The full decode workload (batch 128, 16 heads, 64 steps from position
    8192) on the GPU; the oracle follows 12 sampled sequences."""
    c = W.DECODE
    rng = np.random.default_rng(11)
    sample = [(int(rng.integers(c["b"])), int(rng.integers(c["h"]))) for _ in range(10)] + [(0, 0), (127, 15)]
    _decode(R, c["b"], c["h"], c["dk"], c["dv"], c["steps"], c["flags"], False, seed=0, sample=sample)


def test_prefill_then_decode(R):
    """Chunkwise prefill hands (state, z) to the decode step: the decoded
    outputs equal the oracle's one-pass chunkwise outputs (all normalisations)."""
    b, h, L, dk, dv, L1 = 1, 4, 200, 256, 512, 150
    flags = W.XPOS | W.NORM_ALL
    q, k, v = W.chunkwise_inputs(b, h, L, dk, dv, "bf16", 1 / 16, seed=12)
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    announce("prefill -> decode hand-off")
    o_ref = oracle.retention_chunkwise(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), g, th, flags, 64)[0]
    qd, kd, vd = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    S = torch.zeros((b, h, dk, dv), dtype=torch.float32, device="cuda")
    z = torch.zeros((b, h, dk), dtype=torch.float32, device="cuda")
    o1 = R.chunkwise_fwd(qd[:, :, :L1], kd[:, :, :L1], vd[:, :, :L1], g, th, 64, flags, state_out=S, z_out=z)
    outs = []
    for t in range(L1, L):
        outs.append(R.recurrent_step(qd[:, :, t].contiguous(), kd[:, :, t].contiguous(), vd[:, :, t].contiguous(),
                                     S, g, th, t, t + 1, flags, z=z))
    torch.cuda.synchronize()
    check_bf16_out("prefill part", host64(o1), o_ref[:, :, :L1], TOL["bf16"])
    got = np.stack([host64(o) for o in outs], axis=2)
    check("decode part", got, o_ref[:, :, L1:], TOL["bf16"])


@pytest.mark.parametrize("dtype,dv,affine", [("bf16", 512, False), ("bf16", 64, True), ("f32", 32, True),
                                             ("bf16", 1024, False), ("bf16", 24, False)])
def test_gate_norm(R, dtype, dv, affine):
    b, h, L = 2, 3, 37
    rng = np.random.default_rng(20 + dv)
    y = W.draw(rng, (b, h, L, dv), 0.3, dtype)
    gg = W.draw(rng, (b, L, h * dv), 2.0, dtype)
    w = (1.0 + 0.1 * rng.standard_normal(h * dv)).astype(np.float32) if affine else None
    bias = (0.1 * rng.standard_normal(h * dv)).astype(np.float32) if affine else None
    announce(f"gate_norm {dtype} dv{dv} affine={affine}")
    out = R.gate_norm(dev(y, dtype), dev(gg, dtype), 1e-5,
                      weight=None if w is None else torch.from_numpy(w).cuda(),
                      bias=None if bias is None else torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    ref = oracle.gate_norm(f64(y, dtype), f64(gg, dtype), 1e-5, w, bias)
    if dtype == "bf16":
        check_bf16_out(f"gate_norm {dtype} dv{dv}", host64(out), ref, TOL[dtype])
    else:
        check(f"gate_norm {dtype} dv{dv}", host64(out), ref, TOL[dtype])


def test_gate_norm_strided_full_block_shape(R):
    """The block's shape (2 x 8192 tokens, 16 heads of 512) with Y read as a
    [b,h,L,d] view of a [b,L,h*d] buffer; sampled tokens checked."""
    b, L, h, dv = 2, 8192, 16, 512
    rng = np.random.default_rng(30)
    y = W.draw(rng, (b, L, h * dv), 1.0, "bf16")
    gg = W.draw(rng, (b, L, h * dv), 1.0, "bf16")
    announce("gate_norm block shape")
    yd = dev(y, "bf16").view(b, L, h, dv).transpose(1, 2)
    out = R.gate_norm(yd, dev(gg, "bf16"), 1e-5)
    torch.cuda.synchronize()
    toks = np.array([0, 1, 777, 4095, 8191])
    yv = np.transpose(y.reshape(b, L, h, dv), (0, 2, 1, 3))[:, :, toks]
    ref = oracle.gate_norm(f64(yv, "bf16"), f64(gg[:, toks], "bf16"), 1e-5)
    check_bf16_out("gate_norm block sampled", host64(out)[:, toks], ref, TOL["bf16"])
