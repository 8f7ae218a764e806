"""Parity of retention_chunkwise_bwd (HIP, through the C ABI) with the fp64
oracle's gradients of the normalised retention: ragged lengths spanning
several chunks, every normalisation choice, the score clamp active and
inactive, fp16 inputs, bf16 gradients, the independence of the result from
the backward's chunk size, and the medium workload's shape on sampled heads."""
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


def _inputs(b, h, L, dk, dv, seed, qscale=1.0):
    q, k, v = W.chunkwise_inputs(b, h, L, dk, dv, "bf16", 1.0 / np.sqrt(dk), seed=seed)
    if qscale != 1.0:
        q = W.f32_to_bf16_bits((W.as_f32(q, "bf16") * np.float32(qscale)).astype(np.float32))
    rng = np.random.default_rng(seed + 1000)
    do = W.draw(rng, (b, h, L, dv), 1.0, "bf16")
    return q, k, v, do


def _case(R, b, h, L, dk, dv, chunk, flags, seed, qscale=1.0, in_f16=False, grad_dtype=torch.float32,
          heads=None, pos0=0):
    q, k, v, do = _inputs(b, h, L, dk, dv, seed, qscale)
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    announce(f"bwd b{b} h{h} L{L} dk{dk} dv{dv} B{chunk} flags{flags} f16={in_f16} grad={grad_dtype} pos0={pos0}")
    if in_f16:
        tens = [torch.from_numpy(f64(x, "bf16").astype(np.float16)).cuda() for x in (q, k, v, do)]
        vals = [f64(x, "bf16").astype(np.float16).astype(np.float64) for x in (q, k, v, do)]
    else:
        tens = [dev(x, "bf16") for x in (q, k, v, do)]
        vals = [f64(x, "bf16") for x in (q, k, v, do)]
    dq, dk_, dv_ = R.chunkwise_bwd(*tens, g, th, chunk, flags, pos0=pos0, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    got = [host64(t) for t in (dq, dk_, dv_)]
    pairs = [(bb, hh) for bb in range(b) for hh in range(h)] if heads is None else heads
    name = f"bwd L{L} dk{dk} dv{dv} B{chunk} f{flags}"
    for bb, hh in pairs:
        sl = lambda x: x[bb:bb + 1, hh:hh + 1]
        ref = oracle.retention_parallel_bwd(sl(vals[0]), sl(vals[1]), sl(vals[2]), sl(vals[3]), g[hh:hh + 1], th,
                                            flags, pos0=pos0)
        for nm, gt, rf in zip(("dq", "dk", "dv"), got, ref):
            chk = check_bf16_out if grad_dtype == torch.bfloat16 else check
            chk(f"{name} ({bb},{hh}) {nm}", sl(gt), rf, TOL["bf16"])
    return got


@pytest.mark.parametrize("flags", [W.XPOS | W.NORM_ALL, W.XPOS, 0, W.NORM_SCORE | W.SCALE_QK])
def test_bwd_small(R, flags):
    _case(R, 1, 2, 200, 64, 64, 64, flags, seed=1)


@pytest.mark.parametrize("L,chunk", [(300, 128), (128, 128), (64, 64), (77, 64), (513, 256)])
def test_bwd_shapes(R, L, chunk):
    _case(R, 2, 2, L, 128, 256, chunk, W.XPOS | W.NORM_ALL, seed=L)


def test_bwd_clamp_active(R):
    """q scaled so that |s den| > 1 on many rows: the clamp's gradient path."""
    _case(R, 1, 3, 190, 128, 128, 64, W.XPOS | W.NORM_ALL, seed=7, qscale=40.0)


def test_bwd_f16_inputs_bf16_grads(R):
    _case(R, 1, 2, 150, 128, 256, 64, W.XPOS | W.NORM_ALL, seed=8, in_f16=True)
    _case(R, 1, 2, 150, 128, 256, 64, W.XPOS | W.NORM_ALL, seed=8, grad_dtype=torch.bfloat16, pos0=100)


def test_bwd_chunk_independent(R):
    """The backward's chunk size changes only rounding: B = 64 and B = 320
    agree with each other as closely as each agrees with the oracle."""
    a = _case(R, 1, 2, 320, 128, 256, 64, W.XPOS | W.NORM_ALL, seed=9)
    b = _case(R, 1, 2, 320, 128, 256, 320, W.XPOS | W.NORM_ALL, seed=9)
    for x, y, nm in zip(a, b, ("dq", "dk", "dv")):
        check(f"bwd B64 vs B320 {nm}", x, y, TOL["bf16"])


def test_bwd_deterministic(R):
    q, k, v, do = _inputs(1, 2, 256, 128, 256, 3)
    g, th = W.gamma_vector(2), W.theta_vector(128)
    t = [dev(x, "bf16") for x in (q, k, v, do)]
    r1 = [x.clone() for x in R.chunkwise_bwd(*t, g, th, 128, W.XPOS | W.NORM_ALL)]
    r2 = R.chunkwise_bwd(*t, g, th, 128, W.XPOS | W.NORM_ALL)
    torch.cuda.synchronize()
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("chunk", [256, 512])
def test_bwd_medium_sampled(R, chunk):
    """The medium workload's shape (batch 4, 8 heads, L = 2048, d_k 256,
    d_v 512, bf16); the oracle recomputes three sampled heads."""
    c = W.CHUNKWISE["medium"]
    _case(R, c["b"], c["h"], c["L"], c["dk"], c["dv"], chunk, c["flags"], seed=0,
          heads=[(0, 0), (2, 5), (3, 7)])


@pytest.mark.parametrize("L,chunk,dk,dv", [(1, 64, 128, 256), (65, 64, 128, 256), (130, 128, 128, 128),
                                           (64, 128, 64, 64), (129, 64, 256, 512)])
def test_bwd_edges(R, L, chunk, dk, dv):
    """A single token, a last chunk of one row, the (128, 128) shape, a chunk
    longer than the sequence, and one row past two full chunks."""
    _case(R, 2, 2, L, dk, dv, chunk, W.XPOS | W.NORM_ALL, seed=L + dk)
