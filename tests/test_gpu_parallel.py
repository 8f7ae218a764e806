"""Parity of retention_parallel_fwd (the parallel form: one chunk covering the
sequence) with the oracle's brute-force O(L^2) parallel form -- a different
code path of the oracle from its chunkwise form -- on short sequences of the
medium workload's head shape, ragged lengths, the fused kernels' shapes and
fp32 inputs."""
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


def _case(R, b, h, L, dk, dv, dtype, flags, seed, pos0=0):
    sigma = 1.0 if dtype == "f32" else 1.0 / np.sqrt(dk)
    q, k, v = W.chunkwise_inputs(b, h, L, dk, dv, dtype, sigma, seed=seed)
    g, th = W.gamma_vector(h), W.theta_vector(dk)
    announce(f"parallel b{b} h{h} L{L} dk{dk} dv{dv} {dtype} flags{flags} pos0={pos0}")
    o = R.parallel_fwd(dev(q, dtype), dev(k, dtype), dev(v, dtype), g, th, flags, pos0=pos0)
    torch.cuda.synchronize()
    ref = oracle.retention_parallel(f64(q, dtype), f64(k, dtype), f64(v, dtype), g, th, flags, pos0=pos0)
    name = f"parallel L{L} dk{dk} dv{dv} {dtype} f{flags}"
    if dtype == "bf16":
        check_bf16_out(name, host64(o), ref, TOL["bf16"])
    else:
        check(name, host64(o), ref, TOL["f32"])
    return q, k, v, o


@pytest.mark.parametrize("L", [64, 100, 512, 1000, 2048])
def test_parallel_medium_heads(R, L):
    _case(R, 1, 4, L, 256, 512, "bf16", W.XPOS | W.NORM_ALL, seed=L)


@pytest.mark.parametrize("flags", [W.XPOS, W.NORM_SCORE, W.SCALE_QK | W.NORM_DROW, 0])
def test_parallel_flags(R, flags):
    _case(R, 2, 2, 300, 256, 512, "bf16", flags, seed=3, pos0=17)


@pytest.mark.parametrize("dk,dv", [(128, 256), (64, 64)])
def test_parallel_fused_shapes(R, dk, dv):
    _case(R, 2, 3, 200, dk, dv, "bf16", W.XPOS | W.NORM_ALL, seed=dk)


def test_parallel_tiny_f32(R):
    c = W.CHUNKWISE["tiny"]
    _case(R, c["b"], c["h"], c["L"], c["dk"], c["dv"], "f32", c["flags"], seed=0)


def test_parallel_equals_chunkwise(R):
    """The parallel form and the chunkwise form (B = 64) of one sequence agree
    with each other as closely as each agrees with the oracle."""
    q, k, v, _ = _case(R, 1, 2, 512, 256, 512, "bf16", W.XPOS | W.NORM_ALL, seed=9)
    args = (dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), W.gamma_vector(2), W.theta_vector(256))
    # fp32 outputs, so that the comparison sees the computation, not two bf16 roundings
    o = R.parallel_fwd(*args, W.XPOS | W.NORM_ALL, out_dtype=torch.float32)
    oc = R.chunkwise_fwd(*args, 64, W.XPOS | W.NORM_ALL, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.retention_parallel(f64(q, "bf16"), f64(k, "bf16"), f64(v, "bf16"), W.gamma_vector(2),
                                    W.theta_vector(256), W.XPOS | W.NORM_ALL)
    e1 = check("parallel (f32 out)", host64(o), ref, TOL["bf16"])
    e2 = check("chunkwise B64 (f32 out)", host64(oc), ref, TOL["bf16"])
    check("parallel vs chunkwise B64", host64(o), host64(oc), 2 * max(e1, e2) + 1e-6)


@pytest.mark.parametrize("L", [1, 2])
def test_parallel_tiny_lengths(R, L):
    _case(R, 2, 2, L, 256, 512, "bf16", W.XPOS | W.NORM_ALL, seed=40 + L)
