"""The non-finite output record (retention_range_status): a bf16 input beyond
the fp16 operand range makes the kernels write inf / NaN, and the query
reports it instead of letting it pass; in-range calls leave the record clear
(every GPU test checks that after it runs, through the conftest fixture)."""
import numpy as np
import pytest
import torch

from gpu_util import announce
from linear_attention_sequence_retention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def R():
    from linear_attention_sequence_retention_amd import binding
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    binding.range_status()          # start from a clear record
    return binding


def _inputs(b, h, L, dk, dv, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    mk = lambda d: (torch.randn((b, h, L, d), generator=g) * scale).to(torch.bfloat16).cuda()
    return mk(dk), mk(dk), mk(dv)


# (d_k, d_v, chunk): the large-chunk kernels, the small-chunk state scan and the fused kernel
PATHS = [(256, 512, 512), (256, 512, 64), (128, 256, 128), (64, 64, 64)]


@pytest.mark.parametrize("dk,dv,B", PATHS)
@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_forward_flags_out_of_range_input(R, dk, dv, B, which):
    b, h, L = 1, 2, 300
    q, k, v = _inputs(b, h, L, dk, dv, seed=dk + B)
    gam, th = W.gamma_vector(h), W.theta_vector(dk)
    flags = W.XPOS | W.NORM_ALL
    # v enters an fp16 operand as it is; q and k are rotated (and q may be
    # scaled down) first, so they are pushed far beyond the range
    bad = 7.0e4 if which == "v" else 1.0e30
    announce(f"range forward d_k{dk} d_v{dv} B{B} {which} = {bad:g}")
    o = R.chunkwise_fwd(q, k, v, gam, th, B, flags, out_dtype=torch.float32)
    assert R.range_status() is None, "in-range inputs were reported"
    assert torch.isfinite(o).all()
    t = {"q": q, "k": k, "v": v}[which]
    t[0, 1, 137, 5] = bad            # finite in bf16, beyond fp16's 65504
    o = R.chunkwise_fwd(q, k, v, gam, th, B, flags, out_dtype=torch.float32)
    msg = R.range_status()
    assert msg is not None and "forward" in msg, "out-of-range input not reported"
    assert not torch.isfinite(o[0, 1, 137]).all()
    assert torch.isfinite(o[0, 0]).all(), "another head is not finite"
    assert R.range_status() is None, "the query did not clear the record"


def test_parallel_flags_out_of_range_input(R):
    q, k, v = _inputs(1, 2, 200, 256, 512, seed=3)
    v[0, 0, 50, 7] = -7.0e4
    announce("range parallel v = -7e4")
    R.parallel_fwd(q, k, v, W.gamma_vector(2), W.theta_vector(256), W.XPOS | W.NORM_ALL, out_dtype=torch.bfloat16)
    msg = R.range_status()
    assert msg is not None and "forward" in msg


def test_f16_output_overflow_is_flagged(R):
    """In-range operands whose exact result exceeds fp16: an f16 output is
    flagged, an fp32 output of the same call is not."""
    b, h, L, dk, dv = 1, 1, 256, 64, 64
    q = torch.full((b, h, L, dk), 4.0, dtype=torch.bfloat16, device="cuda")
    k = q.clone()
    v = torch.full((b, h, L, dv), 1000.0, dtype=torch.bfloat16, device="cuda")
    gam = np.array([0.999])
    announce("range f16 output overflow")
    o32 = R.chunkwise_fwd(q, k, v, gam, None, 64, 0, out_dtype=torch.float32)
    assert R.range_status() is None
    assert float(o32.abs().max()) > 65520.0
    R.chunkwise_fwd(q, k, v, gam, None, 64, 0, out_dtype=torch.float16)
    assert R.range_status() is not None


def test_backward_flags_out_of_range_input(R):
    b, h, L, dk, dv = 1, 2, 256, 128, 256
    q, k, v = _inputs(b, h, L, dk, dv, seed=9)
    do = torch.randn((b, h, L, dv)).to(torch.bfloat16).cuda()
    gam, th = W.gamma_vector(h), W.theta_vector(dk)
    flags = W.XPOS | W.NORM_ALL
    announce("range backward")
    R.chunkwise_bwd(q, k, v, do, gam, th, 64, flags)
    assert R.range_status() is None
    v[0, 1, 100, 3] = 7.0e4
    R.chunkwise_bwd(q, k, v, do, gam, th, 64, flags)
    msg = R.range_status()
    assert msg is not None and "backward" in msg
