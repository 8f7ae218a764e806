"""Parity of the bf16 projection GEMM and of the gated MSR block (four
projections, chunkwise retention on head views, GroupNorm + swish gate,
output projection) with the fp64 oracle."""
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


# M <= 128 takes the column-split (decode) kernel: full, ragged M and N, one K step
@pytest.mark.parametrize("M,N,K", [(300, 200, 256), (256, 256, 32), (1, 1000, 96), (513, 257, 4096),
                                   (128, 640, 4096), (77, 300, 512), (128, 17, 32), (129, 64, 64)])
def test_gemm(R, M, N, K):
    rng = np.random.default_rng(M + N + K)
    a = W.draw(rng, (M, K), 1.0, "bf16")
    b = W.draw(rng, (N, K), 0.05, "bf16")
    announce(f"gemm M{M} N{N} K{K}")
    c32 = R.gemm(dev(a, "bf16"), dev(b, "bf16"), out_dtype=torch.float32)
    c16 = R.gemm(dev(a, "bf16"), dev(b, "bf16"), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = f64(a, "bf16") @ f64(b, "bf16").T
    check(f"gemm {M}x{N}x{K} f32", host64(c32), ref, TOL["f32"])
    check_bf16_out(f"gemm {M}x{N}x{K} bf16", host64(c16), ref, TOL["bf16"])
    # fp16 activations against the bf16 weight (converted to fp16 in the kernel)
    a16 = dev(a, "bf16").to(torch.float16)
    c = R.gemm(a16, dev(b, "bf16"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(f"gemm {M}x{N}x{K} f16 A", host64(c), ref, TOL["f32"])


def test_gemm_block_shapes_sampled(R):
    """The block's projection shape (16384 x 4096 activations times a
    4096 -> 8192 weight); 16 sampled rows recomputed in fp64."""
    M, K, N = 16384, 4096, 8192
    rng = np.random.default_rng(5)
    a = W.draw(rng, (M, K), 1.0, "bf16")
    b = W.draw(rng, (N, K), 0.02, "bf16")
    announce("gemm block shape")
    c = R.gemm(dev(a, "bf16"), dev(b, "bf16"))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 4097, 8191, 9000, 12345, 16000, 16383, 77, 300, 2048, 6000, 15000, 16382])
    ref = f64(a[rows], "bf16") @ f64(b, "bf16").T
    got = host64(c)[rows]
    check_bf16_out("gemm 16384x8192x4096 sampled rows", got, ref, TOL["bf16"])


def _block_case(R, b, L, dm, h, dk, dv, chunk, seed, check_tokens=None):
    cfg = dict(b=b, L=L, d_model=dm, h=h, dk=dk, dv=dv, x_sigma=1.0, w_sigma=0.02)
    X, WQ, WK, WV, WG, WO = W.block_inputs(**cfg, seed=seed)
    th = W.theta_vector(dk)
    flags = W.XPOS | W.NORM_ALL
    announce(f"msr block b{b} L{L} dm{dm} h{h} dk{dk} dv{dv} B{chunk}")
    dT = lambda w: dev(np.ascontiguousarray(w.T), "bf16")     # [out, in] on the device
    out = R.msr_block_fwd(dev(X, "bf16"), dT(WQ), dT(WK), dT(WV), dT(WG), dT(WO), W.gamma_vector(h), th, chunk,
                          flags, 1e-5, out_dtype=torch.float32)
    torch.cuda.synchronize()
    nt = L if check_tokens is None else check_tokens
    ref = oracle.msr_forward(f64(X[:1, :nt], "bf16"), f64(WQ, "bf16"), f64(WK, "bf16"), f64(WV, "bf16"),
                             f64(WG, "bf16"), f64(WO, "bf16"), h, th, flags, chunk, 1e-5)
    check(f"msr block b{b} L{L} (batch 0, {nt} tokens)", host64(out)[:1, :nt], ref, TOL["bf16"])


def test_block_small(R):
    _block_case(R, 2, 300, 256, 2, 128, 256, 64, seed=1)


def test_block_full_shape_prefix(R):
    """The full block workload (batch 2, 8192 tokens, d_model 4096, 16 heads
    of 256 / 512, chunk 512); the oracle recomputes batch 0's first 1024
    tokens, which by causality depend on nothing later."""
    c = W.BLOCK
    _block_case(R, c["b"], c["L"], c["d_model"], c["h"], c["dk"], c["dv"], c["chunk"], seed=0, check_tokens=1024)
