"""The seeded input generator: deterministic, piece-size independent, and its
bf16 rounding is round-to-nearest-even (checked against torch's conversion)."""
import numpy as np
import torch

from linear_attention_sequence_retention_amd import workloads as W


def test_bf16_rne_matches_torch():
    r = np.random.default_rng(3)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -1.0 - 2.0 ** -8, 0.0, -0.0,
                                  65504.0, 1e-40], dtype=np.float32)])
    bits = W.f32_to_bf16_bits(x)
    t = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, t)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_draw_deterministic_and_piecewise(monkeypatch):
    a = W.chunkwise_inputs(1, 2, 40, 8, 6, 'bf16', 0.25, seed=0)
    monkeypatch.setattr(W, "_PIECE", 7)
    b = W.chunkwise_inputs(1, 2, 40, 8, 6, 'bf16', 0.25, seed=0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # draw order Q, K, V from one stream
    r = np.random.default_rng(0)
    q = W.f32_to_bf16_bits((r.standard_normal(1 * 2 * 40 * 8) * 0.25).astype(np.float32))
    assert np.array_equal(a[0].ravel(), q)


def test_parameters():
    assert np.array_equal(W.gamma_vector(3), [0.96875, 0.984375, 0.9921875])
    assert np.allclose(W.theta_vector(4), [1.0, 0.01])
    assert W.workload_name(W.CHUNKWISE['long'], 512) == "b1_h16_L32768_dk256_dv512_bf16_B512"
