"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the retention method: it only draws
Gaussian numbers, rounds them to the storage dtype and names the workloads.
Both the HIP path and the fp64 oracle receive exactly the arrays made here
(bf16 values are promoted exactly to wider types on the oracle side).

Recipe: ``numpy.random.default_rng(seed)`` (PCG64), standard normals drawn in
float64 in a fixed order, multiplied by sigma (sigma is a standard deviation),
rounded to float32 (round-to-nearest-even) and, for bf16, to bf16 (RNE on the
float32 bit pattern).  Draws are made in pieces; numpy's stream does not
depend on the piece size.

The per-head decay gamma_i = 1 - 2^(-5-i) is the multi-scale setting of the
RetNet reading notes (§三.2, MSR module) and theta_j = 10000^(-2j/d_k) is the
frequency ladder of the workloads; both are inputs of the method, passed to
the library and to the oracle as float64 host arrays.
"""

import numpy as np

# flag bits of the C ABI (include/retention.h)
XPOS, SCALE_QK, NORM_DROW, NORM_SCORE = 1, 2, 4, 8
NORM_ALL = SCALE_QK | NORM_DROW | NORM_SCORE

_PIECE = 1 << 22


def gamma_vector(h):
    return 1.0 - 2.0 ** (-5.0 - np.arange(h, dtype=np.float64))


def theta_vector(d_k, base=10000.0):
    return base ** (-2.0 * np.arange(d_k // 2, dtype=np.float64) / d_k)


def f32_to_bf16_bits(x32):
    """Round float32 values to bf16 (RNE); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def draw(rng, shape, sigma, dtype):
    """Draw N(0, sigma^2) values of ``shape`` in float64 and round to ``dtype``.

    dtype 'f32' -> float32 array; 'bf16' -> uint16 array of bf16 bit patterns.
    """
    n = int(np.prod(shape))
    if dtype == 'f32':
        out = np.empty(n, dtype=np.float32)
    elif dtype == 'bf16':
        out = np.empty(n, dtype=np.uint16)
    else:
        raise ValueError(dtype)
    for a in range(0, n, _PIECE):
        m = min(_PIECE, n - a)
        x = (rng.standard_normal(m) * sigma).astype(np.float32)
        out[a:a + m] = x if dtype == 'f32' else f32_to_bf16_bits(x)
    return out.reshape(shape)


def as_f32(a, dtype):
    """The exact float32 value of an array made by ``draw``."""
    return bf16_bits_to_f32(a) if dtype == 'bf16' else np.asarray(a, dtype=np.float32)


# --------------------------------------------------------------------------
# Workloads.  Shapes follow the pages' workloads: chunk size 512 and the 8192
# training length (RetNet reading notes, training efficiency; e993 news page,
# training cost), 7B-style heads and the 8k decode point (e993 news page,
# abstract).  No dataset is involved.
# --------------------------------------------------------------------------

CHUNKWISE = {
    'tiny': dict(b=1, h=2, L=128, dk=32, dv=32, dtype='f32', sigma=1.0,
                 flags=XPOS | SCALE_QK | NORM_DROW, chunks=(64,)),
    'medium': dict(b=4, h=8, L=2048, dk=256, dv=512, dtype='bf16', sigma=1.0 / 16,
                   flags=XPOS | NORM_ALL, chunks=(512, 64)),
    'long': dict(b=1, h=16, L=32768, dk=256, dv=512, dtype='bf16', sigma=1.0 / 16,
                 flags=XPOS | NORM_ALL, chunks=(512,)),
}

DECODE = dict(b=128, h=16, dk=256, dv=512, s0_sigma=0.1, sigma=1.0 / 16,
              pos0=8192, steps=64, flags=XPOS)

BLOCK = dict(b=2, L=8192, d_model=4096, h=16, dk=256, dv=512, x_sigma=1.0,
             w_sigma=0.02, chunk=512, flags=XPOS | NORM_ALL, eps=1e-5)

# One RetNet layer (reading notes §三.4) around the block workload: the FFN
# width is not stated there; the one width the pages print is the hotelren.com
# article's example model (§5.1: hidden 768, FFN 3072), i.e. 4 x d_model.
LAYER = dict(BLOCK, d_ff=4 * BLOCK['d_model'], ln_eps=1e-5, ln_sigma=0.1)


def workload_name(cfg, chunk=None):
    s = f"b{cfg['b']}_h{cfg['h']}_L{cfg['L']}_dk{cfg['dk']}_dv{cfg['dv']}_{cfg['dtype']}"
    return s + (f"_B{chunk}" if chunk is not None else "")


def chunkwise_inputs(b, h, L, dk, dv, dtype, sigma, seed=0, **_):
    """Q, K, V of shape [b,h,L,dk], [b,h,L,dk], [b,h,L,dv], drawn in that order."""
    rng = np.random.default_rng(seed)
    q = draw(rng, (b, h, L, dk), sigma, dtype)
    k = draw(rng, (b, h, L, dk), sigma, dtype)
    v = draw(rng, (b, h, L, dv), sigma, dtype)
    return q, k, v


def decode_inputs(b, h, dk, dv, s0_sigma, sigma, steps, seed=0, **_):
    """S0 [b,h,dk,dv] f32, then (q_t, k_t, v_t) bf16 for t = 0..steps-1."""
    rng = np.random.default_rng(seed)
    S0 = draw(rng, (b, h, dk, dv), s0_sigma, 'f32')
    qs, ks, vs = [], [], []
    for _t in range(steps):
        qs.append(draw(rng, (b, h, dk), sigma, 'bf16'))
        ks.append(draw(rng, (b, h, dk), sigma, 'bf16'))
        vs.append(draw(rng, (b, h, dv), sigma, 'bf16'))
    return S0, np.stack(qs), np.stack(ks), np.stack(vs)


def block_inputs(b, L, d_model, h, dk, dv, x_sigma, w_sigma, seed=0, **_):
    """X, W_Q, W_K, W_V, W_G, W_O (bf16), drawn in that order."""
    rng = np.random.default_rng(seed)
    X = draw(rng, (b, L, d_model), x_sigma, 'bf16')
    WQ = draw(rng, (d_model, h * dk), w_sigma, 'bf16')
    WK = draw(rng, (d_model, h * dk), w_sigma, 'bf16')
    WV = draw(rng, (d_model, h * dv), w_sigma, 'bf16')
    WG = draw(rng, (d_model, h * dv), w_sigma, 'bf16')
    WO = draw(rng, (h * dv, d_model), w_sigma, 'bf16')
    return X, WQ, WK, WV, WG, WO


def layer_inputs(b, L, d_model, h, dk, dv, d_ff, x_sigma, w_sigma, ln_sigma, seed=0, **_):
    """The block's X, W_Q, W_K, W_V, W_G, W_O, then W_1 [d_model, d_ff] and
    W_2 [d_ff, d_model] (bf16, N(0, w_sigma)), then the two LayerNorms'
    float32 (weight, bias): weight 1 + N(0, ln_sigma), bias N(0, ln_sigma)."""
    X, WQ, WK, WV, WG, WO = block_inputs(b, L, d_model, h, dk, dv, x_sigma, w_sigma, seed=seed)
    rng = np.random.default_rng([seed, 1])
    W1 = draw(rng, (d_model, d_ff), w_sigma, 'bf16')
    W2 = draw(rng, (d_ff, d_model), w_sigma, 'bf16')
    ln = []
    for _i in range(2):
        w = (1.0 + draw(rng, (d_model,), ln_sigma, 'f32')).astype(np.float32)
        ln.append((w, draw(rng, (d_model,), ln_sigma, 'f32')))
    return (X, WQ, WK, WV, WG, WO), W1, W2, ln[0], ln[1]
