"""Pins of the fp64 oracle against facts the pages and mathematics fix.

Each ``pin_*`` function takes the oracle module (so that the mutation tests can
hand in a copy with a planted mistake) and raises AssertionError when the
module disagrees with a closed form, an invariant, an equivalence of two
different algorithms, or brute-force summation.  None of them re-types the
oracle's own formula: expected values come from special inputs whose result
the pages' definitions give in closed form, or from sums written out here.

Pages (title, section):
  RetNet reading notes (mzeromiko): §2.2 recurrent, §2.3 parallel, §2.4
  chunkwise, §三.2 MSR, §三.3 normalisation.
  e993 news page (RetNet paper translation): the three forms are rewritings of
  one mapping; GroupNorm's scale invariance makes the normalisation tricks
  leave the final result unchanged.
"""

import numpy as np

XPOS, SCALE_QK, NORM_DROW, NORM_SCORE = 1, 2, 4, 8
NORM_ALL = SCALE_QK | NORM_DROW | NORM_SCORE


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _close(a, b, rtol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    ref = max(np.max(np.abs(b)), 1e-300)
    err = np.max(np.abs(a - b)) / ref
    assert err <= rtol, f"{what}: rel err {err:.3e} > {rtol:.1e}"


def _thetas(dk):
    return 10000.0 ** (-2.0 * np.arange(dk // 2) / dk)


# ---------------------------------------------------------------- parameters

def pin_gamma_theta(m):
    # MSR module: gamma = 1 - 2^(-5 - arange(0, h)); exact binary fractions
    g = m.gammas(4)
    assert np.array_equal(g, [0.96875, 0.984375, 0.9921875, 0.99609375]), g
    # theta_j = 10000^(-2j/d_k) with d_k = 8 gives 10^-j
    _close(m.thetas(8), [1.0, 0.1, 0.01, 0.001], 1e-15, "theta ladder")


# -------------------------------------------------------- form equivalence

def pin_forms_agree(m, L=128, flags_list=range(16), chunks=(1, 2, 3, 5, 8, 16, 32, 64, 100, 128),
                    b=1, h=2, dk=8, dv=6, seed=0):
    """Recurrent == parallel == chunkwise (every chunk size) in fp64.

    B = 1 reduces the chunkwise form to the recurrent one and B >= L to the
    parallel one; the normalisers of the parallel form are explicit row sums.
    """
    q = _rand((b, h, L, dk), seed)
    k = _rand((b, h, L, dk), seed + 1)
    v = _rand((b, h, L, dv), seed + 2)
    g = np.array([0.75, 0.96875])[:h] if h <= 2 else m.gammas(h)
    th = _thetas(dk)
    for flags in flags_list:
        o_par = m.retention_parallel(q, k, v, g, th, flags, pos0=3)
        o_rec, S_rec, z_rec = m.retention_recurrent(q, k, v, g, th, flags, pos0=3)
        _close(o_rec, o_par, 1e-12, f"recurrent vs parallel flags={flags}")
        for B in chunks:
            o_ch, S_ch, z_ch = m.retention_chunkwise(q, k, v, g, th, flags, B, pos0=3)
            _close(o_ch, o_par, 1e-12, f"chunkwise B={B} vs parallel flags={flags}")
            _close(S_ch, S_rec, 1e-12, f"chunkwise B={B} final state flags={flags}")
            _close(z_ch, z_rec, 1e-12, f"chunkwise B={B} final key-sum flags={flags}")


def _all_forms(m, q, k, v, g, th, flags, chunks=(1, 3, 4, 7, 64), pos0=0):
    yield "parallel", m.retention_parallel(q, k, v, g, th, flags, pos0=pos0)
    yield "recurrent", m.retention_recurrent(q, k, v, g, th, flags, pos0=pos0)[0]
    for B in chunks:
        yield f"chunkwise B={B}", m.retention_chunkwise(q, k, v, g, th, flags, B, pos0=pos0)[0]


# ------------------------------------------------------------ closed forms

def pin_onehot_decay(m):
    """q_n = e_a, a single key e_a with value e_c at m0: O_n[c] = gamma^(n-m0), n >= m0.

    D is causal including the diagonal (§2.3); no normalisation flags.
    """
    L, dk, dv, a, c, m0 = 20, 4, 3, 1, 2, 6
    g = np.array([0.8, 0.5])
    q = np.zeros((1, 2, L, dk)); q[..., a] = 1.0
    k = np.zeros((1, 2, L, dk)); k[:, :, m0, a] = 1.0
    v = np.zeros((1, 2, L, dv)); v[:, :, m0, c] = 1.0
    n = np.arange(L)
    want = np.zeros((1, 2, L, dv))
    for hh in range(2):
        want[0, hh, :, c] = np.where(n >= m0, g[hh] ** np.maximum(n - m0, 0), 0.0)
    for name, o in _all_forms(m, q, k, v, g, _thetas(dk), 0):
        _close(o, want, 1e-14, f"one-hot decay ({name})")


def _xpos_setup(q_axis, k_axis, L=24, dk=8, dv=3, m0=5, scale=1.0):
    q = np.zeros((1, 1, L, dk)); q[..., q_axis] = scale
    k = np.zeros((1, 1, L, dk)); k[:, :, m0, k_axis] = 1.0
    v = np.zeros((1, 1, L, dv)); v[:, :, m0, 1] = 1.0
    return q, k, v


def pin_xpos_closed_form(m):
    """Real form of e^{i n theta}: pair (2j, 2j+1) rotated by +p theta_j.

    q = e_{2j}, key e_{2j+1} at m0 -> O_n = gamma^(n-m0) sin((n-m0) theta_j);
    key e_{2j} -> cos; q = e_{2j+1}, key e_{2j} -> -sin.  Independent of pos0.
    """
    L, dk, m0, j = 24, 8, 5, 1
    th = _thetas(dk) * 3.0
    g = np.array([0.9])
    n = np.arange(L)
    d = n - m0
    base = np.where(d >= 0, 0.9 ** np.maximum(d, 0), 0.0)
    cases = [(2 * j, 2 * j + 1, np.sin(d * th[j])),
             (2 * j, 2 * j, np.cos(d * th[j])),
             (2 * j + 1, 2 * j, -np.sin(d * th[j])),
             (2 * j + 1, 2 * j + 1, np.cos(d * th[j]))]
    for qa, ka, trig in cases:
        q, k, v = _xpos_setup(qa, ka, L, dk, m0=m0)
        want = np.zeros((1, 1, L, 3))
        want[0, 0, :, 1] = base * trig
        for pos0 in (0, 1000):
            for name, o in _all_forms(m, q, k, v, g, th, XPOS, pos0=pos0):
                _close(o, want, 1e-12, f"xpos q=e{qa} k=e{ka} pos0={pos0} ({name})")


def pin_drow_scale_closed_form(m):
    """QK^T/sqrt(d_k) and D~ = D / sqrt(sum_{i<=n} D_ni) on the one-hot input.

    The D row sum is summed term by term here (the page's definition), not
    taken from the geometric-series closed form.
    """
    L, dk, m0, j = 30, 8, 4, 2
    th = _thetas(dk)
    g = np.array([0.97])
    q, k, v = _xpos_setup(2 * j, 2 * j, L, dk, m0=m0)
    n = np.arange(L)
    rowsum = np.array([sum(0.97 ** (nn - i) for i in range(nn + 1)) for nn in n])
    d = n - m0
    want = np.zeros((1, 1, L, 3))
    want[0, 0, :, 1] = np.where(d >= 0, 0.97 ** np.maximum(d, 0), 0.0) * np.cos(d * th[j])
    w_scale = want / np.sqrt(dk)
    w_drow = want / np.sqrt(rowsum)[None, None, :, None]
    for flags, w in ((XPOS | SCALE_QK, w_scale), (XPOS | NORM_DROW, w_drow),
                     (XPOS | SCALE_QK | NORM_DROW, w_drow / np.sqrt(dk))):
        for name, o in _all_forms(m, q, k, v, g, th, flags):
            _close(o, w, 1e-12, f"flags={flags} ({name})")


def pin_score_clamp(m):
    """R~ = R / max(|sum_i R_ni|, 1): with one live key the row sum is the score.

    With q scaled by 1e4 the clamp is active and the output is sign(score),
    i.e. exactly +-1; rows whose |score| < 1 stay unnormalised.
    """
    L, dk, m0, j = 40, 8, 3, 0
    th = _thetas(dk) * 0.37
    g = np.array([0.95])
    q, k, v = _xpos_setup(2 * j, 2 * j, L, dk, m0=m0, scale=1e4)
    n = np.arange(L)
    d = n - m0
    score = np.where(d >= 0, 1e4 * 0.95 ** np.maximum(d, 0) * np.cos(d * th[j]), 0.0)
    active = np.abs(score) >= 1.0
    assert active.sum() > 20 and (~active & (d >= 0)).sum() >= 0
    for name, o in _all_forms(m, q, k, v, g, th, XPOS | NORM_SCORE):
        o1 = o[0, 0, :, 1]
        assert np.allclose(o1[active], np.sign(score[active]), rtol=0, atol=1e-12), f"clamp ({name})"
        assert np.allclose(o1[~active], score[~active], rtol=0, atol=1e-12), f"unclamped rows ({name})"
        assert np.all(o[0, 0, :, [0, 2]] == 0.0)
    # a row sum that is negative uses |.|: the sign of the output follows the score
    assert np.any(score[active] < 0)


# ------------------------------------------------------------- invariants

def pin_groupnorm_invariance(m):
    """GroupNorm(alpha * head) = GroupNorm(head): the three normalisation
    factors are positive per-row scalars, so GN of the retention output is the
    same for every combination of them (e993 news page, normalisation)."""
    b, h, L, dk, dv = 2, 3, 33, 8, 6
    q = _rand((b, h, L, dk), 10)
    k = _rand((b, h, L, dk), 11)
    v = _rand((b, h, L, dv), 12)
    g = m.gammas(h)
    th = _thetas(dk)
    ref = None
    for f in range(8):
        flags = XPOS | (f << 1)
        o = m.retention_chunkwise(q, k, v, g, th, flags, 7)[0]
        gn = m.group_norm_heads(o, eps=0.0)
        if ref is None:
            ref = gn
        else:
            _close(gn, ref, 1e-10, f"GN invariance flags={flags}")
    # per (token, head) group: mean 0, biased variance 1
    gg = ref.reshape(b, L, h, dv)
    assert np.max(np.abs(gg.mean(-1))) < 1e-12
    assert np.max(np.abs((gg ** 2).mean(-1) - 1.0)) < 1e-10
    # per-token positive rescaling of a head is invisible
    o = m.retention_chunkwise(q, k, v, g, th, XPOS, 7)[0]
    alpha = np.exp(_rand((b, h, L, 1), 13))
    _close(m.group_norm_heads(o * alpha, 0.0), m.group_norm_heads(o, 0.0), 1e-10, "GN per-token alpha")


def pin_groupnorm_values(m):
    """Hand-computed GroupNorm of one group: [1,2,3,4] has mean 2.5 and biased
    variance 1.25, so it maps to [-3,-1,1,3]/sqrt(5); the group of the second
    head is independent of the first; the affine is per channel."""
    y = np.zeros((1, 2, 1, 4))
    y[0, 0, 0] = [1, 2, 3, 4]
    y[0, 1, 0] = [10, 10, 10, 14]          # mean 11, var 3
    out = m.group_norm_heads(y, eps=0.0)
    want = np.array([[-3, -1, 1, 3]]) / np.sqrt(5.0)
    _close(out[0, 0, :4], want[0], 1e-15, "GN head 0")
    _close(out[0, 0, 4:], np.array([-1, -1, -1, 3]) / np.sqrt(3.0), 1e-15, "GN head 1")
    w = np.arange(1, 9, dtype=np.float64)
    bb = -np.arange(8, dtype=np.float64)
    out2 = m.group_norm_heads(y, eps=0.0, weight=w, bias=bb)
    _close(out2, out * w + bb, 1e-15, "GN affine")
    # eps enters under the square root: [1, -1] with eps=3 -> [1,-1]/2
    y2 = np.array([1.0, -1.0]).reshape(1, 1, 1, 2)
    _close(m.group_norm_heads(y2, eps=3.0)[0, 0], [0.5, -0.5], 1e-15, "GN eps")


def pin_swish(m):
    """swish(x) = x sigmoid(x): 0 at 0, ~x for large x, ~0 for very negative x,
    swish(1) = 1/(1 + 1/e) = 0.7310585786300049."""
    x = np.array([0.0, 1.0, 40.0, -40.0, -1.0])
    s = m.swish(x)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-15
    assert abs(s[2] - 40.0) < 1e-12 and abs(s[3]) < 1e-15
    assert abs(s[4] + 0.2689414213699951) < 1e-15
    # gate applies swish(g) elementwise to the normalised heads
    y = np.array([1.0, 2.0, 3.0, 4.0]).reshape(1, 1, 1, 4)
    gate = np.array([[[0.0, 1.0, 40.0, -1.0]]])
    out = m.gate_norm(y, gate, 0.0)
    yn = np.array([-3, -1, 1, 3]) / np.sqrt(5.0)
    _close(out[0, 0], yn * np.array([0.0, 0.7310585786300049, 40.0, -0.2689414213699951]),
           1e-12, "gate")


def pin_relative_position(m):
    """Scores depend on n - m only (§2.1): shifting pos0 leaves O unchanged."""
    b, h, L, dk, dv = 1, 2, 29, 8, 5
    q = _rand((b, h, L, dk), 20)
    k = _rand((b, h, L, dk), 21)
    v = _rand((b, h, L, dv), 22)
    g = m.gammas(h)
    th = _thetas(dk)
    for flags in (XPOS, XPOS | NORM_ALL):
        a = m.retention_chunkwise(q, k, v, g, th, flags, 8, pos0=0)[0]
        bb = m.retention_chunkwise(q, k, v, g, th, flags, 8, pos0=1000)[0]
        _close(bb, a, 1e-10, f"pos0 shift flags={flags}")
        c = m.retention_recurrent(q, k, v, g, th, flags, pos0=777)[0]
        _close(c, a, 1e-10, f"pos0 shift recurrent flags={flags}")


def pin_split_resume(m):
    """The state (R, z) is the whole sequence checkpoint: running L1 tokens,
    handing (R, z) over and running the rest (positions and token counts
    continuing) equals one pass, at any split point and chunk size."""
    b, h, L, dk, dv = 2, 2, 45, 8, 6
    q = _rand((b, h, L, dk), 30)
    k = _rand((b, h, L, dk), 31)
    v = _rand((b, h, L, dv), 32)
    g = m.gammas(h)
    th = _thetas(dk)
    flags = XPOS | NORM_ALL
    full, S_full, z_full = m.retention_chunkwise(q, k, v, g, th, flags, 8)
    for L1, B1, B2 in ((1, 4, 8), (13, 5, 3), (32, 16, 7), (44, 44, 1)):
        o1, S1, z1 = m.retention_chunkwise(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g, th, flags, B1)
        o2, S2, z2 = m.retention_chunkwise(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g, th, flags, B2,
                                           pos0=L1, n_prev=L1, state_in=S1, z_in=z1)
        _close(np.concatenate([o1, o2], axis=2), full, 1e-12, f"split at {L1}")
        _close(S2, S_full, 1e-12, f"state after split {L1}")
        _close(z2, z_full, 1e-12, f"key-sum after split {L1}")
        o3, S3, _ = m.retention_recurrent(q[:, :, L1:], k[:, :, L1:], v[:, :, L1:], g, th, flags,
                                          pos0=L1, n_prev=L1, state_in=S1, z_in=z1)
        _close(o3, o2, 1e-12, f"recurrent resume at {L1}")


def pin_causality_linearity(m):
    """D is zero above the diagonal: tokens after p never change o_<=p.
    Without the score clamp the map is linear in V."""
    b, h, L, dk, dv = 1, 2, 31, 8, 4
    q = _rand((b, h, L, dk), 40)
    k = _rand((b, h, L, dk), 41)
    v = _rand((b, h, L, dv), 42)
    g = m.gammas(h)
    th = _thetas(dk)
    p = 17
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, p + 1:] += 5.0
    k2[:, :, p + 1:] -= 3.0
    v2[:, :, p + 1:] *= -2.0
    for flags in (XPOS, XPOS | NORM_ALL):
        for B in (1, 6, 64):
            a = m.retention_chunkwise(q, k, v, g, th, flags, B)[0]
            c = m.retention_chunkwise(q2, k2, v2, g, th, flags, B)[0]
            assert np.array_equal(a[:, :, :p + 1], c[:, :, :p + 1]) or \
                np.max(np.abs(a[:, :, :p + 1] - c[:, :, :p + 1])) < 1e-13
            assert np.max(np.abs(a[:, :, p + 1:] - c[:, :, p + 1:])) > 1e-3
    w = _rand((b, h, L, dv), 43)
    flags = XPOS | SCALE_QK | NORM_DROW
    lhs = m.retention_chunkwise(q, k, 2.0 * v - 3.0 * w, g, th, flags, 6)[0]
    rhs = 2.0 * m.retention_chunkwise(q, k, v, g, th, flags, 6)[0] - 3.0 * m.retention_chunkwise(q, k, w, g, th, flags, 6)[0]
    _close(lhs, rhs, 1e-12, "linear in V")


# ----------------------------------------------------------------- decode

def pin_decode_zero_kv(m):
    """With k = v = 0 the step only decays: S_t = gamma^t S_0 and
    o_t = gamma^(t+1) q'_t S_0 (state read after the update)."""
    b, h, dk, dv = 2, 3, 8, 5
    g = m.gammas(h)
    th = _thetas(dk)
    S0 = _rand((b, h, dk, dv), 50)
    S = S0.copy()
    zero_k = np.zeros((b, h, dk))
    zero_v = np.zeros((b, h, dv))
    for t in range(6):
        # q = e_0 picks row 0 of the state after rotation by phi = pos*theta_0:
        # q' = (cos phi, sin phi, 0, ...) -> o = cos phi S[0] + sin phi S[1]
        qv = np.zeros((b, h, dk)); qv[..., 0] = 1.0
        pos = 100 + t
        o, S, _ = m.recurrent_step(qv, zero_k, zero_v, S, g, th, XPOS, pos, pos + 1)
        decay = (g ** (t + 1))[None, :, None]
        _close(S, S0 * decay[..., None], 1e-14, f"S_t decay t={t}")
        phi = pos * th[0]
        want = decay * (np.cos(phi) * S0[:, :, 0, :] + np.sin(phi) * S0[:, :, 1, :])
        _close(o, want, 1e-13, f"o_t t={t}")


def pin_decode_vs_chunkwise(m):
    """Prefill with the chunkwise form, then decode token by token: equals
    one chunkwise pass over the whole sequence (all normalisations on, the
    key-sum z carried for the score normaliser)."""
    b, h, L, dk, dv = 1, 2, 20, 8, 6
    q = _rand((b, h, L, dk), 60)
    k = _rand((b, h, L, dk), 61)
    v = _rand((b, h, L, dv), 62)
    g = m.gammas(h)
    th = _thetas(dk)
    flags = XPOS | NORM_ALL
    full = m.retention_chunkwise(q, k, v, g, th, flags, 4)[0]
    L1 = 12
    _, S, z = m.retention_chunkwise(q[:, :, :L1], k[:, :, :L1], v[:, :, :L1], g, th, flags, 5)
    for t in range(L1, L):
        o, S, z = m.recurrent_step(q[:, :, t], k[:, :, t], v[:, :, t], S, g, th, flags, t, t + 1, z=z)
        _close(o, full[:, :, t], 1e-12, f"decode step {t}")


# ------------------------------------------------------------------ block

def pin_block(m):
    """MSR block (§三.2): X W_G = 0 gives 0 (swish(0) = 0); scaling W_O scales
    the output; scaling W_V by alpha > 0 changes nothing (GroupNorm after the
    retention, eps = 0); heads take contiguous column blocks; the chunk size
    does not change the result."""
    b, L, dm, h, dk, dv = 1, 19, 8, 2, 4, 6
    r = np.random.default_rng(70)
    X = r.standard_normal((b, L, dm))
    WQ, WK = r.standard_normal((dm, h * dk)), r.standard_normal((dm, h * dk))
    WV, WG = r.standard_normal((dm, h * dv)), r.standard_normal((dm, h * dv))
    WO = r.standard_normal((h * dv, dm))
    th = _thetas(dk)
    flags = XPOS | NORM_ALL
    out = m.msr_forward(X, WQ, WK, WV, WG, WO, h, th, flags, 5, 0.0)
    assert out.shape == (b, L, dm)
    assert np.max(np.abs(m.msr_forward(X, WQ, WK, WV, 0 * WG, WO, h, th, flags, 5, 0.0))) == 0.0
    _close(m.msr_forward(X, WQ, WK, WV, WG, 3.0 * WO, h, th, flags, 5, 0.0), 3.0 * out, 1e-13, "W_O scale")
    _close(m.msr_forward(X, WQ, WK, WV, WG, WO, h, th, flags, 64, 0.0), out, 1e-11, "chunk size")
    flags2 = XPOS | SCALE_QK | NORM_DROW
    o2 = m.msr_forward(X, WQ, WK, WV, WG, WO, h, th, flags2, 5, 0.0)
    _close(m.msr_forward(X, WQ, WK, 2.5 * WV, WG, WO, h, th, flags2, 5, 0.0), o2, 1e-11, "W_V scale")
    # the gate multiplies the normalised heads before W_O: with W_O a
    # permutation and a positive per-column gate, undoing both leaves groups
    # of mean 0 and variance 1
    dm2 = h * dv
    X2 = r.standard_normal((b, L, dm2)); X2[..., 0] = 1.0
    WQ2, WK2 = r.standard_normal((dm2, h * dk)), r.standard_normal((dm2, h * dk))
    WV2 = r.standard_normal((dm2, h * dv))
    WG2 = np.zeros((dm2, h * dv)); WG2[0] = 2.0 + r.random(h * dv)
    perm = np.arange(dm2)[::-1].copy()
    WO2 = np.eye(dm2)[:, perm]
    out2 = m.msr_forward(X2, WQ2, WK2, WV2, WG2, WO2, h, th, flags, 5, 0.0)
    gate = WG2[0] / (1.0 + np.exp(-WG2[0]))
    ynorm = (out2 @ WO2.T / gate).reshape(b, L, h, dv)
    assert np.max(np.abs(ynorm.mean(-1))) < 1e-12
    assert np.max(np.abs((ynorm ** 2).mean(-1) - 1.0)) < 1e-10
    # hand-assembled block: per head, the projections taken column block by
    # column block, the brute-force parallel form (a separate, separately
    # pinned path), GroupNorm written out as the group mean and biased
    # variance, then swish(X W_G) times the normalised heads, then W_O
    eps = 1e-5
    hand = np.zeros((b, L, dm))
    Yn = np.zeros((b, L, h * dv))
    for i in range(h):
        qi = X @ WQ[:, i * dk:(i + 1) * dk]
        ki = X @ WK[:, i * dk:(i + 1) * dk]
        vi = X @ WV[:, i * dv:(i + 1) * dv]
        oi = m.retention_parallel(qi[:, None], ki[:, None], vi[:, None], m.gammas(h)[i:i + 1], th, flags)[:, 0]
        for bb in range(b):
            for t in range(L):
                row = oi[bb, t]
                mu = sum(row) / dv
                var = sum((x - mu) ** 2 for x in row) / dv
                Yn[bb, t, i * dv:(i + 1) * dv] = (row - mu) / np.sqrt(var + eps)
    G = X @ WG
    hand = (G / (1.0 + np.exp(-G)) * Yn) @ WO
    _close(m.msr_forward(X, WQ, WK, WV, WG, WO, h, th, flags, 5, eps), hand, 1e-10, "block vs hand-assembled")
    swapped = m.msr_forward(X, WK, WQ, WV, WG, WO, h, th, flags, 5, eps)
    assert np.max(np.abs(swapped - hand)) > 1e-3 * np.max(np.abs(hand)), "W_Q / W_K swap not visible"
    # split_heads: column c of head i is input column i*d + c
    x = np.arange(2 * 3 * 8, dtype=np.float64).reshape(2, 3, 8)
    s = m.split_heads(x, 2)
    assert s.shape == (2, 2, 3, 4)
    for bb in range(2):
        for i in range(2):
            for t in range(3):
                for c in range(4):
                    assert s[bb, i, t, c] == x[bb, t, i * 4 + c]
    # fp64 matmul of the block against a triple loop on a small case
    A = r.standard_normal((3, 4)); Bm = r.standard_normal((4, 5))
    C = np.zeros((3, 5))
    for i in range(3):
        for j in range(5):
            for kk in range(4):
                C[i, j] += A[i, kk] * Bm[kk, j]
    _close(A @ Bm, C, 1e-14, "matmul vs loops")


def pin_pages_shape_example(m):
    """The zyxy lecture's examples print torch.Size([2, 5, 8]) for batch 2,
    seq 5, d_model 8 (single head and N = 2 heads); see tests/golden."""
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")) as f:
        gold = json.load(f)
    ex = gold["zyxy_examples"]
    b, L, dm = ex["batch_size"], ex["seq_len"], ex["d_model"]
    r = np.random.default_rng(80)
    Q, K, V = (r.standard_normal((b, 1, L, dm)) for _ in range(3))
    o = m.retention_parallel(Q, K, V, np.array([ex["gamma"]]), None, 0)
    assert list(o.shape[:1]) + list(o.shape[2:]) == ex["printed_shape"]
    Qh = m.split_heads(r.standard_normal((b, L, dm)), ex["N"])
    o2 = m.retention_recurrent(Qh, Qh, Qh, np.array([0.9, 0.8]), None, 0)[0]
    assert list(np.transpose(o2, (0, 2, 1, 3)).reshape(b, L, dm).shape) == ex["printed_shape"]


def pin_layer_norm(m):
    """LayerNorm of the RetNet layer (§三.4): [1,2,3,4] has mean 2.5 and biased
    variance 1.25, so it maps to [-3,-1,1,3]/sqrt(5); rows are independent; eps
    enters under the square root; the affine is per channel; and LN(a x + c) =
    LN(x) for a > 0."""
    x = np.array([[1.0, 2.0, 3.0, 4.0], [10.0, 10.0, 10.0, 14.0]])
    y = m.layer_norm(x, 0.0)
    _close(y[0], np.array([-3, -1, 1, 3]) / np.sqrt(5.0), 1e-15, "LN row 0")
    _close(y[1], np.array([-1, -1, -1, 3]) / np.sqrt(3.0), 1e-15, "LN row 1")
    _close(m.layer_norm(np.array([1.0, -1.0]), 3.0), [0.5, -0.5], 1e-15, "LN eps")
    w = np.arange(1, 5, dtype=np.float64)
    bb = -np.arange(4, dtype=np.float64)
    _close(m.layer_norm(x, 0.0, w, bb), y * w + bb, 1e-15, "LN affine")
    r = _rand((3, 5, 16), 90)
    _close(m.layer_norm(2.5 * r + 7.0, 0.0), m.layer_norm(r, 0.0), 1e-12, "LN invariance")


def pin_gelu(m):
    """gelu(x) = x Phi(x) with the standard normal CDF Phi: gelu(0) = 0,
    gelu(1) = Phi(1) = 0.8413447460685429, gelu(-1) = -(1 - Phi(1)),
    gelu(2) = 2 Phi(2) = 2 * 0.9772498680518208 (textbook values of Phi);
    gelu(x) - gelu(-x) = x since Phi(x) + Phi(-x) = 1; gelu(40) = 40,
    gelu(-40) = 0.  FFN with identity weights is gelu itself (§三.4)."""
    g = m.gelu(np.array([0.0, 1.0, -1.0, 2.0, 40.0, -40.0]))
    assert g[0] == 0.0
    assert abs(g[1] - 0.8413447460685429) < 1e-15
    assert abs(g[2] + 0.15865525393145707) < 1e-15
    assert abs(g[3] - 1.9544997361036416) < 1e-14
    assert abs(g[4] - 40.0) < 1e-12 and abs(g[5]) < 1e-300
    x = _rand((1000,), 91, 3.0)
    _close(m.gelu(x) - m.gelu(-x), x, 1e-13, "gelu odd part")
    eye = np.eye(6)
    xx = _rand((2, 7, 6), 92)
    _close(m.ffn(xx, eye, eye), m.gelu(xx), 1e-15, "FFN identity")
    # the second weight is applied after gelu, the first before it
    W1 = np.diag(np.arange(1.0, 7.0))
    W2 = 2.0 * eye
    _close(m.ffn(xx, W1, W2), 2.0 * m.gelu(xx * np.arange(1.0, 7.0)), 1e-14, "FFN order")


def pin_retnet_layer(m):
    """One RetNet layer (§三.4), Y = MSR(LN(X)) + X, X' = FFN(LN(Y)) + Y:
    zero W_O and W_2 give X' = X; with W_2 = 0, X' - X = MSR(LN(X)) is
    unchanged by a positive rescaling of X (LN sits before MSR); with W_O = 0
    the same holds for the FFN branch; X' - Y is linear in W_2; and token t
    of X' depends on tokens <= t only."""
    b, L, dm, h, dk, dv, dff = 1, 13, 8, 2, 4, 4, 12
    r = np.random.default_rng(93)
    X = r.standard_normal((b, L, dm)) + 0.5
    WQ, WK = r.standard_normal((dm, h * dk)), r.standard_normal((dm, h * dk))
    WV, WG = r.standard_normal((dm, h * dv)), r.standard_normal((dm, h * dv))
    WO = r.standard_normal((h * dv, dm))
    W1, W2 = r.standard_normal((dm, dff)), r.standard_normal((dff, dm))
    th = _thetas(dk)
    flags = XPOS | NORM_ALL
    lay = lambda X_, WO_, W2_: m.retnet_layer(X_, (WQ, WK, WV, WG, WO_), W1, W2_, h, th, flags, 5, 0.0, 0.0)
    _close(lay(X, 0 * WO, 0 * W2), X, 0.0, "identity")
    y1 = lay(X, WO, 0 * W2) - X
    y2 = lay(3.0 * X, WO, 0 * W2) - 3.0 * X
    _close(y2, y1, 1e-11, "pre-norm MSR branch")
    assert np.max(np.abs(y1)) > 1e-3
    f1 = lay(X, 0 * WO, W2) - X
    f2 = lay(3.0 * X, 0 * WO, W2) - 3.0 * X
    _close(f2, f1, 1e-11, "pre-norm FFN branch")
    Y = lay(X, WO, 0 * W2)
    _close(lay(X, WO, 2.0 * W2) - Y, 2.0 * (lay(X, WO, W2) - Y), 1e-11, "linear in W_2")
    full = lay(X, WO, W2)
    X2 = X.copy(); X2[:, 9:] += 5.0
    _close(lay(X2, WO, W2)[:, :9], full[:, :9], 1e-12, "causal")


def _stack_params(r, n_layers, dm, h, dk, dv, dff):
    layers = []
    for _ in range(n_layers):
        msr_w = (0.5 * r.standard_normal((dm, h * dk)), 0.5 * r.standard_normal((dm, h * dk)),
                 0.5 * r.standard_normal((dm, h * dv)), 0.5 * r.standard_normal((dm, h * dv)),
                 0.3 * r.standard_normal((h * dv, dm)))
        W1, W2 = 0.4 * r.standard_normal((dm, dff)), 0.3 * r.standard_normal((dff, dm))
        ln1 = (1.0 + 0.2 * r.standard_normal(dm), 0.2 * r.standard_normal(dm))
        ln2 = (1.0 + 0.2 * r.standard_normal(dm), 0.2 * r.standard_normal(dm))
        layers.append((msr_w, W1, W2, ln1, ln2))
    return layers


def pin_stack_decode(m):
    """A stack of layers (§三.4) decoded token by token in the recurrent form
    (§2.2, each layer carrying its own (S, z)) equals the chunkwise forward
    of the stack at every position; a chunkwise prefill handing each layer's
    state to the decode continues the same sequence; the final states agree.
    The two paths share only LN, FFN and the gate; the retention, the head
    split and the state hand-over differ."""
    b, T, dm, h, dk, dv, dff, n_layers = 2, 9, 8, 2, 4, 4, 12, 2
    r = np.random.default_rng(107)
    layers = _stack_params(r, n_layers, dm, h, dk, dv, dff)
    X = r.standard_normal((b, T, dm))
    th = _thetas(dk)
    for flags in (XPOS | NORM_ALL, XPOS, NORM_SCORE):
        full, fst = m.retnet_stack(X, layers, h, th, flags, 4, 1e-5, 1e-5, return_states=True)
        states = m.zero_states(n_layers, b, h, dk, dv)
        for t in range(T):
            y, states = m.retnet_decode_step(X[:, t], layers, h, th, flags, 1e-5, 1e-5, states, t, t + 1)
            _close(y, full[:, t], 1e-10, f"decode token {t} flags {flags}")
        for (S, z), (S2, z2) in zip(states, fst):
            _close(S, S2, 1e-10, "final state S")
            _close(z, z2, 1e-10, "final key-sum z")
        P = 5
        _, pst = m.retnet_stack(X[:, :P], layers, h, th, flags, 3, 1e-5, 1e-5, return_states=True)
        for t in range(P, T):
            y, pst = m.retnet_decode_step(X[:, t], layers, h, th, flags, 1e-5, 1e-5, pst, t, t + 1)
            _close(y, full[:, t], 1e-10, f"prefill {P} then decode token {t}")
        # a prefilled prefix continued chunkwise is the same sequence too
        _, pst = m.retnet_stack(X[:, :P], layers, h, th, flags, 3, 1e-5, 1e-5, return_states=True)
        rest = m.retnet_stack(X[:, P:], layers, h, th, flags, 2, 1e-5, 1e-5, pos0=P, n_prev=P, states=pst)
        _close(rest, full[:, P:], 1e-10, "prefill then chunkwise continuation")
    # the stack is not trivially the identity, and layer 2 depends on layer 1
    assert np.max(np.abs(full - X)) > 1e-2
    one = m.retnet_stack(X, layers[1:], h, th, XPOS, 4, 1e-5, 1e-5)
    assert np.max(np.abs(one - full)) > 1e-3


def pin_backward(m):
    """The chunkwise backward's definition (gradients of the normalised
    retention): equal to central finite differences of the recurrent form
    (the definition, a different code path) for four flag sets, two of them
    with the score clamp active on some rows and inactive on others; and
    Euler's identity for homogeneous functions -- without the score
    normalisation O is of degree 1 in each of q, k and v, so
    sum(dq . q) = sum(dk . k) = sum(dv . v) = sum(dO . O); with the clamp
    active on every row O is of degree 0 in q and in k."""
    r = np.random.default_rng(211)
    b, h, L, dk, dv = 1, 2, 7, 4, 3
    th = _thetas(dk)
    g = m.gammas(h)
    eps = 1e-6
    for flags, qscale in ((0, 1.0), (XPOS, 1.0), (XPOS | NORM_ALL, 2.0), (XPOS | NORM_SCORE, 1.0)):
        q = r.standard_normal((b, h, L, dk)) * qscale
        k, v = r.standard_normal((b, h, L, dk)), r.standard_normal((b, h, L, dv))
        do = r.standard_normal((b, h, L, dv))
        if flags & NORM_SCORE:
            # keep every row away from the clamp's kink, and both branches in use
            pr = m.retention_parallel(q, k, np.ones((b, h, L, 1)), g, th, flags & ~NORM_SCORE, pos0=3)[..., 0]
            assert np.min(np.abs(np.abs(pr) - 1.0)) > 1e-3
            assert np.any(np.abs(pr) > 1.0) and np.any(np.abs(pr) < 1.0)
        loss = lambda q_, k_, v_: float(np.sum(do * m.retention_recurrent(q_, k_, v_, g, th, flags, pos0=3)[0]))
        grads = m.retention_parallel_bwd(q, k, v, do, g, th, flags, pos0=3)
        for which, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = [q, k, v]
                xp = x.copy(); xp[idx] += eps
                xm = x.copy(); xm[idx] -= eps
                args[which] = xp; fp = loss(*args)
                args[which] = xm; fm = loss(*args)
                fd[idx] = (fp - fm) / (2 * eps)
            _close(grads[which], fd, 1e-7, f"finite differences, input {which}, flags {flags}")
    # Euler's identity at a larger size
    b, h, L, dk, dv = 2, 3, 40, 8, 6
    th = _thetas(dk)
    g = m.gammas(h)
    q, k = r.standard_normal((b, h, L, dk)), r.standard_normal((b, h, L, dk))
    v, do = r.standard_normal((b, h, L, dv)), r.standard_normal((b, h, L, dv))
    for flags in (XPOS, XPOS | SCALE_QK | NORM_DROW):
        o = m.retention_parallel(q, k, v, g, th, flags)
        dq, dk_, dv_ = m.retention_parallel_bwd(q, k, v, do, g, th, flags)
        ref = np.sum(do * o)
        for x, dx in ((q, dq), (k, dk_), (v, dv_)):
            assert abs(np.sum(dx * x) - ref) <= 1e-10 * max(1.0, abs(ref)), "degree-1 homogeneity"
    # positive q, k (no rotation) make every score row sum large: the clamp
    # is active on every row
    flags = SCALE_QK | NORM_SCORE
    qb, kb = 50.0 * np.abs(q), np.abs(k)
    pr = m.retention_parallel(qb, kb, np.ones((b, h, L, 1)), g, th, SCALE_QK)[..., 0]
    assert np.all(np.abs(pr) > 1.0)
    o = m.retention_parallel(qb, kb, v, g, th, flags)
    dq, dk_, dv_ = m.retention_parallel_bwd(qb, kb, v, do, g, th, flags)
    assert abs(np.sum(dq * qb)) <= 1e-10 * np.sqrt(np.sum(dq * dq) * np.sum(qb * qb)), "degree-0 in q"
    assert abs(np.sum(dk_ * kb)) <= 1e-10 * np.sqrt(np.sum(dk_ * dk_) * np.sum(kb * kb)), "degree-0 in k"
    assert np.max(np.abs(dq)) > 1e-6
    assert abs(np.sum(dv_ * v) - np.sum(do * o)) <= 1e-10 * max(1.0, abs(np.sum(do * o))), "degree-1 in v"


ALL_PINS = [pin_gamma_theta, pin_forms_agree, pin_onehot_decay, pin_xpos_closed_form,
            pin_drow_scale_closed_form, pin_score_clamp, pin_groupnorm_invariance,
            pin_groupnorm_values, pin_swish, pin_relative_position, pin_split_resume,
            pin_causality_linearity, pin_decode_zero_kv, pin_decode_vs_chunkwise, pin_block,
            pin_pages_shape_example, pin_layer_norm, pin_gelu, pin_retnet_layer, pin_stack_decode, pin_backward]


def quick_forms(m):
    """A cheaper form-equivalence pass for the mutation tests."""
    pin_forms_agree(m, L=37, flags_list=(0, XPOS, XPOS | NORM_ALL, NORM_SCORE, NORM_DROW | SCALE_QK),
                    chunks=(1, 5, 16, 40), b=1, h=2)
