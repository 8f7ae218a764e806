"""Plain fp64 CPU oracle for RetNet multi-scale retention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, tables or helpers); the only thing both sides
share is the seeded input generator, which holds none of the method's
arithmetic.

Everything here is numpy in float64.  Inputs of any float dtype are promoted
exactly to float64 on entry.  The functions follow the pages' definitions in
the pages' order; where a page leaves a step open, the reading taken is stated
next to the code.  Sources (page title, section):

* RetNet reading notes (mzeromiko.github.io, "阅读笔记：RetNet"):
  §2.1 architecture motivation (the complex-phase derivation),
  §2.2 recurrent mode, §2.3 parallel mode, §2.4 chunkwise recurrent mode,
  §三.2 MSR module, §三.3 normalisation, §三.4 single-layer structure
  (LN, residuals and the gelu FFN around the MSR module; layers stacked).
* zyxy.net lecture ("RetNet（Retentive Network）：多尺度指数衰减…"), §5
  multi-scale grouping: the head split of d_model into contiguous column
  blocks, shape (batch, heads, seq, d_head).

Flags (a bitmask, the same values as the C ABI):
  XPOS = 1        rotate q and k by the position phase (§2.3, Theta_n = e^{i n theta})
  SCALE_QK = 2    QK^T -> QK^T / sqrt(d_k)                (§三.3, first factor)
  NORM_DROW = 4   D_nm -> D_nm / sqrt(sum_{i<=n} D_ni)     (§三.3, second factor)
  NORM_SCORE = 8  R_nm -> R_nm / max(|sum_i R_ni|, 1)      (§三.3, third factor)

Layout: q, k are [b, h, L, d_k]; v and outputs are [b, h, L, d_v]; the
recurrent state S is [b, h, d_k, d_v] and the key-sum z is [b, h, d_k].

Parity status of each function (what pins it) is recorded in the test files
under tests/ that start with ``test_oracle``.  Readings that are choices
rather than facts of the pages ("parity unpinned" by the pages themselves):
the real xPos layout (interleaved pairs, both q and k rotated by +p*theta),
GroupNorm epsilon and affine, the meaning of sigma in N(0, sigma), and for
the layer of §三.4 the LayerNorm variant (biased variance, eps, affine), the
exact gelu x Phi(x), and the FFN width (a parameter).
"""

import math

import numpy as np

XPOS = 1
SCALE_QK = 2
NORM_DROW = 4
NORM_SCORE = 8
NORM_ALL = SCALE_QK | NORM_DROW | NORM_SCORE


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def gammas(h):
    """Per-head decay of the MSR module (reading notes §三.2): 1 - 2^(-5-i)."""
    return 1.0 - 2.0 ** (-5.0 - np.arange(h, dtype=np.float64))


def thetas(d_k, base=10000.0):
    """Rotation frequencies theta_j = base^(-2j/d_k) for the d_k/2 pairs.

    The pages only say theta is a real vector (reading notes §2.1); this
    frequency ladder is the workload's stated choice.
    """
    j = np.arange(d_k // 2, dtype=np.float64)
    return base ** (-2.0 * j / d_k)


def xpos_rotate(x, positions, theta):
    """Multiply each complex pair of x by e^{i p theta_j} (reading notes §2.3).

    x: [..., L, d] with d even; positions: [L] absolute (0-based) positions.
    The pair (x_{2j}, x_{2j+1}) is read as the complex number
    x_{2j} + i x_{2j+1}; multiplying by e^{i phi} with phi = p * theta_j gives
      x'_{2j}   = x_{2j} cos phi - x_{2j+1} sin phi
      x'_{2j+1} = x_{2j} sin phi + x_{2j+1} cos phi.
    Rotating both q_n and k_m this way makes q'_n . k'_m equal the real part of
    (q_n e^{in theta})(k_m e^{im theta})^dagger (§2.1), a function of n - m only.
    """
    x = _f64(x)
    phi = np.asarray(positions, dtype=np.float64)[:, None] * np.asarray(theta, dtype=np.float64)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def _row_scale(flags, gamma, d_k, n):
    """Per-row positive scalar s = (1/sqrt(d_k)) * sqrt((1-g)/(1-g^n)).

    gamma: [h]; n: array of token counts (n >= 1) -> returns [h, len(n)].
    sum_{i=1}^{n} gamma^{n-i} = (1 - gamma^n)/(1 - gamma) is the D row sum of
    §三.3 for a row that has seen n tokens (a geometric series).
    """
    gamma = _f64(gamma)
    n = np.asarray(n, dtype=np.float64)
    s = np.ones((gamma.shape[0], n.shape[0]))
    if flags & SCALE_QK:
        s = s / np.sqrt(d_k)
    if flags & NORM_DROW:
        s = s * np.sqrt((1.0 - gamma[:, None]) / (1.0 - gamma[:, None] ** n[None, :]))
    return s


def _finish(num, den, s, flags):
    """o = s*num, divided by max(|s*den|, 1) when NORM_SCORE (§三.3 third factor).

    num: [b,h,L,dv]; den: [b,h,L] (unscaled row sum of the retention scores);
    s: [h, L].
    """
    o = num * s[None, :, :, None]
    if flags & NORM_SCORE:
        o = o / np.maximum(np.abs(den * s[None, :, :]), 1.0)[..., None]
    return o


def retention_recurrent(q, k, v, gamma, theta, flags, pos0=0, n_prev=0,
                        state_in=None, z_in=None):
    """Recurrent form, the definition (reading notes §2.2 with §2.3/§三.3).

    For each position p (0-based) with n = n_prev + p + 1 tokens seen:
      S <- gamma S + k'_p^T v_p ,  z <- gamma z + k'_p      (state includes token p)
      num = q'_p S ,  den = q'_p . z = sum_{m<=p} gamma^{p-m} q'_p . k'_m
      o_p = s num / max(|s den|, 1)   (the division only with NORM_SCORE)
    where ' marks the xPos rotation at absolute position pos0 + p.
    Returns (o [b,h,L,dv], S [b,h,dk,dv], z [b,h,dk]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    gamma = _f64(gamma)
    b, h, L, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((b, h, dk, dv)) if state_in is None else _f64(state_in).copy()
    z = np.zeros((b, h, dk)) if z_in is None else _f64(z_in).copy()
    o = np.empty((b, h, L, dv))
    g4 = gamma[None, :, None, None]
    g3 = gamma[None, :, None]
    for p in range(L):
        qp, kp = q[:, :, p, :], k[:, :, p, :]
        if flags & XPOS:
            pp = np.array([pos0 + p])
            qp = xpos_rotate(qp[:, :, None, :], pp, theta)[:, :, 0, :]
            kp = xpos_rotate(kp[:, :, None, :], pp, theta)[:, :, 0, :]
        S = g4 * S + kp[:, :, :, None] * v[:, :, p, None, :]
        z = g3 * z + kp
        num = np.einsum('bhd,bhde->bhe', qp, S)
        den = np.einsum('bhd,bhd->bh', qp, z)
        s = _row_scale(flags, gamma, dk, [n_prev + p + 1])
        o[:, :, p, :] = _finish(num[:, :, None, :], den[:, :, None], s, flags)[:, :, 0, :]
    return o, S, z


def retention_parallel(q, k, v, gamma, theta, flags, pos0=0):
    """Parallel form for a fresh sequence, brute force O(L^2) (§2.3 + §三.3).

      Q' = Q (.) Theta, K' = K (.) conj(Theta),  D_nm = gamma^(n-m) (n >= m) else 0
      QK^T -> QK^T / sqrt(d_k)
      D~_nm = D_nm / sqrt(sum_{i=1}^{n} D_ni)          (the D row sum, summed here)
      R = (Q'K'^T) (.) D~ ,   R~_nm = R_nm / max(|sum_i R_ni|, 1)
      O = R~ V
    The normalisers are computed as explicit row sums of the matrices, not
    through a closed form, so this is an independent check of the others.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    gamma = _f64(gamma)
    b, h, L, dk = q.shape
    if flags & XPOS:
        pos = pos0 + np.arange(L)
        q = xpos_rotate(q, pos, theta)
        k = xpos_rotate(k, pos, theta)
    scores = q @ np.swapaxes(k, -1, -2)                     # [b,h,L,L]
    if flags & SCALE_QK:
        scores = scores / np.sqrt(dk)
    n = np.arange(L)
    diff = n[:, None] - n[None, :]
    D = np.where(diff[None] >= 0, gamma[:, None, None] ** np.maximum(diff, 0)[None], 0.0)  # [h,L,L]
    if flags & NORM_DROW:
        D = D / np.sqrt(D.sum(axis=-1, keepdims=True))
    R = scores * D[None]
    if flags & NORM_SCORE:
        R = R / np.maximum(np.abs(R.sum(axis=-1, keepdims=True)), 1.0)
    return R @ v


def retention_chunkwise(q, k, v, gamma, theta, flags, chunk, pos0=0, n_prev=0,
                        state_in=None, z_in=None):
    """Chunkwise recurrent form (reading notes §2.4), normalised per §三.3.

    For chunk i covering rows [iB, iB + B_i) (B_i = B except a ragged last chunk):
      inner = (Q_[i] K_[i]^T (.) D) V_[i]          D_jl = gamma^(j-l), j >= l
      cross = (Q_[i] R_{i-1}) (.) xi               xi_j = gamma^(j+1)
      R_i   = K_[i]^T (V_[i] (.) zeta) + gamma^(B_i) R_{i-1},  zeta_j = gamma^(B_i-j-1)
    The normalisers are defined on the parallel form; the chunkwise result
    must equal the normalised parallel one, so the row sum of the scores is
    carried across chunks with the key-sum z_i = K_[i]^T zeta + gamma^(B_i) z_{i-1}
    (den = inner row sum + xi * (Q_[i] . z_{i-1})), and the D-row factor uses
    the row's global token count.  Returns (o, S, z) like the recurrent form.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    gamma = _f64(gamma)
    b, h, L, dk = q.shape
    dv = v.shape[-1]
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    R = np.zeros((b, h, dk, dv)) if state_in is None else _f64(state_in).copy()
    z = np.zeros((b, h, dk)) if z_in is None else _f64(z_in).copy()
    if flags & XPOS:
        pos = pos0 + np.arange(L)
        q = xpos_rotate(q, pos, theta)
        k = xpos_rotate(k, pos, theta)
    o = np.empty((b, h, L, dv))
    g = gamma[:, None, None]
    for c0 in range(0, L, chunk):
        Bc = min(chunk, L - c0)
        Qc, Kc, Vc = q[:, :, c0:c0 + Bc], k[:, :, c0:c0 + Bc], v[:, :, c0:c0 + Bc]
        j = np.arange(Bc)
        diff = j[:, None] - j[None, :]
        D = np.where(diff[None] >= 0, g ** np.maximum(diff, 0)[None], 0.0)     # [h,Bc,Bc]
        P = (Qc @ np.swapaxes(Kc, -1, -2)) * D[None]
        xi = gamma[:, None] ** (j[None, :] + 1.0)                              # [h,Bc]
        num = P @ Vc + (Qc @ R) * xi[None, :, :, None]
        den = P.sum(axis=-1) + np.einsum('bhjd,bhd->bhj', Qc, z) * xi[None]
        s = _row_scale(flags, gamma, dk, n_prev + c0 + j + 1)
        o[:, :, c0:c0 + Bc] = _finish(num, den, s, flags)
        zeta = gamma[:, None] ** (Bc - j[None, :] - 1.0)                       # [h,Bc]
        gB = (gamma ** Bc)[None, :, None, None]
        R = np.swapaxes(Kc, -1, -2) @ (Vc * zeta[None, :, :, None]) + gB * R
        z = np.einsum('bhjd,bhj->bhd', Kc, np.broadcast_to(zeta[None], Kc.shape[:3])) + gB[..., 0] * z
    return o, R, z


def retention_parallel_bwd(q, k, v, do, gamma, theta, flags, pos0=0):
    """Gradients dL/dq, dL/dk, dL/dv of the normalised retention of a fresh
    sequence, given dL/dO (the chunkwise backward's definition: the training
    path of §三.5 and §四.3 differentiates the forward of §2.3 with §三.3's normalisers).

    Written out on the parallel form: with q', k' the rotated inputs,
      A_pm   = (q'_p . k'_m) gamma^(p-m)  for m <= p         (unscaled scores)
      num_p  = sum_m A_pm v_m,   den_p = sum_m A_pm
      o_p    = s_p num_p / n_p,  n_p = max(|s_p den_p|, 1) with NORM_SCORE, else 1
    the chain rule gives
      dL/dnum_p = s_p g_p / n_p
      dL/dden_p = -s_p^2 sign(den_p) (g_p . num_p) / n_p^2  where |s_p den_p| > 1, else 0
      dL/dA_pm  = dL/dnum_p . v_m + dL/dden_p
      dq'_p = sum_m dL/dA_pm gamma^(p-m) k'_m,  dk'_m = sum_p dL/dA_pm gamma^(p-m) q'_p
      dv_m  = sum_p A_pm dL/dnum_p
    and dq, dk rotate dq', dk' back by -p theta (the rotation is orthogonal).
    Reading: nothing is detached (the pages leave it open); on the clamp's
    boundary |s den| = 1 the constant branch is taken.  Returns (dq, dk, dv).
    """
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(do)
    gamma = _f64(gamma)
    b, h, L, dk = q.shape
    pos = pos0 + np.arange(L)
    if flags & XPOS:
        q = xpos_rotate(q, pos, theta)
        k = xpos_rotate(k, pos, theta)
    n = np.arange(L)
    diff = n[:, None] - n[None, :]
    D = np.where(diff[None] >= 0, gamma[:, None, None] ** np.maximum(diff, 0)[None], 0.0)    # [h,L,L]
    A = (q @ np.swapaxes(k, -1, -2)) * D[None]
    num = A @ v
    den = A.sum(axis=-1)
    s = _row_scale(flags, gamma, dk, n + 1)[None]                                         # [1,h,L]
    if flags & NORM_SCORE:
        nrm = np.maximum(np.abs(s * den), 1.0)
        active = np.abs(s * den) > 1.0
        gden = np.where(active, -(s ** 2) * np.sign(den) * np.einsum('bhpe,bhpe->bhp', g, num) / nrm ** 2, 0.0)
    else:
        nrm = np.ones_like(den)
        gden = np.zeros_like(den)
    gnum = (s / nrm)[..., None] * g
    dA = gnum @ np.swapaxes(v, -1, -2) + gden[..., None]
    dS = dA * D[None]
    dqr = dS @ k
    dkr = np.swapaxes(dS, -1, -2) @ q
    dv = np.swapaxes(A, -1, -2) @ gnum
    if flags & XPOS:
        dqr = xpos_rotate(dqr, -pos, theta)
        dkr = xpos_rotate(dkr, -pos, theta)
    return dqr, dkr, dv


def recurrent_step(q, k, v, S, gamma, theta, flags, pos, n_tokens, z=None):
    """One decode step of the recurrent form (reading notes §2.2).

    q, k: [b,h,dk]; v: [b,h,dv]; S: [b,h,dk,dv]; z: [b,h,dk] or None.
    S <- gamma S + k'^T v (the current token included), o = q' S, and with a
    key-sum z the row normalisers of §三.3 for a row that has seen n_tokens.
    Returns (o [b,h,dv], S_new, z_new or None).  Inputs are not modified.
    """
    q, k, v, S = _f64(q), _f64(k), _f64(v), _f64(S)
    gamma = _f64(gamma)
    dk = q.shape[-1]
    if flags & XPOS:
        pp = np.array([pos])
        q = xpos_rotate(q[:, :, None, :], pp, theta)[:, :, 0, :]
        k = xpos_rotate(k[:, :, None, :], pp, theta)[:, :, 0, :]
    S = gamma[None, :, None, None] * S + k[:, :, :, None] * v[:, :, None, :]
    num = np.einsum('bhd,bhde->bhe', q, S)
    if z is not None:
        z = gamma[None, :, None] * _f64(z) + k
        den = np.einsum('bhd,bhd->bh', q, z)
    else:
        if flags & NORM_SCORE:
            raise ValueError("NORM_SCORE needs the key-sum z")
        den = np.zeros(num.shape[:2])
    s = _row_scale(flags, gamma, dk, [n_tokens])
    o = _finish(num[:, :, None, :], den[:, :, None], s, flags)[:, :, 0, :]
    return o, S, z


def swish(x):
    """swish(x) = x * sigmoid(x), the gate of the MSR module (§三.2), beta = 1."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def group_norm_heads(y, eps, weight=None, bias=None):
    """GroupNorm_h over the concatenated heads (§三.2): one group per head.

    y: [b, h, L, dv] (head outputs).  For every (b, token, head) the dv values
    are normalised with their own mean and biased variance, then the optional
    per-channel affine [h*dv] is applied.  Returns [b, L, h*dv] (Concat order:
    head i occupies columns [i*dv, (i+1)*dv)).
    """
    y = _f64(y)
    b, h, L, dv = y.shape
    yt = np.transpose(y, (0, 2, 1, 3))                       # [b,L,h,dv]
    mu = yt.mean(axis=-1, keepdims=True)
    var = ((yt - mu) ** 2).mean(axis=-1, keepdims=True)
    yhat = ((yt - mu) / np.sqrt(var + eps)).reshape(b, L, h * dv)
    if weight is not None:
        yhat = yhat * _f64(weight)
    if bias is not None:
        yhat = yhat + _f64(bias)
    return yhat


def gate_norm(y, g, eps, weight=None, bias=None):
    """swish(G) (.) GroupNorm_h(Y) of the MSR module (§三.2), before W_O.

    y: [b,h,L,dv] head outputs; g: [b,L,h*dv] = X W_G.  Returns [b,L,h*dv].
    """
    return swish(g) * group_norm_heads(y, eps, weight, bias)


def split_heads(x, h):
    """[b, L, h*d] -> [b, h, L, d]: head i takes columns [i*d, (i+1)*d)."""
    b, L, hd = x.shape
    return np.transpose(x.reshape(b, L, h, hd // h), (0, 2, 1, 3))


def msr_forward(X, WQ, WK, WV, WG, WO, h, theta, flags, chunk, eps, pos0=0, n_prev=0, state=None,
                return_state=False):
    """Gated multi-scale retention block forward (reading notes §三.2).

      Q = X W_Q, K = X W_K, V = X W_V  (§2.1), heads split as contiguous columns
      head_i = Retention(X, gamma_i)   (chunkwise form, per-head gamma_i)
      Y = GroupNorm_h(Concat(heads));  MSR(X) = (swish(X W_G) (.) Y) W_O
    X: [b, L, d_model]; W_Q, W_K: [d_model, h*dk]; W_V, W_G: [d_model, h*dv];
    W_O: [h*dv, d_model].  Returns [b, L, d_model], and with return_state the
    heads' final (S, z) as well.  state = (S, z) continues a sequence whose
    first n_prev tokens (phases from pos0 - n_prev) are in it.
    """
    X = _f64(X)
    Q = split_heads(X @ _f64(WQ), h)
    K = split_heads(X @ _f64(WK), h)
    V = split_heads(X @ _f64(WV), h)
    G = X @ _f64(WG)
    S0, z0 = (None, None) if state is None else state
    Y, S, z = retention_chunkwise(Q, K, V, gammas(h), theta, flags, chunk, pos0=pos0, n_prev=n_prev,
                                  state_in=S0, z_in=z0)
    out = gate_norm(Y, G, eps) @ _f64(WO)
    return (out, (S, z)) if return_state else out


# ---------------------------------------------------------------------------
# One RetNet layer (reading notes §三.4, the single-layer structure):
#   Y = MSR(LN(X)) + X,   X' = FFN(LN(Y)) + Y,   FFN(X) = gelu(X W_1) W_2
# The page names LN and gelu without their variants; the readings taken are
# LayerNorm over the model width with the biased variance, eps under the
# square root and an optional per-channel affine, and the exact gelu
# x Phi(x).  The FFN width is a parameter (the page does not state it).
# ---------------------------------------------------------------------------

_ERF = np.vectorize(math.erf, otypes=[np.float64])


def _erf(x):
    """erf of every element, by the standard library's math.erf (correctly
    rounded to within an ulp or so)."""
    return _ERF(_f64(x))


def layer_norm(x, eps, weight=None, bias=None):
    """LN over the last axis (d_model): (x - mean) / sqrt(biased var + eps),
    then the optional per-channel affine (§三.4; variant: see above)."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if weight is not None:
        y = y * _f64(weight)
    if bias is not None:
        y = y + _f64(bias)
    return y


def gelu(x):
    """gelu(x) = x Phi(x) = x (1 + erf(x / sqrt 2)) / 2 (§三.4, exact form)."""
    x = _f64(x)
    return 0.5 * x * (1.0 + _erf(x / np.sqrt(2.0)))


def ffn(X, W1, W2):
    """FFN(X) = gelu(X W_1) W_2 (§三.4).  W_1: [d_model, d_ff], W_2: [d_ff, d_model]."""
    return gelu(_f64(X) @ _f64(W1)) @ _f64(W2)


def retnet_layer(X, msr_w, W1, W2, h, theta, flags, chunk, gn_eps, ln_eps,
                 ln1=(None, None), ln2=(None, None), pos0=0, n_prev=0, state=None, return_state=False):
    """One RetNet layer (§三.4): Y = MSR(LN(X)) + X;  X' = FFN(LN(Y)) + Y.

    msr_w = (W_Q, W_K, W_V, W_G, W_O) as in msr_forward; ln1 / ln2 are the
    (weight, bias) of the two LayerNorms (None = 1 and 0).  Returns X' of the
    shape of X (and the retention state, as msr_forward, with return_state)."""
    X = _f64(X)
    WQ, WK, WV, WG, WO = msr_w
    m, st = msr_forward(layer_norm(X, ln_eps, *ln1), WQ, WK, WV, WG, WO, h, theta, flags, chunk, gn_eps,
                        pos0=pos0, n_prev=n_prev, state=state, return_state=True)
    Y = m + X
    out = ffn(layer_norm(Y, ln_eps, *ln2), W1, W2) + Y
    return (out, st) if return_state else out


# ---------------------------------------------------------------------------
# A stack of layers and its token-by-token decode.  The model stacks identical
# layers (§三.4); decoding runs each layer's MSR in the recurrent form (§2.2),
# one token at a time, each layer carrying its own heads' state (S, z):
# [b,h,dk,dv] and [b,h,dk].  A layer's parameters are the tuple
# (msr_w, W1, W2, ln1, ln2) of retnet_layer.
# ---------------------------------------------------------------------------

def retnet_stack(X, layers, h, theta, flags, chunk, gn_eps, ln_eps, pos0=0, n_prev=0, states=None,
                 return_states=False):
    """The layers applied in order (chunkwise MSR).  states: one (S, z) per
    layer to continue from, or None; with return_states the layers' final
    states are returned too."""
    X = _f64(X)
    out_states = []
    for i, (msr_w, W1, W2, ln1, ln2) in enumerate(layers):
        X, st = retnet_layer(X, msr_w, W1, W2, h, theta, flags, chunk, gn_eps, ln_eps, ln1, ln2, pos0=pos0,
                             n_prev=n_prev, state=None if states is None else states[i], return_state=True)
        out_states.append(st)
    return (X, out_states) if return_states else X


def msr_step(x, WQ, WK, WV, WG, WO, h, theta, flags, eps, state, pos, n_tokens):
    """One token of the MSR module in the recurrent form (§三.2 with §2.2).

    x: [b, d_model]; state = (S, z) of the h heads.  The projections are split
    into heads like split_heads (head i takes columns [i*d, (i+1)*d)); each
    head takes one recurrent_step; GroupNorm and the gate act on the one
    token.  Returns ([b, d_model], (S_new, z_new))."""
    x = _f64(x)
    b = x.shape[0]
    Q, K, V = x @ _f64(WQ), x @ _f64(WK), x @ _f64(WV)
    dk, dv = Q.shape[1] // h, V.shape[1] // h
    S, z = state
    o, S, z = recurrent_step(Q.reshape(b, h, dk), K.reshape(b, h, dk), V.reshape(b, h, dv), S, gammas(h), theta,
                             flags, pos, n_tokens, z)
    Z = gate_norm(o[:, :, None, :], (x @ _f64(WG))[:, None, :], eps)[:, 0]
    return Z @ _f64(WO), (S, z)


def retnet_decode_step(x, layers, h, theta, flags, gn_eps, ln_eps, states, pos, n_tokens):
    """One token through the stack: for each layer Y = MSR_step(LN(x)) + x,
    x <- FFN(LN(Y)) + Y.  x: [b, d_model]; states: one (S, z) per layer.
    Returns (x', new states)."""
    x = _f64(x)
    new_states = []
    for (msr_w, W1, W2, ln1, ln2), st in zip(layers, states):
        m, st = msr_step(layer_norm(x, ln_eps, *ln1), *msr_w, h, theta, flags, gn_eps, st, pos, n_tokens)
        y = m + x
        x = ffn(layer_norm(y, ln_eps, *ln2), W1, W2) + y
        new_states.append(st)
    return x, new_states


def zero_states(n_layers, b, h, dk, dv):
    """Empty per-layer states (S, z) for a fresh sequence."""
    return [(np.zeros((b, h, dk, dv)), np.zeros((b, h, dk))) for _ in range(n_layers)]
