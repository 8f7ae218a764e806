"""ctypes binding of libretention.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers, strides and the current HIP stream to the C ABI declared in
include/retention.h, and raises RuntimeError with the library's message on a
non-OK status.  torch provides memory and streams; all computation happens in
the library's HIP kernels.  There is no fallback: if the library is missing
the import fails.
"""
import ctypes
import functools
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libretention.so")

XPOS, SCALE_QK, NORM_DROW, NORM_SCORE = 1, 2, 4, 8
NORM_ALL = SCALE_QK | NORM_DROW | NORM_SCORE
RET_F32, RET_BF16, RET_F16 = 0, 1, 2
STATUS = {0: "RET_OK", 1: "RET_E_INVAL", 2: "RET_E_UNSUPPORTED", 3: "RET_E_ALIGN",
          4: "RET_E_WORKSPACE", 5: "RET_E_HIP", 6: "RET_E_RANGE"}


class Strides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64)]


def load_library(path=LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m linear_attention_sequence_retention_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, u32, f32, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint,
                                  ctypes.c_float, ctypes.c_size_t)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.retention_chunkwise_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                            i32, i32, i32, i32, i32, i32, dp, dp, i64, i64, u32,
                                            i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.retention_chunkwise_fwd.restype = i32
    lib.retention_chunkwise_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, u32]
    lib.retention_chunkwise_workspace_bytes.restype = sz
    lib.retention_recurrent_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, dp, dp,
                                             i64, i64, u32, i32, i32, vp]
    lib.retention_recurrent_step.restype = i32
    lib.msr_gate_norm.argtypes = [vp, Strides, vp, vp, i32, i32, i32, i32, vp, vp, f32,
                                  i32, i32, i32, vp]
    lib.msr_gate_norm.restype = i32
    lib.msr_gemm.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp]
    lib.msr_gemm.restype = i32
    lib.msr_gemm_bf16.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    lib.msr_gemm_bf16.restype = i32
    lib.retention_parallel_fwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                           i32, i32, i32, i32, i32, dp, dp, i64, u32, i32, i32, vp, sz, vp]
    lib.retention_parallel_fwd.restype = i32
    lib.retention_parallel_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, u32]
    lib.retention_parallel_workspace_bytes.restype = sz
    lib.retention_chunkwise_bwd.argtypes = [vp, Strides, vp, Strides, vp, Strides, vp, Strides,
                                            vp, Strides, vp, Strides, vp, Strides,
                                            i32, i32, i32, i32, i32, i32, dp, dp, i64, u32, i32, i32, vp, sz, vp]
    lib.retention_chunkwise_bwd.restype = i32
    lib.retention_chunkwise_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.retention_chunkwise_bwd_workspace_bytes.restype = sz
    lib.msr_gemm_ex.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, u32, vp]
    lib.msr_gemm_ex.restype = i32
    lib.msr_gemm_ws.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, u32, vp, sz, vp]
    lib.msr_gemm_ws.restype = i32
    lib.msr_gemm_scratch.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, u32, vp]
    lib.msr_gemm_scratch.restype = i32
    lib.msr_gemm_workspace_bytes.argtypes = [i32, i32, i32]
    lib.msr_gemm_workspace_bytes.restype = sz
    lib.ret_layer_norm.argtypes = [vp, vp, i32, i32, vp, vp, f32, i32, i32, vp]
    lib.ret_layer_norm.restype = i32
    lib.ret_calib_copy.argtypes = [vp, vp, sz, vp]
    lib.ret_calib_copy.restype = i32
    lib.ret_calib_mfma.argtypes = [vp, i32, i32, vp]
    lib.ret_calib_mfma.restype = i32
    lib.retention_range_status.argtypes = [vp]
    lib.retention_range_status.restype = i32
    lib.retention_last_error.argtypes = []
    lib.retention_last_error.restype = ctypes.c_char_p
    lib.retention_abi_version.argtypes = []
    lib.retention_abi_version.restype = i32
    return lib


LIB = load_library()
LIB_SCRATCH_BYTES = 32 << 20          # MSR_GEMM_SCRATCH_BYTES of include/retention.h


def _check(status, what):
    if status != 0:
        msg = LIB.retention_last_error().decode()
        raise RuntimeError(f"{what} failed with {STATUS.get(status, status)}: {msg}")


def range_status(stream=None):
    """None when no retention call on the current device wrote a non-finite
    value since the last query, else the library's message naming the forward
    and / or backward call (the record is cleared; the stream is waited for)."""
    st = LIB.retention_range_status(_stream(stream))
    if st == 6:
        return LIB.retention_last_error().decode()
    _check(st, "retention_range_status")
    return None


def _dt(t):
    if t.dtype == torch.bfloat16:
        return RET_BF16
    if t.dtype == torch.float32:
        return RET_F32
    if t.dtype == torch.float16:
        return RET_F16
    raise TypeError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")


def _torch_dt(code):
    return {RET_BF16: torch.bfloat16, RET_F16: torch.float16}.get(code, torch.float32)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _strides4(t, name):
    if t.dim() != 4 or t.stride(-1) != 1:
        raise ValueError(f"{name} must be a 4-D [b,h,L,d] view with a contiguous last axis")
    return Strides(t.stride(0), t.stride(1), t.stride(2))


def _f64(a, n, name):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if a.shape != (n,):
        raise ValueError(f"{name} must have shape ({n},)")
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def chunkwise_workspace_bytes(b, h, L, d_k, d_v, chunk, flags):
    return int(LIB.retention_chunkwise_workspace_bytes(b, h, L, d_k, d_v, chunk, flags))


def chunkwise_fwd(q, k, v, gamma, theta, chunk, flags, pos0=0, n_prev=0, state_in=None,
                  z_in=None, state_out=None, z_out=None, out=None, out_dtype=None,
                  workspace=None, stream=None):
    """O = chunkwise retention of q, k, v ([b,h,L,d] views on the GPU).

    Returns ``out`` (allocated as [b,h,L,d_v] of ``out_dtype`` when None).
    ``state_out`` / ``z_out`` (float32 [b,h,d_k,d_v] / [b,h,d_k]) are filled
    when given.
    """
    b, h, L, dk = q.shape
    dv = v.shape[-1]
    in_dt = _dt(q)
    if _dt(k) != in_dt or _dt(v) != in_dt:
        raise TypeError("q, k and v must share one dtype")
    if out is None:
        od = _torch_dt(in_dt) if out_dtype is None else out_dtype
        out = torch.empty((b, h, L, dv), dtype=od, device=q.device)
    g, gp = _f64(gamma, h, "gamma")
    th, tp = (None, None) if theta is None else _f64(theta, dk // 2, "theta")
    need = chunkwise_workspace_bytes(b, h, L, dk, dv, chunk, flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    for t in (state_in, z_in, state_out, z_out):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise TypeError("state and key-sum buffers must be contiguous float32")
    st = LIB.retention_chunkwise_fwd(
        _ptr(q), _strides4(q, "q"), _ptr(k), _strides4(k, "k"), _ptr(v), _strides4(v, "v"),
        _ptr(out), _strides4(out, "o"), b, h, L, dk, dv, chunk, gp, tp, pos0, n_prev, flags,
        in_dt, _dt(out), _ptr(state_in), _ptr(state_out), _ptr(z_in), _ptr(z_out),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _check(st, "retention_chunkwise_fwd")
    return out


def parallel_fwd(q, k, v, gamma, theta, flags, pos0=0, out=None, out_dtype=None, workspace=None, stream=None):
    """O = the parallel form of retention ([b,h,L,d] views on the GPU) for a
    fresh sequence: the whole causal L x L score matrix as one chunk."""
    b, h, L, dk = q.shape
    dv = v.shape[-1]
    in_dt = _dt(q)
    if _dt(k) != in_dt or _dt(v) != in_dt:
        raise TypeError("q, k and v must share one dtype")
    if out is None:
        od = _torch_dt(in_dt) if out_dtype is None else out_dtype
        out = torch.empty((b, h, L, dv), dtype=od, device=q.device)
    g, gp = _f64(gamma, h, "gamma")
    th, tp = (None, None) if theta is None else _f64(theta, dk // 2, "theta")
    need = LIB.retention_parallel_workspace_bytes(b, h, L, dk, dv, in_dt, flags)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = LIB.retention_parallel_fwd(
        _ptr(q), _strides4(q, "q"), _ptr(k), _strides4(k, "k"), _ptr(v), _strides4(v, "v"),
        _ptr(out), _strides4(out, "o"), b, h, L, dk, dv, gp, tp, pos0, flags, in_dt, _dt(out),
        _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    _check(st, "retention_parallel_fwd")
    return out


def chunkwise_bwd_workspace_bytes(b, h, L, dk, dv, chunk):
    return LIB.retention_chunkwise_bwd_workspace_bytes(b, h, L, dk, dv, chunk)


def chunkwise_bwd(q, k, v, dout, gamma, theta, chunk, flags, pos0=0, dq=None, dk=None, dv=None,
                  grad_dtype=torch.float32, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of chunkwise_fwd for a fresh sequence given
    dout = dL/dO ([b,h,L,d] views of one bf16 or fp16 dtype).  chunk is the
    backward's own chunk size (a multiple of 64)."""
    b, h, L, d_k = q.shape
    d_v = v.shape[-1]
    in_dt = _dt(q)
    if _dt(k) != in_dt or _dt(v) != in_dt or _dt(dout) != in_dt:
        raise TypeError("q, k, v and dout must share one dtype")
    dq = torch.empty((b, h, L, d_k), dtype=grad_dtype, device=q.device) if dq is None else dq
    dk = torch.empty((b, h, L, d_k), dtype=grad_dtype, device=q.device) if dk is None else dk
    dv = torch.empty((b, h, L, d_v), dtype=grad_dtype, device=q.device) if dv is None else dv
    if _dt(dk) != _dt(dq) or _dt(dv) != _dt(dq):
        raise TypeError("dq, dk and dv must share one dtype")
    g, gp = _f64(gamma, h, "gamma")
    th, tp = (None, None) if theta is None else _f64(theta, d_k // 2, "theta")
    need = chunkwise_bwd_workspace_bytes(b, h, L, d_k, d_v, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = LIB.retention_chunkwise_bwd(
        _ptr(q), _strides4(q, "q"), _ptr(k), _strides4(k, "k"), _ptr(v), _strides4(v, "v"),
        _ptr(dout), _strides4(dout, "dout"), _ptr(dq), _strides4(dq, "dq"), _ptr(dk), _strides4(dk, "dk"),
        _ptr(dv), _strides4(dv, "dv"), b, h, L, d_k, d_v, chunk, gp, tp, pos0, flags, in_dt, _dt(dq),
        _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "retention_chunkwise_bwd")
    return dq, dk, dv


def recurrent_step(q, k, v, S, gamma, theta, pos, n_tokens, flags, z=None, out=None,
                   out_dtype=torch.float32, stream=None):
    """One decode step; S (and z) are updated in place.  q, k: [b,h,d_k]; v: [b,h,d_v]."""
    b, h, dk = q.shape
    dv = v.shape[-1]
    if out is None:
        out = torch.empty((b, h, dv), dtype=out_dtype, device=q.device)
    g, gp = _f64(gamma, h, "gamma")
    th, tp = (None, None) if theta is None else _f64(theta, dk // 2, "theta")
    for t in (q, k, v, S, out) + ((z,) if z is not None else ()):
        if not t.is_contiguous():
            raise ValueError("recurrent_step needs contiguous tensors")
    st = LIB.retention_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(S), _ptr(z), _ptr(out),
                                      b, h, dk, dv, gp, tp, pos, n_tokens, flags, _dt(q), _dt(out),
                                      _stream(stream))
    _check(st, "retention_recurrent_step")
    return out


def gate_norm(y, g, eps, weight=None, bias=None, out=None, out_dtype=None, stream=None):
    """swish(g) * GroupNorm_h(y): y [b,h,L,d_v] (view), g [b,L,h*d_v] -> [b,L,h*d_v]."""
    b, h, L, dv = y.shape
    if out is None:
        out = torch.empty((b, L, h * dv), dtype=g.dtype if out_dtype is None else out_dtype, device=y.device)
    if not g.is_contiguous() or not out.is_contiguous():
        raise ValueError("g and out must be contiguous")
    st = LIB.msr_gate_norm(_ptr(y), _strides4(y, "y"), _ptr(g), _ptr(out), b, L, h, dv,
                           _ptr(weight), _ptr(bias), float(eps), _dt(y), _dt(g), _dt(out), _stream(stream))
    _check(st, "msr_gate_norm")
    return out


def gemm_workspace_bytes(M, N, K):
    return int(LIB.msr_gemm_workspace_bytes(M, N, K))


def gemm(a, b_nk, out=None, out_dtype=torch.bfloat16, residual=None, gelu=False, workspace=None, stream=None):
    """C = act(a . b_nk^T) (+ residual) for a [M, K] (bf16 or fp16) and a bf16
    weight b_nk [N, K]; act is the exact gelu when gelu is set, and residual
    ([M, N], float32, bf16 or fp16, added in fp32) may be out itself.  With
    M <= 128 (a decode step) and K a multiple of 128 the split-K path runs
    (msr_gemm_ws) in workspace, a uint8 device tensor of at least
    gemm_workspace_bytes(M, N, K) bytes, allocated here when not given."""
    if a.dtype not in (torch.bfloat16, torch.float16) or b_nk.dtype != torch.bfloat16:
        raise TypeError("gemm takes a bf16 or fp16 A and a bf16 weight")
    if not a.is_contiguous() or not b_nk.is_contiguous():
        raise ValueError("gemm needs contiguous operands")
    M, K = a.shape
    N = b_nk.shape[0]
    if b_nk.shape[1] != K:
        raise ValueError("inner dimensions differ")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    if residual is not None:
        if tuple(residual.shape) != (M, N) or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous [M, N] tensor")
    need = gemm_workspace_bytes(M, N, K)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=a.device)
        st = LIB.msr_gemm_ws(_ptr(a), _dt(a), _ptr(b_nk), _ptr(out), _dt(out), M, N, K, _ptr(residual),
                             _dt(out if residual is None else residual), 1 if gelu else 0,
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
        _check(st, "msr_gemm_ws")
        return out
    if residual is None and not gelu:
        st = LIB.msr_gemm(_ptr(a), _dt(a), _ptr(b_nk), _ptr(out), _dt(out), M, N, K, _stream(stream))
        _check(st, "msr_gemm")
        return out
    st = LIB.msr_gemm_ex(_ptr(a), _dt(a), _ptr(b_nk), _ptr(out), _dt(out), M, N, K, _ptr(residual),
                         _dt(out if residual is None else residual), 1 if gelu else 0, _stream(stream))
    _check(st, "msr_gemm_ex")
    return out


def layer_norm(x, eps, weight=None, bias=None, out=None, out_dtype=None, stream=None):
    """LayerNorm over the last axis (RetNet reading notes, §三.4): biased
    variance, eps under the square root, optional float32 affine."""
    if not x.is_contiguous():
        raise ValueError("layer_norm needs a contiguous input")
    d = x.shape[-1]
    rows = x.numel() // d
    if out is None:
        out = torch.empty(x.shape, dtype=x.dtype if out_dtype is None else out_dtype, device=x.device)
    if not out.is_contiguous() or out.numel() != x.numel():
        raise ValueError("out must be contiguous and of x's size")
    for t, name in ((weight, "weight"), (bias, "bias")):
        if t is not None and (t.dtype != torch.float32 or t.numel() != d or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float32 vector of {d}")
    st = LIB.ret_layer_norm(_ptr(x), _ptr(out), rows, d, _ptr(weight), _ptr(bias), float(eps), _dt(x), _dt(out),
                            _stream(stream))
    _check(st, "ret_layer_norm")
    return out


def msr_block_fwd(x, wq_t, wk_t, wv_t, wg_t, wo_t, gamma, theta, chunk, flags, eps, out_dtype=torch.bfloat16,
                  residual=None, pos0=0, n_prev=0, state=None, state_out=None, stream=None):
    """Gated multi-scale retention block forward (RetNet reading notes, §三.2):
    MSR(X) = (swish(X W_G) (.) GroupNorm_h(Retention heads)) W_O.

    x: [b, L, d_model] bf16 or fp16; w*_t: weights as [out_features,
    in_features] bf16;
    gamma: the h per-head decays (host float64).
    Every step runs in the library's kernels: four projections, the
    chunkwise retention over [b, h, L, d] views of the projections, the
    GroupNorm + swish gate, and the output projection, whose epilogue adds
    residual ([b*L, d_model]) when one is given.  Intermediates (the
    projections, the head outputs and the gated heads) are stored as fp16.
    state = (S, z) continues a sequence of n_prev tokens (phases from pos0);
    state_out = (S, z) receives the heads' final state (float32
    [b,h,d_k,d_v], [b,h,d_k]).
    """
    b, L, dm = x.shape
    h = len(gamma)
    x2 = x.reshape(b * L, dm)
    dk = wq_t.shape[0] // h
    dv = wv_t.shape[0] // h
    f16 = torch.float16
    Q = gemm(x2, wq_t, out_dtype=f16, stream=stream)
    K = gemm(x2, wk_t, out_dtype=f16, stream=stream)
    V = gemm(x2, wv_t, out_dtype=f16, stream=stream)
    G = gemm(x2, wg_t, out_dtype=f16, stream=stream)
    qv = Q.view(b, L, h, dk).transpose(1, 2)
    kv = K.view(b, L, h, dk).transpose(1, 2)
    vv = V.view(b, L, h, dv).transpose(1, 2)
    Y = torch.empty((b, L, h * dv), dtype=f16, device=x.device)
    yv = Y.view(b, L, h, dv).transpose(1, 2)
    S0, z0 = (None, None) if state is None else state
    S1, z1 = (None, None) if state_out is None else state_out
    chunkwise_fwd(qv, kv, vv, gamma, theta, chunk, flags, pos0=pos0, n_prev=n_prev, state_in=S0, z_in=z0,
                  state_out=S1, z_out=z1, out=yv, stream=stream)
    Z = gate_norm(yv, G.view(b, L, h * dv), eps, stream=stream)
    out = gemm(Z.view(b * L, h * dv), wo_t, out_dtype=out_dtype, residual=residual, stream=stream)
    return out.view(b, L, -1)


def retnet_layer_fwd(x, msr_w_t, w1_t, w2_t, gamma, theta, chunk, flags, gn_eps, ln_eps, ln1=(None, None),
                     ln2=(None, None), pos0=0, n_prev=0, state=None, state_out=None, out_dtype=None, stream=None):
    """One RetNet layer forward (reading notes §三.4):
        Y = MSR(LN(X)) + X,   X' = FFN(LN(Y)) + Y,   FFN(Y) = gelu(Y W_1) W_2.

    x: [b, L, d_model] float32 or bf16; the result has x's dtype (or out_dtype);
    msr_w_t: (W_Q, W_K, W_V, W_G, W_O) as [out_features, in_features] bf16;
    w1_t: [d_ff, d_model] and w2_t: [d_model, d_ff] bf16; ln1 / ln2: the two
    LayerNorms' float32 (weight, bias), None for 1 and 0.  Every step runs in
    the library: the LayerNorms (stored as fp16, the GEMMs' activation
    operand), the MSR block whose output projection adds X in its epilogue
    and keeps Y in float32, the first FFN projection with gelu in its
    epilogue (hidden stored as fp16) and the second with Y added.  state /
    state_out: the MSR heads' (S, z), as in msr_block_fwd.
    """
    if x.dtype not in (torch.float32, torch.bfloat16) or not x.is_contiguous():
        raise TypeError("x must be a contiguous float32 or bf16 tensor")
    b, L, dm = x.shape
    x2 = x.view(b * L, dm)
    xn = layer_norm(x2, ln_eps, *ln1, out_dtype=torch.float16, stream=stream)
    Y = msr_block_fwd(xn.view(b, L, dm), *msr_w_t, gamma, theta, chunk, flags, gn_eps, out_dtype=torch.float32,
                      residual=x2, pos0=pos0, n_prev=n_prev, state=state, state_out=state_out,
                      stream=stream).view(b * L, dm)
    yn = layer_norm(Y, ln_eps, *ln2, out_dtype=torch.float16, stream=stream)
    H = gemm(yn, w1_t, out_dtype=torch.float16, gelu=True, stream=stream)
    out = gemm(H, w2_t, out_dtype=x.dtype if out_dtype is None else out_dtype, residual=Y, stream=stream)
    return out.view(b, L, dm)


def new_states(n_layers, b, h, d_k, d_v, device="cuda"):
    """Zeroed per-layer retention states (S, z) for a fresh sequence."""
    return [(torch.zeros((b, h, d_k, d_v), dtype=torch.float32, device=device),
             torch.zeros((b, h, d_k), dtype=torch.float32, device=device)) for _ in range(n_layers)]


def retnet_stack_fwd(x, layers, gamma, theta, chunk, flags, gn_eps, ln_eps, pos0=0, n_prev=0, states=None,
                     states_out=None, stream=None):
    """A stack of RetNet layers (reading notes §三.4) over a sequence, the MSR
    heads in the chunkwise form.  layers: (msr_w_t, w1_t, w2_t, ln1, ln2) per
    layer as in retnet_layer_fwd; states: per-layer (S, z) to continue from;
    states_out: per-layer (S, z) buffers receiving the final states (a
    prefill for retnet_decode_step).  Between layers the activations stay
    float32; the result has x's dtype."""
    final_dtype = x.dtype
    for i, (msr_w_t, w1_t, w2_t, ln1, ln2) in enumerate(layers):
        last = i == len(layers) - 1
        x = retnet_layer_fwd(x, msr_w_t, w1_t, w2_t, gamma, theta, chunk, flags, gn_eps, ln_eps, ln1, ln2,
                             pos0=pos0, n_prev=n_prev, state=None if states is None else states[i],
                             state_out=None if states_out is None else states_out[i],
                             out_dtype=final_dtype if last else torch.float32, stream=stream)
    return x


def retnet_decode_step(x, layers, states, gamma, theta, pos, n_tokens, flags, gn_eps, ln_eps, stream=None):
    """One token per sequence through a stack of RetNet layers, each layer's
    MSR in the recurrent form (reading notes §2.2, §三.4).

    x: [b, d_model] float32 or bf16 (the result has its dtype); states: the
    layers' (S, z), updated in place; pos: the token's position (xPos phase);
    n_tokens: tokens seen including this one.  Per layer: LayerNorm (fp16),
    four projections, retention_recurrent_step on the [b, h, d] views,
    GroupNorm + gate on the one token, W_O with x added (Y in float32),
    LayerNorm, the gelu FFN with Y added -- all in the library's kernels.
    Between layers the activations stay float32."""
    if x.dtype not in (torch.float32, torch.bfloat16) or not x.is_contiguous() or x.dim() != 2:
        raise TypeError("x must be a contiguous [b, d_model] float32 or bf16 tensor")
    b, dm = x.shape
    h = len(gamma)
    f16 = torch.float16
    final_dtype = x.dtype
    for li, ((wq, wk, wv, wg, wo), w1, w2, ln1, ln2) in enumerate(layers):
        S, z = states[li]
        dk, dv = wq.shape[0] // h, wv.shape[0] // h
        xn = layer_norm(x, ln_eps, *ln1, out_dtype=f16, stream=stream)
        Q = gemm(xn, wq, out_dtype=f16, stream=stream)
        K = gemm(xn, wk, out_dtype=f16, stream=stream)
        V = gemm(xn, wv, out_dtype=f16, stream=stream)
        G = gemm(xn, wg, out_dtype=f16, stream=stream)
        o = recurrent_step(Q.view(b, h, dk), K.view(b, h, dk), V.view(b, h, dv), S, gamma, theta, pos, n_tokens,
                           flags, z=z, out_dtype=torch.float32, stream=stream)
        Z = gate_norm(o.view(b, h, 1, dv), G.view(b, 1, h * dv), gn_eps, stream=stream)
        Y = gemm(Z.view(b, h * dv), wo, out_dtype=torch.float32, residual=x, stream=stream)
        yn = layer_norm(Y, ln_eps, *ln2, out_dtype=f16, stream=stream)
        H = gemm(yn, w1, out_dtype=f16, gelu=True, stream=stream)
        x = gemm(H, w2, out_dtype=final_dtype if li == len(layers) - 1 else torch.float32, residual=Y,
                 stream=stream)
    return x


def _on_stream(fn):
    """Run fn with ``stream`` as torch's current stream.  Every tensor the
    wrapper allocates (outputs, workspaces, intermediates) then belongs to the
    stream its kernels run on, so torch's caching allocator cannot hand the
    memory to another stream while those kernels still use it."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None or stream == torch.cuda.current_stream(stream.device):
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=None, **kw)
    return run


for _name in ("chunkwise_fwd", "parallel_fwd", "chunkwise_bwd", "recurrent_step", "gate_norm", "gemm",
              "layer_norm", "msr_block_fwd", "retnet_layer_fwd", "retnet_stack_fwd", "retnet_decode_step"):
    globals()[_name] = _on_stream(globals()[_name])
del _name


def calib_copy(src, dst, stream=None):
    """dst <- src (equal-size contiguous device tensors, a multiple of 16 bytes):
    the measured HBM ceiling of the benchmark."""
    n = src.numel() * src.element_size()
    if n % 16 or dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst must have the same size, a multiple of 16 bytes")
    _check(LIB.ret_calib_copy(_ptr(src), _ptr(dst), n // 16, _stream(stream)), "ret_calib_copy")


def calib_mfma(out, blocks, iters, stream=None):
    """blocks x 4 waves x iters x 4 fp16 32x32x16 MFMAs (out: float32, blocks * 256):
    the measured matrix-core ceiling of the benchmark."""
    if out.dtype != torch.float32 or out.numel() < blocks * 256:
        raise ValueError("out must be float32 with blocks * 256 elements")
    _check(LIB.ret_calib_mfma(_ptr(out), blocks, iters, _stream(stream)), "ret_calib_mfma")
