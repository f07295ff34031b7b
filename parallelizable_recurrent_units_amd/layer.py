"""Convenience wrappers: allocate outputs with torch, then call the C ABI.

Each function is a single entry point (or a fixed sequence of them) of
libsru; no arithmetic happens here.  Layouts are those of include/sru.h.
"""
from __future__ import annotations

import torch

from . import _binding as B


def round_bf16(x, out=None, stream=None):
    """bf16(x), nearest even (the operand X~ of the bf16 projection)."""
    if out is None:
        out = torch.empty(x.shape, device=x.device, dtype=torch.bfloat16)
    B.sru_round_bf16(x, out, stream)
    return out


def project(shape, X, W, U=None, accumulate=False, stream=None):
    """Eq. 1: U[L*B, ndir*3d] (+)= X W^T (X rounded to bf16 when W is bf16)."""
    s = B._shape(shape)
    if U is None:
        U = torch.empty((s.L, s.B, s.ndir, 3, s.d), device=X.device, dtype=torch.float32)
    B.sru_project(s, B.SRU_PROJ_FWD, X, W, U, accumulate, stream)
    return U


def transpose_weight(shape, W, Wt=None, stream=None):
    """Wt = W^T ([d, ndir*3d]) for the transposed backward-data product."""
    s = B._shape(shape)
    if Wt is None:
        Wt = torch.empty((s.d, s.ndir * 3 * s.d), device=W.device, dtype=W.dtype)
    B.sru_transpose_weight(s, W, Wt, stream)
    return Wt


def project_bwd_data(shape, dU, W, dX=None, accumulate=False, Wt=None, stream=None):
    """dX[L*B, d] (+)= dU W (gradient through Eq. 1).

    With ``Wt`` (= W^T from transpose_weight) the K-contiguous kernel path is
    used; otherwise W is transposed while it is staged into LDS."""
    s = B._shape(shape)
    if dX is None:
        dX = torch.empty((s.L, s.B, s.d), device=dU.device, dtype=torch.float32)
    if Wt is not None:
        B.sru_project(s, B.SRU_PROJ_BWD_DATA_WT, dU, Wt, dX, accumulate, stream)
    else:
        B.sru_project(s, B.SRU_PROJ_BWD_DATA, dU, W, dX, accumulate, stream)
    return dX


def project_bwd_weight(shape, dU, X, dW=None, accumulate=False, f32_math=False, ws=None,
                       stream=None):
    """dW[ndir*3d, d] (+)= dU^T X (weight gradient through Eq. 1).

    bf16 MFMA on operands rounded to bf16 unless ``f32_math``."""
    s = B._shape(shape)
    if dW is None:
        dW = torch.empty((s.ndir * 3 * s.d, s.d), device=dU.device, dtype=torch.float32)
    if ws is None and not f32_math:
        n = B.sru_workspace_size(s, B.SRU_WS_BWD_WEIGHT, 0)
        ws = torch.empty(n, device=dU.device, dtype=torch.uint8) if n else None
    B.sru_project_bwd_weight(s, dU, X, dW, B.SRU_F32 if f32_math else B.SRU_BF16, accumulate,
                             ws, stream)
    return dW


def project_factored(shape, d_inner, X, Wq, Wo, stream=None):
    """Fig. 2(b) of the SRU++ paper: Q = X Wq^T, U = Q Wo^T (two calls).
    Returns (Q [L*B, d'], U [L, B, ndir, 3, d])."""
    s = B._shape(shape)
    Q = torch.empty((s.L * s.B, d_inner), device=X.device, dtype=torch.float32)
    U = torch.empty((s.L, s.B, s.ndir, 3, s.d), device=X.device, dtype=torch.float32)
    B.sru_project_factored(s, d_inner, B.SRU_FACT_Q, X, Wq, Q, False, stream)
    B.sru_project_factored(s, d_inner, B.SRU_FACT_U, Q, Wo, U, False, stream)
    return Q, U


def project_factored_backward(shape, d_inner, X, Q, Wq, Wo, dU, dX=None, accumulate=False,
                              f32_math=None, ws=None, stream=None):
    """Gradients of project_factored given dU: (dQ, dX, dWq, dWo).  dX is
    added to when ``accumulate`` (e.g. onto sru_backward's highway dx)."""
    s = B._shape(shape)
    dev = dU.device
    f32 = dict(device=dev, dtype=torch.float32)
    if f32_math is None:
        f32_math = Wq.dtype == torch.float32
    dQ = torch.empty((s.L * s.B, d_inner), **f32)
    if dX is None:
        dX = torch.empty((s.L, s.B, s.d), **f32)
    dWq = torch.empty((d_inner, s.d), **f32)
    dWo = torch.empty((s.ndir * 3 * s.d, d_inner), **f32)
    if ws is None and not f32_math:
        n = B.sru_workspace_size(s, B.SRU_WS_FACTORED_WEIGHT, d_inner)
        ws = torch.empty(n, device=dev, dtype=torch.uint8) if n else None
    math = B.SRU_F32 if f32_math else B.SRU_BF16
    B.sru_project_factored(s, d_inner, B.SRU_FACT_BWD_Q, dU, Wo, dQ, False, stream)
    B.sru_project_factored(s, d_inner, B.SRU_FACT_BWD_X, dQ, Wq, dX, accumulate, stream)
    B.sru_project_factored_bwd_weight(s, d_inner, B.SRU_FACT_WGRAD_Q, dQ, X, dWq, math, False,
                                      ws, stream)
    B.sru_project_factored_bwd_weight(s, d_inner, B.SRU_FACT_WGRAD_O, dU, Q, dWo, math, False,
                                      ws, stream)
    return dQ, dX, dWq, dWo


def attention_forward(shape, cfg, X, Wq, Wkv, Wo, gamma=None, beta=None, KV=None, ws=None,
                      u_dtype=torch.float32, stream=None):
    """SRU++ attention U-producer.  ``KV`` (bf16 [mem_len + L, B, 2 d']) may
    carry the previous segment's keys and values in its first mem_len rows;
    its remaining rows are written.  U is float32 or bfloat16 (``u_dtype``).
    Returns (Q, KV, R, U)."""
    s = B._shape(shape)
    dev = X.device
    dp, Lm = cfg.d_inner, cfg.mem_len
    f32 = dict(device=dev, dtype=torch.float32)
    Q = torch.empty((s.L * s.B, dp), **f32)
    R = torch.empty((s.L * s.B, dp), **f32)
    U = torch.empty((s.L, s.B, s.ndir, 3, s.d), device=dev, dtype=u_dtype)
    if KV is None:
        KV = torch.empty((Lm + s.L, s.B, 2 * dp), device=dev, dtype=torch.bfloat16)
    if ws is None:
        ws = torch.empty(B.sru_attention_workspace_size(s, cfg), device=dev, dtype=torch.uint8)
    B.sru_attention_forward(s, cfg, X, Wq, Wkv, Wo, gamma, beta, Q, KV, R, U, ws, stream)
    return Q, KV, R, U


def attention_backward(shape, cfg, X, Wq, Wkv, Wo, Q, KV, R, dU, gamma=None, dX=None,
                       accumulate_dx=False, ws=None, stream=None):
    """Gradients of attention_forward for dU: returns a dict with dX (added
    to the given dX when accumulate_dx), dWq, dWkv, dWo, dalpha [1] and, with
    layer norm, dgamma and dbeta."""
    s = B._shape(shape)
    dev = X.device
    dp = cfg.d_inner
    f32 = dict(device=dev, dtype=torch.float32)
    if dX is None:
        dX = torch.empty((s.L * s.B, s.d), **f32)
    out = dict(dX=dX, dWq=torch.empty((dp, s.d), **f32), dWkv=torch.empty((2 * dp, dp), **f32),
               dWo=torch.empty((s.ndir * 3 * s.d, dp), **f32), dalpha=torch.empty(1, **f32),
               dgamma=torch.empty(dp, **f32) if cfg.layernorm else None,
               dbeta=torch.empty(dp, **f32) if cfg.layernorm else None)
    if ws is None:
        ws = torch.empty(B.sru_attention_backward_workspace_size(s, cfg), device=dev,
                         dtype=torch.uint8)
    B.sru_attention_backward(s, cfg, X, Wq, Wkv, Wo, gamma, Q, KV, R, dU, out["dX"], out["dWq"],
                             out["dWkv"], out["dWo"], out["dalpha"], out["dgamma"],
                             out["dbeta"], ws, accumulate_dx, stream)
    return out


def step(shape, x, W, v, b, c=None, h=None, stream=None):
    """One decoding step: (h, c_next) for input rows x [B, d] from state c
    [B, d] (zero when None).  Pass the same tensor as ``c`` each call to carry
    the state in place; h is allocated unless given."""
    s = B._shape(shape)
    f32 = dict(device=x.device, dtype=torch.float32)
    if h is None:
        h = torch.empty((s.B, s.d), **f32)
    c_next = c if c is not None else torch.empty((s.B, s.d), **f32)
    B.sru_step(s, x, W, v, b, c, h, c_next, stream)
    return h, c_next


def forward(shape, U, x, v, b, c0=None, keep_c_seq=False, stream=None):
    s = B._shape(shape)
    dev = U.device
    h = torch.empty((s.L, s.B, s.ndir, s.d), device=dev, dtype=torch.float32)
    c_seq = (torch.empty((s.L, s.B, s.ndir, s.d), device=dev, dtype=torch.float32)
             if keep_c_seq else None)
    c_last = torch.empty((s.ndir, s.B, s.d), device=dev, dtype=torch.float32)
    B.sru_forward(s, U, x, v, b, c0, h, c_seq, c_last, stream)
    return h, c_seq, c_last


def workspace(shape, op, chunk=0, device="cuda"):
    n = B.sru_workspace_size(shape, op, chunk)
    return torch.empty(n, device=device, dtype=torch.uint8)


# When True, backward() and the linear scans read their workspace's error
# word after the call (a synchronising 4-byte read, skipped while a graph is
# being captured) and raise if a wait between chunks ran out.
CHECK_SCAN_ERRORS = False


def _checked(ws, what):
    if CHECK_SCAN_ERRORS and not torch.cuda.is_current_stream_capturing():
        B.check_workspace(ws, what)


def backward(shape, U, x, v, b, c0, c_seq, dh, dc_last=None, ws=None, bf16_copy=False,
             stream=None):
    """Returns (dU, dx, dv, db, dc0), plus dU rounded to bf16 when bf16_copy."""
    s = B._shape(shape)
    dev = U.device
    dU = torch.empty((s.L, s.B, s.ndir, 3, s.d), device=dev, dtype=torch.float32)
    dU_lp = torch.empty_like(dU, dtype=torch.bfloat16) if bf16_copy else None
    dx = torch.empty((s.L, s.B, s.d), device=dev, dtype=torch.float32)
    dv = torch.empty((s.ndir, 2, s.d), device=dev, dtype=torch.float32)
    db = torch.empty((s.ndir, 2, s.d), device=dev, dtype=torch.float32)
    dc0 = torch.empty((s.ndir, s.B, s.d), device=dev, dtype=torch.float32)
    if ws is None:
        ws = workspace(s, B.SRU_WS_BACKWARD, 0, dev)
    B.sru_backward(s, U, x, v, b, c0, c_seq, dh, dc_last, dU, dx, dv, db, dc0, ws, dU_lp, stream)
    _checked(ws, "sru_backward")
    if bf16_copy:
        return dU, dx, dv, db, dc0, dU_lp
    return dU, dx, dv, db, dc0


def linear_forward(shape, chunk, U, x, b, c0=None, keep_c_seq=True, ws=None, stream=None):
    s = B._shape(shape)
    dev = U.device
    h = torch.empty((s.L, s.B, s.ndir, s.d), device=dev, dtype=torch.float32)
    c_seq = (torch.empty((s.L, s.B, s.ndir, s.d), device=dev, dtype=torch.float32)
             if keep_c_seq else None)
    c_last = torch.empty((s.ndir, s.B, s.d), device=dev, dtype=torch.float32)
    if ws is None:
        ws = workspace(s, B.SRU_WS_LINEAR_FWD, chunk, dev)
    B.sru_linear_scan(s, B.SRU_FWD, chunk, U, x, b, c0, h=h, c_seq=c_seq, c_last=c_last,
                      workspace=ws, stream=stream)
    _checked(ws, "sru_linear_scan forward")
    return h, c_seq, c_last


def linear_backward(shape, chunk, U, x, b, c0, c_seq, dh, dc_last=None, ws=None, stream=None):
    s = B._shape(shape)
    dev = U.device
    dU = torch.empty((s.L, s.B, s.ndir, 3, s.d), device=dev, dtype=torch.float32)
    dx = torch.empty((s.L, s.B, s.d), device=dev, dtype=torch.float32)
    db = torch.empty((s.ndir, 2, s.d), device=dev, dtype=torch.float32)
    dc0 = torch.empty((s.ndir, s.B, s.d), device=dev, dtype=torch.float32)
    if ws is None:
        ws = workspace(s, B.SRU_WS_LINEAR_BWD, chunk, dev)
    B.sru_linear_scan(s, B.SRU_BWD, chunk, U, x, b, c0, c_seq=c_seq, dh=dh, dc_last=dc_last,
                      dU=dU, dx=dx, db=db, dc0=dc0, workspace=ws, stream=stream)
    _checked(ws, "sru_linear_scan backward")
    return dU, dx, db, dc0
