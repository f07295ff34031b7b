"""ctypes binding of libsru (include/sru.h): argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
torch tensors as raw device pointers plus the caller's current HIP stream.
All arithmetic runs in the library's HIP kernels; there is no fallback: if
libsru.so is missing, importing the functions raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsru.so")

SRU_OK, SRU_ERR_INVALID_ARG, SRU_ERR_UNSUPPORTED = 0, 1, 2
SRU_ERR_NO_DEVICE, SRU_ERR_LAUNCH, SRU_ERR_WORKSPACE = 3, 4, 5
SRU_F32, SRU_BF16 = 0, 1
SRU_FWD, SRU_BWD = 0, 1
SRU_PROJ_FWD, SRU_PROJ_BWD_DATA, SRU_PROJ_BWD_DATA_WT = 0, 1, 2
SRU_WS_BACKWARD, SRU_WS_LINEAR_FWD, SRU_WS_LINEAR_BWD, SRU_WS_BWD_WEIGHT = 1, 2, 3, 4
SRU_WS_FACTORED_WEIGHT = 5
SRU_FACT_Q, SRU_FACT_U, SRU_FACT_BWD_Q, SRU_FACT_BWD_X = 0, 1, 2, 3
SRU_FACT_WGRAD_Q, SRU_FACT_WGRAD_O = 0, 1

# Every symbol include/sru.h declares.
EXPORTED = ("sru_project", "sru_project_bwd_weight", "sru_project_factored",
            "sru_project_factored_bwd_weight", "sru_attention_forward",
            "sru_attention_workspace_size", "sru_attention_backward",
            "sru_attention_backward_workspace_size", "sru_step", "sru_forward", "sru_backward",
            "sru_backward_static", "sru_linear_scan",
            "sru_transpose_weight", "sru_round_bf16", "sru_workspace_size", "sru_status_string",
            "sru_last_error")


class SruShape(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("B", ctypes.c_int64), ("d", ctypes.c_int64),
                ("bidirectional", ctypes.c_int32), ("alpha", ctypes.c_float)]

    def __init__(self, L, B, d, bidirectional=False, alpha=1.0):
        super().__init__(int(L), int(B), int(d), int(bool(bidirectional)), float(alpha))

    @property
    def ndir(self) -> int:
        return 2 if self.bidirectional else 1

    def __repr__(self):
        return (f"SruShape(L={self.L}, B={self.B}, d={self.d}, "
                f"bidirectional={bool(self.bidirectional)}, alpha={self.alpha})")


class SruAttnCfg(ctypes.Structure):
    _fields_ = [("d_inner", ctypes.c_int64), ("mem_len", ctypes.c_int64),
                ("causal", ctypes.c_int32), ("layernorm", ctypes.c_int32),
                ("attn_alpha", ctypes.c_float), ("ln_eps", ctypes.c_float)]

    def __init__(self, d_inner, mem_len=0, causal=True, layernorm=False, attn_alpha=0.0,
                 ln_eps=1e-5):
        super().__init__(int(d_inner), int(mem_len), int(bool(causal)), int(bool(layernorm)),
                         float(attn_alpha), float(ln_eps))


class SruError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


_lib = None
_vp = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libsru.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m parallelizable_recurrent_units_amd.build`")
    lib = ctypes.CDLL(path)
    sp = ctypes.POINTER(SruShape)
    i32, sz = ctypes.c_int32, ctypes.c_size_t
    lib.sru_project.restype = ctypes.c_int
    lib.sru_project.argtypes = [sp, ctypes.c_int, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp,
                                ctypes.c_int, i32, _vp]
    lib.sru_project_bwd_weight.restype = ctypes.c_int
    lib.sru_project_bwd_weight.argtypes = [sp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp,
                                           ctypes.c_int, i32, _vp, sz, _vp]
    lib.sru_project_factored.restype = ctypes.c_int
    lib.sru_project_factored.argtypes = [sp, ctypes.c_int64, ctypes.c_int, _vp, ctypes.c_int, _vp,
                                         ctypes.c_int, _vp, i32, _vp]
    lib.sru_project_factored_bwd_weight.restype = ctypes.c_int
    lib.sru_project_factored_bwd_weight.argtypes = [sp, ctypes.c_int64, ctypes.c_int, _vp,
                                                    ctypes.c_int, _vp, ctypes.c_int, _vp,
                                                    ctypes.c_int, i32, _vp, sz, _vp]
    cp = ctypes.POINTER(SruAttnCfg)
    lib.sru_attention_forward.restype = ctypes.c_int
    lib.sru_attention_forward.argtypes = [sp, cp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, ctypes.c_int, _vp, sz, _vp]
    lib.sru_attention_workspace_size.restype = sz
    lib.sru_attention_workspace_size.argtypes = [sp, cp]
    lib.sru_attention_backward.restype = ctypes.c_int
    lib.sru_attention_backward.argtypes = [sp, cp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, ctypes.c_int, _vp, i32, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, sz, _vp]
    lib.sru_attention_backward_workspace_size.restype = sz
    lib.sru_attention_backward_workspace_size.argtypes = [sp, cp]
    lib.sru_step.restype = ctypes.c_int
    lib.sru_step.argtypes = [sp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                             _vp]
    lib.sru_round_bf16.restype = ctypes.c_int
    lib.sru_round_bf16.argtypes = [ctypes.c_int64, _vp, _vp, _vp]
    lib.sru_forward.restype = ctypes.c_int
    lib.sru_forward.argtypes = [sp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                ctypes.c_int, _vp, _vp, _vp]
    lib.sru_backward.restype = ctypes.c_int
    lib.sru_backward.argtypes = [sp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, sz, _vp]
    lib.sru_backward_static.restype = ctypes.c_int
    lib.sru_backward_static.argtypes = [sp, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.sru_linear_scan.restype = ctypes.c_int
    lib.sru_linear_scan.argtypes = [sp, ctypes.c_int, i32, _vp, ctypes.c_int, _vp, ctypes.c_int,
                                    _vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _vp, sz, _vp]
    lib.sru_transpose_weight.restype = ctypes.c_int
    lib.sru_transpose_weight.argtypes = [sp, _vp, ctypes.c_int, _vp, _vp]
    lib.sru_workspace_size.restype = sz
    lib.sru_workspace_size.argtypes = [sp, ctypes.c_int, i32]
    lib.sru_status_string.restype = ctypes.c_char_p
    lib.sru_status_string.argtypes = [ctypes.c_int]
    lib.sru_last_error.restype = ctypes.c_char_p
    lib.sru_last_error.argtypes = []
    _lib = lib
    return lib


def _check(status: int):
    if status != SRU_OK:
        lib = load_library()
        raise SruError(status, lib.sru_status_string(status).decode(),
                       lib.sru_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SRU_F32
    if t.dtype == torch.bfloat16:
        return SRU_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libsru must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsru must be contiguous")
    return t.data_ptr()


def _need_f32(**tensors):
    """The arguments libsru reads or writes only as fp32 (None is skipped)."""
    import torch
    for name, t in tensors.items():
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32 (got {t.dtype})")


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _shape(shape) -> SruShape:
    return shape if isinstance(shape, SruShape) else SruShape(*shape)


def sru_workspace_size(shape, op: int, chunk: int = 0) -> int:
    s = _shape(shape)
    n = load_library().sru_workspace_size(ctypes.byref(s), int(op), int(chunk))
    if n == 0 and load_library().sru_last_error():
        raise SruError(SRU_ERR_INVALID_ARG, "SRU_ERR_INVALID_ARG",
                       load_library().sru_last_error().decode())
    return int(n)


def sru_project(shape, op: int, A, W, C, accumulate: bool = False, stream=None):
    s = _shape(shape)
    _check(load_library().sru_project(ctypes.byref(s), int(op), _ptr(A), _dtype_code(A),
                                      _ptr(W), _dtype_code(W), _ptr(C), _dtype_code(C),
                                      int(bool(accumulate)), _stream(stream)))


def sru_project_bwd_weight(shape, dU, X, dW, math_dtype: int = SRU_BF16, accumulate: bool = False,
                           workspace=None, stream=None):
    s = _shape(shape)
    _need_f32(dW=dW)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().sru_project_bwd_weight(
        ctypes.byref(s), _ptr(dU), _dtype_code(dU), _ptr(X), _dtype_code(X), _ptr(dW),
        int(math_dtype), int(bool(accumulate)), _ptr(workspace), ws_bytes, _stream(stream)))


def sru_project_factored(shape, d_inner: int, op: int, A, W, C, accumulate: bool = False,
                         stream=None):
    s = _shape(shape)
    if _dtype_code(C) != SRU_F32:
        raise TypeError("C must be float32")
    _check(load_library().sru_project_factored(
        ctypes.byref(s), int(d_inner), int(op), _ptr(A), _dtype_code(A), _ptr(W), _dtype_code(W),
        _ptr(C), int(bool(accumulate)), _stream(stream)))


def sru_project_factored_bwd_weight(shape, d_inner: int, which: int, G, Y, dW,
                                    math_dtype: int = SRU_BF16, accumulate: bool = False,
                                    workspace=None, stream=None):
    s = _shape(shape)
    if _dtype_code(dW) != SRU_F32:
        raise TypeError("dW must be float32")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().sru_project_factored_bwd_weight(
        ctypes.byref(s), int(d_inner), int(which), _ptr(G), _dtype_code(G), _ptr(Y),
        _dtype_code(Y), _ptr(dW), int(math_dtype), int(bool(accumulate)), _ptr(workspace),
        ws_bytes, _stream(stream)))


def sru_attention_workspace_size(shape, cfg) -> int:
    s = _shape(shape)
    n = load_library().sru_attention_workspace_size(ctypes.byref(s), ctypes.byref(cfg))
    if n == 0:
        raise SruError(SRU_ERR_INVALID_ARG, "SRU_ERR_INVALID_ARG",
                       load_library().sru_last_error().decode())
    return int(n)


def sru_attention_forward(shape, cfg, X, Wq, Wkv, Wo, gamma, beta, Q, KV, R, U, workspace,
                          stream=None):
    s = _shape(shape)
    for name, t in (("Wq", Wq), ("Wkv", Wkv), ("Wo", Wo), ("KV", KV)):
        if _dtype_code(t) != SRU_BF16:
            raise TypeError(f"{name} must be bfloat16")
    _need_f32(Q=Q, R=R, gamma=gamma, beta=beta)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().sru_attention_forward(
        ctypes.byref(s), ctypes.byref(cfg), _ptr(X), _dtype_code(X), _ptr(Wq), _ptr(Wkv),
        _ptr(Wo), _ptr(gamma), _ptr(beta), _ptr(Q), _ptr(KV), _ptr(R), _ptr(U), _dtype_code(U),
        _ptr(workspace), ws_bytes, _stream(stream)))


def sru_attention_backward_workspace_size(shape, cfg) -> int:
    s = _shape(shape)
    n = load_library().sru_attention_backward_workspace_size(ctypes.byref(s), ctypes.byref(cfg))
    if n == 0:
        raise SruError(SRU_ERR_INVALID_ARG, "SRU_ERR_INVALID_ARG",
                       load_library().sru_last_error().decode())
    return int(n)


def sru_attention_backward(shape, cfg, X, Wq, Wkv, Wo, gamma, Q, KV, R, dU, dX, dWq, dWkv, dWo,
                           dalpha, dgamma, dbeta, workspace, accumulate_dx: bool = False,
                           stream=None):
    s = _shape(shape)
    for name, t in (("Wq", Wq), ("Wkv", Wkv), ("Wo", Wo), ("KV", KV)):
        if _dtype_code(t) != SRU_BF16:
            raise TypeError(f"{name} must be bfloat16")
    _need_f32(gamma=gamma, Q=Q, R=R, dX=dX, dWq=dWq, dWkv=dWkv, dWo=dWo, dalpha=dalpha,
              dgamma=dgamma, dbeta=dbeta)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().sru_attention_backward(
        ctypes.byref(s), ctypes.byref(cfg), _ptr(X), _dtype_code(X), _ptr(Wq), _ptr(Wkv),
        _ptr(Wo), _ptr(gamma), _ptr(Q), _ptr(KV), _ptr(R), _ptr(dU), _dtype_code(dU), _ptr(dX),
        int(bool(accumulate_dx)), _ptr(dWq), _ptr(dWkv), _ptr(dWo), _ptr(dalpha), _ptr(dgamma),
        _ptr(dbeta), _ptr(workspace), ws_bytes, _stream(stream)))


def sru_step(shape, x, W, v, b, c_prev, h, c_next, stream=None):
    s = _shape(shape)
    _need_f32(v=v, b=b, c_prev=c_prev, h=h, c_next=c_next)
    _check(load_library().sru_step(ctypes.byref(s), _ptr(x), _dtype_code(x), _ptr(W),
                                   _dtype_code(W), _ptr(v), _ptr(b), _ptr(c_prev), _ptr(h),
                                   _ptr(c_next), _stream(stream)))


def sru_round_bf16(src, dst, stream=None):
    if _dtype_code(src) != SRU_F32 or _dtype_code(dst) != SRU_BF16:
        raise TypeError("src must be float32 and dst bfloat16")
    if src.numel() != dst.numel():
        raise ValueError("src and dst differ in size")
    _check(load_library().sru_round_bf16(int(src.numel()), _ptr(src), _ptr(dst), _stream(stream)))


def sru_transpose_weight(shape, W, Wt, stream=None):
    s = _shape(shape)
    _check(load_library().sru_transpose_weight(ctypes.byref(s), _ptr(W), _dtype_code(W), _ptr(Wt),
                                               _stream(stream)))


def sru_forward(shape, U, x, v, b, c0, h, c_seq=None, c_last=None, stream=None):
    s = _shape(shape)
    _need_f32(v=v, b=b, c0=c0, c_seq=c_seq, c_last=c_last)
    _check(load_library().sru_forward(ctypes.byref(s), _ptr(U), _dtype_code(U), _ptr(x),
                                      _dtype_code(x), _ptr(v), _ptr(b), _ptr(c0), _ptr(h),
                                      _dtype_code(h), _ptr(c_seq), _ptr(c_last),
                                      _stream(stream)))


def sru_backward(shape, U, x, v, b, c0, c_seq, dh, dc_last, dU, dx, dv, db, dc0,
                 workspace, dU_lp=None, stream=None):
    s = _shape(shape)
    _need_f32(v=v, b=b, c0=c0, c_seq=c_seq, dh=dh, dc_last=dc_last, dU=dU, dx=dx, dv=dv, db=db,
              dc0=dc0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if dU_lp is not None and _dtype_code(dU_lp) != SRU_BF16:
        raise TypeError("dU_lp must be bfloat16")
    _check(load_library().sru_backward(ctypes.byref(s), _ptr(U), _dtype_code(U), _ptr(x),
                                       _dtype_code(x), _ptr(v), _ptr(b), _ptr(c0), _ptr(c_seq),
                                       _ptr(dh), _ptr(dc_last), _ptr(dU), _ptr(dU_lp), _ptr(dx),
                                       _ptr(dv), _ptr(db), _ptr(dc0), _ptr(workspace), ws_bytes,
                                       _stream(stream)))


# Bytes of the static scratch sru_backward_static uses on each GPU
# (SRU_BACKWARD_STATIC_SCRATCH_BYTES in include/sru.h).
SRU_BACKWARD_STATIC_SCRATCH_BYTES = 16 << 20


def sru_backward_static(shape, U, x, v, b, c0, c_seq, dh, dc_last, dU, dx, dv, db, dc0,
                        dU_lp=None, error_word=None, stream=None):
    """sru_backward with the library's static scratch (no workspace argument);
    ``error_word``: an optional int32 device tensor of one element."""
    s = _shape(shape)
    _need_f32(v=v, b=b, c0=c0, c_seq=c_seq, dh=dh, dc_last=dc_last, dU=dU, dx=dx, dv=dv, db=db,
              dc0=dc0)
    if dU_lp is not None and _dtype_code(dU_lp) != SRU_BF16:
        raise TypeError("dU_lp must be bfloat16")
    _check(load_library().sru_backward_static(
        ctypes.byref(s), _ptr(U), _dtype_code(U), _ptr(x), _dtype_code(x), _ptr(v), _ptr(b),
        _ptr(c0), _ptr(c_seq), _ptr(dh), _ptr(dc_last), _ptr(dU), _ptr(dU_lp), _ptr(dx), _ptr(dv),
        _ptr(db), _ptr(dc0), _ptr(error_word), _stream(stream)))


def sru_linear_scan(shape, pass_: int, chunk: int, U, x, b, c0, h=None, c_seq=None,
                    c_last=None, dh=None, dc_last=None, dU=None, dx=None, db=None, dc0=None,
                    workspace=None, stream=None):
    s = _shape(shape)
    _need_f32(b=b, c0=c0, c_seq=c_seq, c_last=c_last, dh=dh, dc_last=dc_last, dU=dU, dx=dx,
              db=db, dc0=dc0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    h_dt = _dtype_code(h) if h is not None else SRU_F32
    _check(load_library().sru_linear_scan(
        ctypes.byref(s), int(pass_), int(chunk), _ptr(U), _dtype_code(U), _ptr(x),
        _dtype_code(x), _ptr(b), _ptr(c0), _ptr(h), h_dt, _ptr(c_seq), _ptr(c_last),
        _ptr(dh), _ptr(dc_last), _ptr(dU), _ptr(dx), _ptr(db), _ptr(dc0), _ptr(workspace),
        ws_bytes, _stream(stream)))


# Byte offset of the error word in the workspaces of sru_backward and
# sru_linear_scan (SRU_WS_ERROR_OFFSET in include/sru.h).
SRU_WS_ERROR_OFFSET = 0


def workspace_error_word(workspace) -> int:
    """The 32-bit error word of a workspace last passed to sru_backward or
    sru_linear_scan: 0, or nonzero when a bounded wait between chunks ran out
    (that call's outputs are then invalid).  Reads 4 bytes from the device,
    which waits for the work queued before it on the current stream."""
    import torch
    raw = workspace.view(torch.uint8)[SRU_WS_ERROR_OFFSET:SRU_WS_ERROR_OFFSET + 4]
    return int(raw.cpu().view(torch.int32)[0])


def check_workspace(workspace, what: str = "scan"):
    """Raise if the workspace's error word is set (see workspace_error_word)."""
    w = workspace_error_word(workspace)
    if w != 0:
        raise SruError(SRU_ERR_LAUNCH, "SRU_ERR_LAUNCH",
                       f"{what}: a wait between chunks ran out (error word {w:#x}); "
                       "the outputs of that call are invalid")
