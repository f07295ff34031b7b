"""Host-side checks of the C ABI (CPU only; no kernel is ever launched here).

* libsru.so loads and exports every function include/sru.h declares;
* workspace sizes follow their stated formulas;
* every validation path returns its status before touching a device;
* a valid call on a machine without a GPU returns SRU_ERR_NO_DEVICE.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import parallelizable_recurrent_units_amd as sru
from parallelizable_recurrent_units_amd import _binding as Bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    # The checks below hand fake device addresses to the library and expect
    # SRU_ERR_NO_DEVICE from calls that are otherwise valid; where a GPU is
    # visible those calls would launch kernels on the fake addresses, so the
    # module runs only where none is.
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only checks (fake device addresses): a GPU is visible")
    if not os.path.exists(Bd.LIB_PATH):
        from parallelizable_recurrent_units_amd import build
        build.build()
    return sru.load_library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "sru.h")).read()
    return sorted(set(re.findall(r"\b(sru_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    declared = header_functions()
    assert declared == sorted(Bd.EXPORTED)
    for name in declared:
        assert getattr(lib, name) is not None


def test_status_strings(lib):
    for code, name in [(0, "SRU_OK"), (1, "SRU_ERR_INVALID_ARG"), (2, "SRU_ERR_UNSUPPORTED"),
                       (3, "SRU_ERR_NO_DEVICE"), (4, "SRU_ERR_LAUNCH"), (5, "SRU_ERR_WORKSPACE")]:
        assert lib.sru_status_string(code).decode() == name


def round256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("L,B,d,bi", [(4, 2, 64, 0), (7, 3, 5, 1), (16384, 4, 4096, 0),
                                      (64, 128, 512, 1), (128, 16, 128, 0)])
def test_workspace_sizes(lib, L, B, d, bi):
    s = sru.SruShape(L, B, d, bi, 1.0)
    nd = 2 if bi else 1
    nC64 = -(-L // 64)    # chunk count of the shortest backward chunk
    assert sru.sru_workspace_size(s, sru.SRU_WS_BACKWARD) == round256(
        (2 * nC64 * B * d + 64 + nd * nC64 * B * 4 * d) * 4)
    for chunk in (1, 7, 256):
        nC = -(-L // chunk)
        assert sru.sru_workspace_size(s, sru.SRU_WS_LINEAR_FWD, chunk) == round256((3 * nC * B * d + 64) * 4)
        assert sru.sru_workspace_size(s, sru.SRU_WS_LINEAR_BWD, chunk) == round256((5 * nC * B * d + 64) * 4)
    # weight gradient: the split-reduction workspace of [ndir*3d, d] = dU^T X
    # and room for a bf16 copy of an fp32 X
    assert sru.sru_workspace_size(s, sru.SRU_WS_BWD_WEIGHT) == wgrad_query(3 * nd * d, d, L * B)
    assert lib.sru_workspace_size(ctypes.byref(s), sru.SRU_WS_LINEAR_FWD, 0) == 0
    assert b"chunk" in lib.sru_last_error()
    assert lib.sru_workspace_size(ctypes.byref(s), 9, 1) == 0


# Fake, 16-byte aligned "device" addresses: validation fails before any use.
P = [0x10000 * (i + 1) for i in range(24)]


def fwd(lib, s, **kw):
    a = dict(U=P[0], u_dt=0, x=P[1], x_dt=0, v=P[2], b=P[3], c0=None, h=P[4], h_dt=0,
             c_seq=None, c_last=None)
    a.update(kw)
    return lib.sru_forward(ctypes.byref(s) if s is not None else None, a["U"], a["u_dt"],
                           a["x"], a["x_dt"], a["v"], a["b"], a["c0"], a["h"], a["h_dt"],
                           a["c_seq"], a["c_last"], None)


def bwd(lib, s, ws_bytes, **kw):
    a = dict(U=P[0], x=P[1], v=P[2], b=P[3], c0=None, c_seq=P[5], dh=P[6], dc_last=None,
             dU=P[7], dU_lp=None, dx=P[8], dv=None, db=None, dc0=None, ws=P[9])
    a.update(kw)
    return lib.sru_backward(ctypes.byref(s), a["U"], 0, a["x"], 0, a["v"], a["b"], a["c0"],
                            a["c_seq"], a["dh"], a["dc_last"], a["dU"], a["dU_lp"], a["dx"],
                            a["dv"], a["db"], a["dc0"], a["ws"], ws_bytes, None)


def lin(lib, s, pass_, chunk, ws_bytes, **kw):
    a = dict(U=P[0], x=P[1], b=P[3], c0=None, h=P[4], h_dt=0, c_seq=P[5], c_last=None,
             dh=P[6], dc_last=None, dU=P[7], dx=P[8], db=None, dc0=None, ws=P[9])
    a.update(kw)
    return lib.sru_linear_scan(ctypes.byref(s), pass_, chunk, a["U"], 0, a["x"], 0, a["b"],
                               a["c0"], a["h"], a["h_dt"], a["c_seq"], a["c_last"], a["dh"],
                               a["dc_last"], a["dU"], a["dx"], a["db"], a["dc0"], a["ws"],
                               ws_bytes, None)


def test_invalid_shapes(lib):
    assert fwd(lib, None) == sru.SRU_ERR_INVALID_ARG
    for L, B, d, bi, al in [(0, 1, 1, 0, 1.0), (1, 0, 1, 0, 1.0), (1, 1, 0, 0, 1.0),
                            (1, 1, 1, 2, 1.0), (1, 1, 1, 0, float("inf")),
                            (1, 1, 1, 0, float("nan")), (-3, 1, 1, 0, 1.0),
                            (1 << 40, 1 << 20, 1 << 10, 0, 1.0)]:
        s = Bd.SruShape.__new__(Bd.SruShape)
        ctypes.Structure.__init__(s, L, B, d, bi, al)
        assert fwd(lib, s) == sru.SRU_ERR_INVALID_ARG, (L, B, d, bi, al)


def test_invalid_pointers_and_codes(lib):
    s = sru.SruShape(8, 2, 64, 0, 1.0)
    assert fwd(lib, s, U=None) == sru.SRU_ERR_INVALID_ARG
    assert b"U" in lib.sru_last_error()
    assert fwd(lib, s, h=None) == sru.SRU_ERR_INVALID_ARG
    assert fwd(lib, s, x=P[1] + 4) == sru.SRU_ERR_INVALID_ARG       # misaligned
    assert b"aligned" in lib.sru_last_error()
    assert fwd(lib, s, c0=P[10] + 8) == sru.SRU_ERR_INVALID_ARG
    assert fwd(lib, s, u_dt=7) == sru.SRU_ERR_INVALID_ARG
    assert fwd(lib, s, h_dt=1) == sru.SRU_ERR_UNSUPPORTED
    # projection
    assert lib.sru_project(ctypes.byref(s), 5, P[0], 0, P[1], 1, P[2], 0, 0, None) == 1
    assert lib.sru_project(ctypes.byref(s), 0, P[0], 0, P[1], 1, P[2], 1, 0, None) == 2
    assert lib.sru_project(ctypes.byref(s), 0, P[0], 0, P[1], 1, P[2], 0, 3, None) == 1
    assert lib.sru_project(ctypes.byref(s), 0, None, 0, P[1], 1, P[2], 0, 0, None) == 1


def test_workspace_errors(lib):
    s = sru.SruShape(8, 2, 64, 1, 1.0)
    need = sru.sru_workspace_size(s, sru.SRU_WS_BACKWARD)
    assert bwd(lib, s, need - 1) == sru.SRU_ERR_WORKSPACE
    assert bwd(lib, s, need, ws=None) == sru.SRU_ERR_WORKSPACE
    assert bwd(lib, s, need, c_seq=None) == sru.SRU_ERR_INVALID_ARG
    assert bwd(lib, s, need, dU=None) == sru.SRU_ERR_INVALID_ARG
    assert bwd(lib, s, need, dU_lp=P[11] + 2) == sru.SRU_ERR_INVALID_ARG
    lneed = sru.sru_workspace_size(s, sru.SRU_WS_LINEAR_BWD, 4)
    assert lin(lib, s, 1, 4, lneed - 256) == sru.SRU_ERR_WORKSPACE
    assert lin(lib, s, 1, 0, lneed) == sru.SRU_ERR_INVALID_ARG
    assert lin(lib, s, 2, 4, lneed) == sru.SRU_ERR_INVALID_ARG
    assert lin(lib, s, 1, 4, lneed, dh=None) == sru.SRU_ERR_INVALID_ARG
    assert lin(lib, s, 0, 4, lneed, h=None) == sru.SRU_ERR_INVALID_ARG
    assert lin(lib, s, 0, 4, lneed, h_dt=1) == sru.SRU_ERR_UNSUPPORTED


# Fake addresses far enough apart for the overlap check of dW.
Q = [(i + 1) << 32 for i in range(4)]


def wgrad(lib, s, ws_bytes, **kw):
    a = dict(dU=Q[0], du_dt=1, X=Q[1], x_dt=0, dW=Q[2], math=1, acc=0, ws=Q[3])
    a.update(kw)
    return lib.sru_project_bwd_weight(ctypes.byref(s), a["dU"], a["du_dt"], a["X"], a["x_dt"],
                                      a["dW"], a["math"], a["acc"], a["ws"], ws_bytes, None)


def test_bwd_weight_validation(lib):
    s = sru.SruShape(128, 16, 128, 0, 1.0)
    need = sru.sru_workspace_size(s, sru.SRU_WS_BWD_WEIGHT)
    assert need > 0 and need == wgrad_ws(384, 128, 2048)   # no copy on this plan
    assert wgrad(lib, s, need, dU=None) == sru.SRU_ERR_INVALID_ARG
    assert wgrad(lib, s, need, X=Q[1] + 2) == sru.SRU_ERR_INVALID_ARG
    assert wgrad(lib, s, need, du_dt=3) == sru.SRU_ERR_INVALID_ARG
    assert wgrad(lib, s, need, math=2) == sru.SRU_ERR_INVALID_ARG
    assert wgrad(lib, s, need, acc=2) == sru.SRU_ERR_INVALID_ARG
    assert wgrad(lib, s, need - 1) == sru.SRU_ERR_WORKSPACE
    assert wgrad(lib, s, need, ws=None) == sru.SRU_ERR_WORKSPACE
    assert wgrad(lib, s, need, ws=Q[3] + 8) == sru.SRU_ERR_INVALID_ARG
    # dW [384, 128] fp32 starting inside dU, or ending inside X
    assert wgrad(lib, s, need, dW=Q[0] + 1024) == sru.SRU_ERR_INVALID_ARG
    assert b"overlap" in lib.sru_last_error()
    assert wgrad(lib, s, need, dW=Q[1] - 4096) == sru.SRU_ERR_INVALID_ARG
    assert b"overlap" in lib.sru_last_error()
    # fp32 arithmetic needs no workspace
    if __import__("torch").cuda.device_count() == 0:
        assert wgrad(lib, s, 0, math=0, ws=None) == sru.SRU_ERR_NO_DEVICE
    # the reported size adds room for a bf16 copy of an fp32 X (L = 512,
    # B = 32, d = 1024: 256 x 256 plan in 5 splits); a workspace that holds
    # only the partial sums is still accepted
    s4 = sru.SruShape(512, 32, 1024, 0, 1.0)
    part, full = wgrad_ws(3072, 1024, 16384), sru.sru_workspace_size(s4, sru.SRU_WS_BWD_WEIGHT)
    assert full == part + 16384 * 1024 * 2 and part > 0
    assert wgrad(lib, s4, part - 1) == sru.SRU_ERR_WORKSPACE
    if __import__("torch").cuda.device_count() == 0:
        assert wgrad(lib, s4, part) == sru.SRU_ERR_NO_DEVICE
        assert wgrad(lib, s4, full) == sru.SRU_ERR_NO_DEVICE
    # no split: no workspace at all
    s1 = sru.SruShape(3, 5, 64, 0, 1.0)
    assert sru.sru_workspace_size(s1, sru.SRU_WS_BWD_WEIGHT) == 0
    assert lib.sru_last_error() == b""


def wgrad_plan(M, N, K):
    """(splits, 256 x 256 tiles) of one weight-gradient product: 128 x 128
    output tiles in 512 block slots or 256 x 256 in 256, 64-deep k-tiles,
    >= 8 k-tiles per split, cost in k-tile rounds plus M*N/1e6 per split."""
    kt = K // 64
    sp, big, best = 1, False, None
    if K % 64 == 0 and kt >= 16:
        for t, slots in ((128, 512), (256, 256)):
            tiles = -(-M // t) * -(-N // t)
            for n in range(1, min(kt // 8, 64) + 1):
                cost = -(-tiles * n // slots) * -(-kt // n) + (M * N * 1e-6 * n if n > 1 else 0)
                if best is None or cost < best:
                    sp, big, best = n, t == 256, cost
    return sp, big


def wgrad_ws(M, N, K):
    """Split-reduction workspace of one weight-gradient product: partial
    products [splits, M, N] when the reduction over L*B is split."""
    sp, _ = wgrad_plan(M, N, K)
    return 0 if sp == 1 else round256(sp * M * N * 4)


def wgrad_query(M, N, K):
    """What the workspace queries report for it: the partial products, then
    room for a bf16 copy of an fp32 [K, N] operand where the product would
    take the K-major LDS-copy kernel (256 x 256 plan, M and N multiples of 8)."""
    _, big = wgrad_plan(M, N, K)
    copy = round256(K * N * 2) if big and M % 8 == 0 and N % 8 == 0 and K % 64 == 0 else 0
    return wgrad_ws(M, N, K) + copy


@pytest.mark.parametrize("L,B,d,bi,di", [(128, 16, 128, 0, 32), (64, 128, 512, 1, 128),
                                         (512, 32, 1024, 0, 256), (3, 5, 64, 0, 16)])
def test_factored_workspace_size(lib, L, B, d, bi, di):
    s = sru.SruShape(L, B, d, bi, 1.0)
    n3 = 3 * (2 if bi else 1) * d
    want = max(wgrad_query(di, d, L * B), wgrad_query(n3, di, L * B))
    assert sru.sru_workspace_size(s, sru.SRU_WS_FACTORED_WEIGHT, di) == want
    assert lib.sru_workspace_size(ctypes.byref(s), sru.SRU_WS_FACTORED_WEIGHT, 0) == 0
    assert b"inner" in lib.sru_last_error()


def fact(lib, s, di, op, **kw):
    a = dict(A=Q[0], a_dt=0, W=Q[1], w_dt=1, C=Q[2], acc=0)
    a.update(kw)
    return lib.sru_project_factored(ctypes.byref(s), di, op, a["A"], a["a_dt"], a["W"],
                                    a["w_dt"], a["C"], a["acc"], None)


def fact_w(lib, s, di, which, ws_bytes, **kw):
    a = dict(G=Q[0], g_dt=1, Y=Q[1], y_dt=0, dW=Q[2], math=1, acc=0, ws=Q[3])
    a.update(kw)
    return lib.sru_project_factored_bwd_weight(ctypes.byref(s), di, which, a["G"], a["g_dt"],
                                               a["Y"], a["y_dt"], a["dW"], a["math"], a["acc"],
                                               a["ws"], ws_bytes, None)


def test_factored_validation(lib):
    s = sru.SruShape(128, 16, 128, 0, 1.0)
    import torch
    gpu = torch.cuda.device_count() > 0
    for op in range(4):
        assert fact(lib, s, 0, op) == sru.SRU_ERR_INVALID_ARG
        assert fact(lib, s, 32, op, A=None) == sru.SRU_ERR_INVALID_ARG
        assert fact(lib, s, 32, op, C=Q[2] + 4) == sru.SRU_ERR_INVALID_ARG
        assert fact(lib, s, 32, op, acc=5) == sru.SRU_ERR_INVALID_ARG
        # C [L*B, >= 32] fp32 starting inside the weights
        assert fact(lib, s, 32, op, C=Q[1] + 256) == sru.SRU_ERR_INVALID_ARG
        assert b"overlaps" in lib.sru_last_error()
        if not gpu:
            assert fact(lib, s, 32, op) == sru.SRU_ERR_NO_DEVICE
            assert fact(lib, s, 32, op, w_dt=0) == sru.SRU_ERR_NO_DEVICE   # fp32 arithmetic
    assert fact(lib, s, 32, 4) == sru.SRU_ERR_INVALID_ARG
    need = sru.sru_workspace_size(s, sru.SRU_WS_FACTORED_WEIGHT, 32)
    assert need > 0
    own = (wgrad_ws(32, 128, 2048), wgrad_ws(384, 32, 2048))   # dWq, dWo
    assert need == max(own) and min(own) > 0
    for which in range(2):
        assert fact_w(lib, s, 32, which, own[which] - 1) == sru.SRU_ERR_WORKSPACE
        assert fact_w(lib, s, 32, which, need, ws=None) == sru.SRU_ERR_WORKSPACE
        assert fact_w(lib, s, 32, which, need, g_dt=4) == sru.SRU_ERR_INVALID_ARG
        assert fact_w(lib, s, 0, which, need) == sru.SRU_ERR_INVALID_ARG
        if not gpu:
            assert fact_w(lib, s, 32, which, need) == sru.SRU_ERR_NO_DEVICE
            assert fact_w(lib, s, 32, which, 0, math=0, ws=None) == sru.SRU_ERR_NO_DEVICE
    assert fact_w(lib, s, 32, 2, need) == sru.SRU_ERR_INVALID_ARG


def attn(lib, s, cfg, ws_bytes, **kw):
    a = dict(X=Q[0], x_dt=0, Wq=Q[1], Wkv=Q[1] + (1 << 30), Wo=Q[1] + (2 << 30), gamma=None,
             beta=None, Qo=Q[2], KV=Q[2] + (1 << 30), R=Q[2] + (2 << 30), U=Q[2] + (3 << 30),
             u_dt=0, ws=Q[3])
    a.update(kw)
    return lib.sru_attention_forward(ctypes.byref(s), ctypes.byref(cfg) if cfg else None, a["X"],
                                     a["x_dt"], a["Wq"], a["Wkv"], a["Wo"], a["gamma"], a["beta"],
                                     a["Qo"], a["KV"], a["R"], a["U"], a["u_dt"], a["ws"],
                                     ws_bytes, None)


def test_attention_workspace_and_validation(lib):
    s = sru.SruShape(64, 4, 128, 0, 1.0)
    cfg = sru.SruAttnCfg(32, mem_len=16, causal=True, layernorm=False, attn_alpha=0.5)
    Lk = 16 + 64
    want = (round256(4 * 64 * Lk * 4) + round256(4 * 64 * Lk * 2) + round256(64 * 4 * 32 * 4))
    assert sru.sru_attention_workspace_size(s, cfg) == want
    bad = [sru.SruAttnCfg(0), sru.SruAttnCfg(32, mem_len=-1), sru.SruAttnCfg(32, attn_alpha=np.nan),
           sru.SruAttnCfg(32, layernorm=True, ln_eps=0.0)]
    c2 = sru.SruAttnCfg(32)
    c2.causal = 2
    bad.append(c2)
    for c in bad:
        assert lib.sru_attention_workspace_size(ctypes.byref(s), ctypes.byref(c)) == 0
        assert lib.sru_last_error() != b""
        assert attn(lib, s, c, want) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, None, want) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, cfg, want, Wq=None) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, cfg, want, KV=Q[2] + (1 << 30) + 8) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, cfg, want, x_dt=5) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, cfg, want, u_dt=5) == sru.SRU_ERR_INVALID_ARG
    assert attn(lib, s, cfg, want - 1) == sru.SRU_ERR_WORKSPACE
    assert attn(lib, s, cfg, want, ws=Q[3] + 16) == sru.SRU_ERR_INVALID_ARG   # 256-byte alignment
    # outputs overlapping each other or an input
    assert attn(lib, s, cfg, want, R=Q[2] + 64) == sru.SRU_ERR_INVALID_ARG
    assert b"overlaps" in lib.sru_last_error()
    assert attn(lib, s, cfg, want, U=Q[1] + 1024) == sru.SRU_ERR_INVALID_ARG
    # U's extent follows its dtype: 64 * 4 * 384 elements of 4 or 2 bytes end
    # before R only in bf16
    nU = 64 * 4 * 384
    assert attn(lib, s, cfg, want, U=Q[2] + (2 << 30) - 2 * nU) == sru.SRU_ERR_INVALID_ARG
    # layer norm needs gamma and beta
    cln = sru.SruAttnCfg(32, layernorm=True)
    nln = sru.sru_attention_workspace_size(s, cln)
    assert attn(lib, s, cln, nln) == sru.SRU_ERR_INVALID_ARG
    import torch
    if torch.cuda.device_count() == 0:   # the addresses here are not memory: no launches
        assert attn(lib, s, cfg, want) == sru.SRU_ERR_NO_DEVICE
        assert attn(lib, s, cfg, want, U=Q[2] + (2 << 30) - 2 * nU,
                    u_dt=sru.SRU_BF16) == sru.SRU_ERR_NO_DEVICE
        assert attn(lib, s, cln, nln, gamma=Q[3] + (1 << 30),
                    beta=Q[3] + (1 << 30) + 4096) == sru.SRU_ERR_NO_DEVICE


def stepc(lib, s, **kw):
    a = dict(x=Q[0], x_dt=0, W=Q[1], w_dt=1, v=Q[2], b=Q[2] + 4096, c=None, h=Q[3],
             cn=Q[3] + (1 << 30))
    a.update(kw)
    return lib.sru_step(ctypes.byref(s), a["x"], a["x_dt"], a["W"], a["w_dt"], a["v"], a["b"],
                        a["c"], a["h"], a["cn"], None)


def test_step_validation(lib):
    s = sru.SruShape(1, 4, 256, 0, 1.0)
    assert stepc(lib, sru.SruShape(2, 4, 256, 0, 1.0)) == sru.SRU_ERR_INVALID_ARG
    assert stepc(lib, sru.SruShape(1, 4, 256, 1, 1.0)) == sru.SRU_ERR_INVALID_ARG
    assert b"unidirectional" in lib.sru_last_error()
    assert stepc(lib, s, W=None) == sru.SRU_ERR_INVALID_ARG
    assert stepc(lib, s, w_dt=3) == sru.SRU_ERR_INVALID_ARG
    assert stepc(lib, s, c=Q[3] + (2 << 30) + 4) == sru.SRU_ERR_INVALID_ARG   # misaligned
    assert stepc(lib, s, h=Q[3], cn=Q[3] + 64) == sru.SRU_ERR_INVALID_ARG       # h and c_next
    assert stepc(lib, s, c=Q[3] + (1 << 30) + 16) == sru.SRU_ERR_INVALID_ARG   # partial alias
    assert stepc(lib, s, h=Q[1] + 64) == sru.SRU_ERR_INVALID_ARG               # h inside W
    import torch
    if torch.cuda.device_count() == 0:
        assert stepc(lib, s) == sru.SRU_ERR_NO_DEVICE
        # the state updated in place is allowed
        assert stepc(lib, s, c=Q[3] + (1 << 30)) == sru.SRU_ERR_NO_DEVICE


def test_round_bf16_validation(lib):
    assert lib.sru_round_bf16(0, Q[0], Q[1], None) == sru.SRU_ERR_INVALID_ARG
    assert lib.sru_round_bf16(16, None, Q[1], None) == sru.SRU_ERR_INVALID_ARG
    assert lib.sru_round_bf16(16, Q[0], Q[0] + 32, None) == sru.SRU_ERR_INVALID_ARG   # overlap
    assert lib.sru_round_bf16(16, Q[0], Q[1] + 2, None) == sru.SRU_ERR_INVALID_ARG    # misaligned
    import torch
    if torch.cuda.device_count() == 0:
        assert lib.sru_round_bf16(16, Q[0], Q[1], None) == sru.SRU_ERR_NO_DEVICE


def test_binding_raises_sru_error(lib):
    s = sru.SruShape(8, 2, 64, 0, 1.0)
    with pytest.raises(sru.SruError) as ei:
        sru.sru_workspace_size(s, 42)
    assert ei.value.status == sru.SRU_ERR_INVALID_ARG


def test_no_device_status_without_gpu(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; this check is for GPU-less hosts")
    s = sru.SruShape(8, 2, 64, 0, 1.0)
    assert fwd(lib, s) == sru.SRU_ERR_NO_DEVICE
    assert b"no HIP device" in lib.sru_last_error()


def test_outputs_overlapping_inputs_are_rejected(lib):
    """An output that overlaps an input or another output is refused before
    any launch (the kernels read and write them concurrently)."""
    s = sru.SruShape(8, 2, 64, 1, 1.0)
    # forward: h on top of U, c_seq on top of h, c_last inside x
    assert fwd(lib, s, h=P[0]) == sru.SRU_ERR_INVALID_ARG
    assert b"overlaps" in lib.sru_last_error()
    assert fwd(lib, s, c_seq=P[4] + 16) == sru.SRU_ERR_INVALID_ARG
    assert fwd(lib, s, c_last=P[1] + 64) == sru.SRU_ERR_INVALID_ARG
    need = sru.sru_workspace_size(s, sru.SRU_WS_BACKWARD)
    assert bwd(lib, s, need, dU=P[6]) == sru.SRU_ERR_INVALID_ARG        # dU on dh
    assert bwd(lib, s, need, dx=P[7] + 256) == sru.SRU_ERR_INVALID_ARG  # dx inside dU
    assert bwd(lib, s, need, ws=P[5]) == sru.SRU_ERR_INVALID_ARG        # workspace on c_seq
    assert bwd(lib, s, need, dv=P[8], db=P[12]) == sru.SRU_ERR_INVALID_ARG   # dv inside dx
    lneed = sru.sru_workspace_size(s, sru.SRU_WS_LINEAR_BWD, 4)
    assert lin(lib, s, 1, 4, lneed, dx=P[6]) == sru.SRU_ERR_INVALID_ARG
    assert lin(lib, s, 0, 4, lneed, h=P[1]) == sru.SRU_ERR_INVALID_ARG
    # projection: C on top of A, and C inside W
    assert lib.sru_project(ctypes.byref(s), 0, P[0], 0, P[1], 1, P[0], 0, 0, None) == 1
    assert b"overlaps" in lib.sru_last_error()
    assert lib.sru_project(ctypes.byref(s), 1, P[0], 0, P[1], 1, P[1] + 512, 0, 0, None) == 1
    # disjoint buffers still reach the device check
    assert lib.sru_project(ctypes.byref(s), 0, P[0], 0, P[1], 1, P[2], 0, 0, None) in (
        sru.SRU_ERR_NO_DEVICE, sru.SRU_OK)


def test_error_word_offset_matches_the_header():
    """The binding reads the error word where include/sru.h says it is."""
    text = open(os.path.join(ROOT, "include", "sru.h")).read()
    m = re.search(r"#define\s+SRU_WS_ERROR_OFFSET\s+(\d+)", text)
    assert m and int(m.group(1)) == Bd.SRU_WS_ERROR_OFFSET


def test_error_word_reader_on_host_bytes():
    """workspace_error_word / check_workspace read 4 bytes at the offset as a
    little-endian int32 (exercised on a host tensor: no device needed)."""
    import torch
    ws = torch.zeros(1024, dtype=torch.uint8)
    assert Bd.workspace_error_word(ws) == 0
    Bd.check_workspace(ws)
    ws[Bd.SRU_WS_ERROR_OFFSET] = 1
    assert Bd.workspace_error_word(ws) == 1
    with pytest.raises(Bd.SruError, match="ran out"):
        Bd.check_workspace(ws, "test")
    ws.zero_()
    ws[Bd.SRU_WS_ERROR_OFFSET + 4] = 7          # the ticket word is not the error word
    assert Bd.workspace_error_word(ws) == 0


# Fake addresses 64 GiB apart: room for the large shape's tensors.
Z = [(i + 1) << 36 for i in range(16)]


def test_static_scratch_backward_validation(lib):
    """sru_backward_static: the static scratch bounds the shape (checked
    before any device use), and its error word must be 4-byte aligned and
    apart from the outputs."""
    def call(s, **kw):
        a = dict(U=Z[0], x=Z[1], v=Z[2], b=Z[3], c0=None, c_seq=Z[5], dh=Z[6], dc_last=None,
                 dU=Z[7], dU_lp=None, dx=Z[8], dv=None, db=None, dc0=None, err=None)
        a.update(kw)
        return lib.sru_backward_static(ctypes.byref(s), a["U"], 0, a["x"], 0, a["v"], a["b"],
                                       a["c0"], a["c_seq"], a["dh"], a["dc_last"], a["dU"],
                                       a["dU_lp"], a["dx"], a["dv"], a["db"], a["dc0"], a["err"],
                                       None)
    big = sru.SruShape(4096, 16, 4096, 0, 1.0)
    assert sru.sru_workspace_size(big, sru.SRU_WS_BACKWARD) > Bd.SRU_BACKWARD_STATIC_SCRATCH_BYTES
    assert call(big) == sru.SRU_ERR_WORKSPACE
    assert b"static scratch" in lib.sru_last_error()
    s = sru.SruShape(512, 32, 1024, 0, 1.0)      # the training step: 6.3 MB of scratch, fits
    assert sru.sru_workspace_size(s, sru.SRU_WS_BACKWARD) <= Bd.SRU_BACKWARD_STATIC_SCRATCH_BYTES
    assert call(s, err=Z[9] + 2) == sru.SRU_ERR_INVALID_ARG
    assert call(s, err=Z[8]) == sru.SRU_ERR_INVALID_ARG          # on top of dx
    assert call(s, dU=None) == sru.SRU_ERR_INVALID_ARG
    assert call(s, err=Z[9]) in (sru.SRU_ERR_NO_DEVICE, sru.SRU_OK)
    # the header's constant is the binding's
    text = open(os.path.join(ROOT, "include", "sru.h")).read()
    m = re.search(r"#define\s+SRU_BACKWARD_STATIC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == Bd.SRU_BACKWARD_STATIC_SCRATCH_BYTES


def test_attention_backward_validation(lib):
    """sru_attention_backward: workspace size and its checks, the d' limit,
    required pointers (gamma and the norm's gradients only with layer norm),
    and outputs overlapping inputs, all before any device use."""
    s = sru.SruShape(16, 2, 64, 0, 1.0)
    cfg = Bd.SruAttnCfg(16, 8, True, True, 0.5, 1e-5)
    need = Bd.sru_attention_backward_workspace_size(s, cfg)
    assert need > 0 and need % 256 == 0

    def call(c=cfg, ws_bytes=need, **kw):
        a = dict(X=Z[0], Wq=Z[1], Wkv=Z[2], Wo=Z[3], gamma=Z[4], Q=Z[5], KV=Z[6], R=Z[7], dU=Z[8],
                 dX=Z[9], dWq=Z[10], dWkv=Z[11], dWo=Z[12], dalpha=Z[13], dgamma=Z[14],
                 dbeta=Z[15], ws=Z[15] + (1 << 20))
        a.update(kw)
        return lib.sru_attention_backward(
            ctypes.byref(s), ctypes.byref(c), a["X"], 0, a["Wq"], a["Wkv"], a["Wo"], a["gamma"],
            a["Q"], a["KV"], a["R"], a["dU"], 0, a["dX"], 0, a["dWq"], a["dWkv"], a["dWo"],
            a["dalpha"], a["dgamma"], a["dbeta"], a["ws"], ws_bytes, None)
    assert call() in (sru.SRU_ERR_NO_DEVICE, sru.SRU_OK)
    assert call(ws_bytes=need - 256) == sru.SRU_ERR_WORKSPACE
    assert call(ws=None) == sru.SRU_ERR_WORKSPACE
    assert call(gamma=None) == sru.SRU_ERR_INVALID_ARG
    assert call(dgamma=None) == sru.SRU_ERR_INVALID_ARG
    assert call(dX=Z[0]) == sru.SRU_ERR_INVALID_ARG             # dX on top of X
    assert b"overlaps" in lib.sru_last_error()
    assert call(dWq=Z[5] + 64) == sru.SRU_ERR_INVALID_ARG       # dWq inside Q
    no_ln = Bd.SruAttnCfg(16, 8, True, False, 0.5, 1e-5)
    assert call(c=no_ln, gamma=None, dgamma=None, dbeta=None,
                ws_bytes=Bd.sru_attention_backward_workspace_size(s, no_ln)) in (
        sru.SRU_ERR_NO_DEVICE, sru.SRU_OK)
    wide = Bd.SruAttnCfg(2048, 0, True, False, 0.5, 1e-5)
    assert call(c=wide, ws_bytes=Bd.sru_attention_backward_workspace_size(s, wide)) == \
        sru.SRU_ERR_UNSUPPORTED
