"""CPU oracle for one SRU layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and this package never imports the product.

Everything here is plain double-precision evaluation of the Simple Recurrent
Unit as defined in "When Attention Meets Fast Recurrence: Training Language
Models with Reduced Compute" (Lei), background section, Eqs. 1-5, with the
readings listed in the C source header (highway scale alpha, initial state
c0, bidirectional = two independent directions, backward by the chain rule,
linear mode = the same recurrence with v = 0).  The arithmetic lives in
``sru_oracle.c``; this module only marshals numpy arrays.

Layouts (row-major): U [L, B, ndir, 3, d]; x [L, B, d]; v, b [ndir, 2, d];
c0 [ndir, B, d]; h, c [L, B, ndir, d]; c_last [ndir, B, d].

The factorised projection of the same paper (Fig. 2(b): U = Wo (Wq X), inner
dimension d' < d) and its gradients are compositions of a plain double
matrix product (``matmul``).

Pins (tests/test_oracle_pins.py): textbook matmul, saturated gates, the EMA
closed form, brute-force unrolled recurrences at L <= 4, central finite
differences for every gradient, the bidirectional time-flip invariant,
channel/batch permutation equivariance, and for the factorised projection
associativity (one projection with the product weight), hand-computed bf16
rounding of X and Q, and central differences; for the SRU++ attention, the
uniform-weight average, the single visible key, the two-key sigmoid form,
saturation, convexity and key-permutation invariance, rounded weights, the
layer-norm closed form, and the pages' alpha = 0 reduction to the factorised
projection; for its composition (attention_project) at alpha != 0, the
closed form with all keys zero (uniform weights: A is a mean of value rows,
context rows first), the layer norm applied by hand before Wo, and the bf16
rounding points worked out by hand on a one-key example.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_sru.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.sru_oracle_sigmoid.restype = ctypes.c_double
    lib.sru_oracle_sigmoid.argtypes = [ctypes.c_double]
    lib.sru_oracle_round_bf16.restype = ctypes.c_float
    lib.sru_oracle_round_bf16.argtypes = [ctypes.c_float]
    lib.sru_oracle_attention_backward.restype = None
    lib.sru_oracle_attention_backward.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _dp, _dp,
                                                  _dp, _dp, _dp, _dp, _dp]
    lib.sru_oracle_layernorm_backward.restype = None
    lib.sru_oracle_layernorm_backward.argtypes = [_i64, _i64, _dp, _dp, ctypes.c_double, _dp,
                                                  _dp, _dp, _dp]
    lib.sru_oracle_project.restype = None
    lib.sru_oracle_project.argtypes = [_i64, _i64, _i64, _fp, ctypes.c_int, _fp,
                                       _ip, _i64, _ip, _i64, _dp]
    lib.sru_oracle_project_bwd_data.restype = None
    lib.sru_oracle_project_bwd_data.argtypes = [_i64, _i64, _i64, _dp, _fp,
                                                _ip, _i64, _dp]
    d = ctypes.c_double
    lib.sru_oracle_project_bwd_weight.restype = None
    lib.sru_oracle_project_bwd_weight.argtypes = [_i64, _i64, _i64, _dp, _fp, ctypes.c_int, _dp]
    lib.sru_oracle_chain_forward.restype = None
    lib.sru_oracle_chain_forward.argtypes = [_i64, ctypes.c_int, ctypes.c_int, d,
                                             _dp, _dp, _dp, _dp,
                                             d, d, d, d, d, _dp, _dp, _dp]
    lib.sru_oracle_chain_backward.restype = None
    lib.sru_oracle_chain_backward.argtypes = [_i64, ctypes.c_int, ctypes.c_int, d,
                                              _dp, _dp, _dp, _dp,
                                              d, d, d, d, d, _dp, _dp, d,
                                              _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.sru_oracle_forward.restype = None
    lib.sru_oracle_forward.argtypes = [_i64, _i64, _i64, ctypes.c_int, d,
                                       _dp, _fp, _fp, _fp, _fp, _dp, _dp, _dp]
    lib.sru_oracle_backward.restype = None
    lib.sru_oracle_backward.argtypes = [_i64, _i64, _i64, ctypes.c_int, d,
                                        _dp, _fp, _fp, _fp, _fp, _dp, _fp, _fp,
                                        _dp, _dp, _dp, _dp, _dp]
    lib.sru_oracle_round_bf16_n.restype = None
    lib.sru_oracle_round_bf16_n.argtypes = [_i64, _fp, _fp]
    lib.sru_oracle_matmul.restype = None
    lib.sru_oracle_matmul.argtypes = [_i64, _i64, _i64, _dp, ctypes.c_int, _dp, ctypes.c_int,
                                      _dp]
    lib.sru_oracle_attention.restype = None
    lib.sru_oracle_attention.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int, _dp, _dp, _dp,
                                         ctypes.c_int, _dp]
    lib.sru_oracle_layernorm.restype = None
    lib.sru_oracle_layernorm.argtypes = [_i64, _i64, _dp, _dp, _dp, ctypes.c_double, _dp]
    lib.sru_oracle_num_threads.restype = ctypes.c_int
    lib.sru_oracle_num_threads.argtypes = []
    _lib = lib
    return lib


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data_as(_fp)


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _i64arr(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(_ip)


def _optf32(a):
    if a is None:
        return None, None
    return _f32(a)


def set_num_threads(n: int) -> None:
    """Threads the whole-tensor routines use from now on (1: single-threaded)."""
    lib = _load()
    lib.sru_oracle_set_num_threads.restype = None
    lib.sru_oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.sru_oracle_set_num_threads(int(n))


def num_threads() -> int:
    """Threads the oracle's whole-tensor routines spread independent chains over."""
    return int(_load().sru_oracle_num_threads())


def sigmoid(z: float) -> float:
    return float(_load().sru_oracle_sigmoid(float(z)))


def round_bf16(a) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned widened to fp32.  Wider
    values are taken to fp32 first, as a kernel's fp32 register holds them."""
    flat, pin = _f32(np.asarray(a).ravel())
    out = np.empty_like(flat)
    _load().sru_oracle_round_bf16_n(flat.size, pin, out.ctypes.data_as(_fp))
    return out.reshape(np.shape(a))


def matmul(A, B, a_km: bool = False, b_nk: bool = False) -> np.ndarray:
    """C = A B in double: A [M, K] (or [K, M] with a_km), B [K, N] (or [N, K]
    with b_nk)."""
    A, pa = _f64(A)
    B, pb = _f64(B)
    M, K = (A.shape[1], A.shape[0]) if a_km else A.shape
    N, K2 = B.shape if b_nk else (B.shape[1], B.shape[0])
    assert K == K2, (A.shape, B.shape, a_km, b_nk)
    C = np.empty((M, N), dtype=np.float64)
    _load().sru_oracle_matmul(M, N, K, pa, int(bool(a_km)), pb, int(bool(b_nk)),
                              C.ctypes.data_as(_dp))
    return C


def _maybe_bf16(a, on):
    return round_bf16(a).astype(np.float64) if on else np.asarray(a, np.float64)


def factored_project(X, Wq, Wo, round_ops: bool):
    """The factorised projection of the SRU++ paper (Fig. 2(b); the same map is
    its attention layer's output projection with alpha = 0): Q = Xt Wq^T,
    U = Qt Wo^T, with X [M, d], Wq [d', d], Wo [ndir*3d, d'].  round_ops:
    X and Q enter their products rounded to bf16 (nearest even), as the bf16
    kernels multiply them; the weights are used as given."""
    Q = matmul(_maybe_bf16(X, round_ops), Wq, b_nk=True)
    U = matmul(_maybe_bf16(Q, round_ops), Wo, b_nk=True)
    return {"Q": Q, "U": U}


def factored_project_backward(X, Q, Wq, Wo, dU, round_ops: bool):
    """Gradients of factored_project given dU (chain rule through both
    products): dQ = dUt Wo, dX = dQt Wq, dWo = dUt^T Qt, dWq = dQt^T Xt, where
    t marks bf16 rounding of the activation-side operands when round_ops."""
    dUt = _maybe_bf16(dU, round_ops)
    dQ = matmul(dUt, Wo)
    dQt = _maybe_bf16(dQ, round_ops)
    return {"dQ": dQ,
            "dX": matmul(dQt, Wq),
            "dWo": matmul(dUt, _maybe_bf16(Q, round_ops), a_km=True),
            "dWq": matmul(dQt, _maybe_bf16(X, round_ops), a_km=True)}


def project(A, W, round_a: bool, rows=None, cols=None) -> np.ndarray:
    """Eq. 1 on selected rows x columns: out[i, k] = sum_q Atilde[rows[i], q] W[cols[k], q]."""
    A, pa = _f32(A)
    W, pw = _f32(W)
    M, K = A.shape
    N, K2 = W.shape
    assert K == K2
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    rows, pr = _i64arr(rows)
    cols, pc = _i64arr(cols)
    out = np.empty((rows.size, cols.size), dtype=np.float64)
    _load().sru_oracle_project(M, N, K, pa, int(bool(round_a)), pw, pr, rows.size,
                               pc, cols.size, out.ctypes.data_as(_dp))
    return out


def project_bwd_data(G, W, rows=None) -> np.ndarray:
    """out[i, q] = sum_n G[rows[i], n] W[n, q] (gradient of Eq. 1 w.r.t. its input)."""
    G, pg = _f64(G)
    W, pw = _f32(W)
    M, N = G.shape
    N2, K = W.shape
    assert N == N2
    rows = np.arange(M) if rows is None else np.asarray(rows)
    rows, pr = _i64arr(rows)
    out = np.empty((rows.size, K), dtype=np.float64)
    _load().sru_oracle_project_bwd_data(M, N, K, pg, pw, pr, rows.size,
                                        out.ctypes.data_as(_dp))
    return out


def project_bwd_weight(G, X, round_x: bool) -> np.ndarray:
    """out[n, q] = sum_m G[m, n] Xtilde[m, q] (gradient of Eq. 1 w.r.t. its weights)."""
    G, pg = _f64(G)
    X, px = _f32(X)
    M, N = G.shape
    M2, K = X.shape
    assert M == M2
    out = np.empty((N, K), dtype=np.float64)
    _load().sru_oracle_project_bwd_weight(M, N, K, pg, px, int(bool(round_x)),
                                          out.ctypes.data_as(_dp))
    return out


def chain_forward(uf, ur, ux, x, vf, vr, bf, br, c0, alpha, direction=0, linear=False):
    """One chain (Eqs. 2-5).  Returns (h[L], c[L], c_last).

    linear=True: the linear mode, whose gates do not see the state (vf, vr
    ignored; the v*c terms are not formed)."""
    uf, p1 = _f64(uf)
    ur, p2 = _f64(ur)
    ux, p3 = _f64(ux)
    x, p4 = _f64(x)
    L = uf.size
    h = np.empty(L)
    c = np.empty(L)
    cl = ctypes.c_double()
    _load().sru_oracle_chain_forward(L, int(direction), int(bool(linear)), float(alpha),
                                     p1, p2, p3, p4,
                                     float(vf), float(vr), float(bf), float(br), float(c0),
                                     h.ctypes.data_as(_dp), c.ctypes.data_as(_dp),
                                     ctypes.byref(cl))
    return h, c, cl.value


def chain_backward(uf, ur, ux, x, vf, vr, bf, br, c0, c, dh, dc_last, alpha, direction=0,
                   linear=False):
    """Chain rule through one chain.  Returns a dict of per-step and scalar grads.

    linear=True as for chain_forward: the state adjoint has no gate terms."""
    uf, p1 = _f64(uf)
    ur, p2 = _f64(ur)
    ux, p3 = _f64(ux)
    x, p4 = _f64(x)
    c, pc = _f64(c)
    dh, pd = _f64(dh)
    L = uf.size
    outs = {k: np.empty(L) for k in ("duf", "dur", "dux", "dx_hw")}
    sc = {k: ctypes.c_double() for k in ("dvf", "dvr", "dbf", "dbr", "dc0")}
    _load().sru_oracle_chain_backward(
        L, int(direction), int(bool(linear)), float(alpha), p1, p2, p3, p4,
        float(vf), float(vr), float(bf), float(br), float(c0), pc, pd, float(dc_last),
        *(outs[k].ctypes.data_as(_dp) for k in ("duf", "dur", "dux", "dx_hw")),
        *(ctypes.byref(sc[k]) for k in ("dvf", "dvr", "dbf", "dbr", "dc0")))
    res = dict(outs)
    res.update({k: v.value for k, v in sc.items()})
    return res


def forward(U, x, v, b, c0, alpha):
    """Whole-tensor forward.  U [L,B,ndir,3,d] -> h, c [L,B,ndir,d], c_last [ndir,B,d].

    U may be fp32 values (given U) or the oracle's own double projection.
    v None: the linear mode (gates that do not see the state)."""
    U, pu = _f64(U)
    L, B, ndir, three, d = U.shape
    assert three == 3
    x, px = _f32(x)
    v, pv = _optf32(v)
    b, pb = _f32(b)
    c0, pc0 = _optf32(c0)
    h = np.empty((L, B, ndir, d))
    c = np.empty((L, B, ndir, d))
    cl = np.empty((ndir, B, d))
    _load().sru_oracle_forward(L, B, d, ndir, float(alpha), pu, px, pv, pb, pc0,
                               h.ctypes.data_as(_dp), c.ctypes.data_as(_dp),
                               cl.ctypes.data_as(_dp))
    return {"h": h, "c": c, "c_last": cl}


def backward(U, x, v, b, c0, c, dh, dc_last, alpha):
    """Whole-tensor backward given the oracle's own forward states ``c``.

    v None: the linear mode, as for forward."""
    U, pu = _f64(U)
    L, B, ndir, _, d = U.shape
    x, px = _f32(x)
    v, pv = _optf32(v)
    b, pb = _f32(b)
    c0, pc0 = _optf32(c0)
    c, pc = _f64(c)
    dh, pdh = _f32(dh)
    dc_last, pdcl = _optf32(dc_last)
    dU = np.empty(U.shape)
    dx = np.empty((L, B, d))
    dv = np.empty((ndir, 2, d))
    db = np.empty((ndir, 2, d))
    dc0 = np.empty((ndir, B, d))
    _load().sru_oracle_backward(L, B, d, ndir, float(alpha), pu, px, pv, pb, pc0, pc,
                                pdh, pdcl, dU.ctypes.data_as(_dp), dx.ctypes.data_as(_dp),
                                dv.ctypes.data_as(_dp), db.ctypes.data_as(_dp),
                                dc0.ctypes.data_as(_dp))
    return {"dU": dU, "dx_hw": dx, "dv": dv, "db": db, "dc0": dc0}


def layer_U(X, W, round_x: bool, L, B, ndir, d):
    """Eq. 1 for a whole layer: X [L,B,d], W [ndir*3d, d] -> U [L,B,ndir,3,d] (double)."""
    U = project(np.asarray(X, np.float32).reshape(L * B, d), W, round_x)
    return U.reshape(L, B, ndir, 3, d)


def chain_inputs_from_projection(X, W, round_x, L, B, d, ndir, direction, b, j):
    """The three U slots of chain (direction, b, j) computed by Eq. 1 from X and W."""
    rows = np.arange(L) * B + b
    cols = [(direction * 3 + g) * d + j for g in range(3)]
    u = project(np.asarray(X, np.float32).reshape(L * B, d), W, round_x, rows=rows, cols=cols)
    return u[:, 0], u[:, 1], u[:, 2]


def attention(Q, K, V, mem_len: int, causal: bool, round_p: bool = False) -> np.ndarray:
    """Single-head scaled dot-product attention of an SRU++ layer.  Q [L, B, d'];
    K, V [mem_len + L, B, d'] (the previous segment's rows first).  Returns
    A [L, B, d'] (see sru_oracle_attention)."""
    Q, pq = _f64(Q)
    K, pk = _f64(K)
    V, pv = _f64(V)
    L, B, dp = Q.shape
    assert K.shape == (mem_len + L, B, dp) and V.shape == K.shape
    A = np.empty_like(Q)
    _load().sru_oracle_attention(L, B, dp, int(mem_len), int(bool(causal)), pq, pk, pv,
                                 int(bool(round_p)), A.ctypes.data_as(_dp))
    return A


def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    """Layer normalisation over the last dimension (biased variance)."""
    x, px = _f64(x)
    g, pg = _f64(gamma)
    b, pb = _f64(beta)
    w = x.shape[-1]
    y = np.empty_like(x)
    _load().sru_oracle_layernorm(x.size // w, w, px, pg, pb, float(eps), y.ctypes.data_as(_dp))
    return y


def attention_project(X, Wq, Wk, Wv, Wo, L, B, alpha, mem_len=0, Kmem=None, Vmem=None,
                      causal=True, ln=None, round_ops=False):
    """The U-producer of an SRU++ layer (SRU++ paper, section on SRU++):
    Q = Xt Wq^T, K = Qt Wk^T, V = Qt Wv^T over this segment's L steps (the
    previous segment's keys and values Kmem, Vmem [mem_len, B, d'] in front),
    A = attention(Q, K, V), R = Q + alpha A, optionally R <- layernorm(R)
    (ln = (gamma, beta, eps)), U = Rt Wo^T.  X is [L*B, d]; returns a dict
    with Q, K, V (all rows, memory included), A, R, U as [L*B, .] or
    [Lk, B, .] arrays.  round_ops rounds every product's activation operand to
    bf16 and the attention weights p to bf16, as the bf16 GPU path does."""
    dp = Wq.shape[0]
    Q = matmul(_maybe_bf16(X, round_ops), Wq, b_nk=True)
    Qt = _maybe_bf16(Q, round_ops)
    Kc = matmul(Qt, Wk, b_nk=True).reshape(L, B, dp)
    Vc = matmul(Qt, Wv, b_nk=True).reshape(L, B, dp)
    if mem_len:
        Kc = np.concatenate([np.asarray(Kmem, np.float64), Kc])
        Vc = np.concatenate([np.asarray(Vmem, np.float64), Vc])
    A = attention(_maybe_bf16(Q, round_ops).reshape(L, B, dp), _maybe_bf16(Kc, round_ops),
                  _maybe_bf16(Vc, round_ops), mem_len, causal, round_p=round_ops)
    R = Q + alpha * A.reshape(L * B, dp)
    if ln is not None:
        R = layernorm(R, ln[0], ln[1], ln[2])
    U = matmul(_maybe_bf16(R, round_ops), Wo, b_nk=True)
    return {"Q": Q, "K": Kc, "V": Vc, "A": A.reshape(L * B, dp), "R": R, "U": U}


def attention_backward(Q, K, V, dA, mem_len: int, causal: bool):
    """Gradient of ``attention`` with respect to Q, K and V given dA [L, B, d']
    (see sru_oracle_attention_backward).  Returns (dQ [L, B, d'], dK, dV
    [mem_len + L, B, d'])."""
    Q, pq = _f64(Q)
    K, pk = _f64(K)
    V, pv = _f64(V)
    dA, pa = _f64(dA)
    L, B, dp = Q.shape
    assert K.shape == (mem_len + L, B, dp) and V.shape == K.shape and dA.shape == Q.shape
    dQ = np.empty_like(Q)
    dK = np.empty_like(K)
    dV = np.empty_like(V)
    _load().sru_oracle_attention_backward(L, B, dp, int(mem_len), int(bool(causal)), pq, pk, pv,
                                          pa, dQ.ctypes.data_as(_dp), dK.ctypes.data_as(_dp),
                                          dV.ctypes.data_as(_dp))
    return dQ, dK, dV


def layernorm_backward(x, gamma, eps: float, dy):
    """Gradient of ``layernorm`` given dy: (dx, dgamma, dbeta)."""
    x, px = _f64(x)
    g, pg = _f64(gamma)
    dy, pd = _f64(dy)
    w = x.shape[-1]
    dx = np.empty_like(x)
    dg = np.empty(w)
    db = np.empty(w)
    _load().sru_oracle_layernorm_backward(x.size // w, w, px, pg, float(eps), pd,
                                          dx.ctypes.data_as(_dp), dg.ctypes.data_as(_dp),
                                          db.ctypes.data_as(_dp))
    return dx, dg, db


def attention_project_backward(X, Wq, Wk, Wv, Wo, L, B, alpha, dU, mem_len=0, Kmem=None,
                               Vmem=None, causal=True, ln=None, round_ops=False):
    """Gradients of ``attention_project`` (chain rule; the pages give no
    backward) for the upstream gradient dU [L*B, n3] of U: with respect to X,
    Wq, Wk, Wv, Wo, the residual weight alpha and, when ln, gamma and beta.
    The previous segment's keys and values (Kmem, Vmem) are constants: no
    gradient flows into them.  round_ops rounds every product's operands to
    bf16 where the GPU path does (the forward's, and in the backward dU, R,
    dO, dS', dK, dV, dQ as they enter their products), the rounding itself
    passed through as the identity.  Returns a dict of the gradients and the
    intermediates dR, dS, dO, dQ."""
    f = attention_project(X, Wq, Wk, Wv, Wo, L, B, alpha, mem_len, Kmem, Vmem, causal, ln,
                          round_ops)
    rb = lambda a: _maybe_bf16(a, round_ops)
    dp = Wq.shape[0]
    Q, A, R = f["Q"], f["A"], f["R"]
    dUt = rb(dU)
    dWo = matmul(dUt, rb(R), a_km=True)                  # dU^T R~         [n3, dp]
    dR = matmul(dUt, Wo)                                 # dU Wo           [LB, dp]
    S = Q + alpha * A                                    # before the norm
    if ln is not None:
        dS, dgamma, dbeta = layernorm_backward(S, ln[0], ln[2], dR)
    else:
        dS, dgamma, dbeta = dR, None, None
    dalpha = float(np.sum(dS * A))
    dO = alpha * dS
    Qt = rb(Q).reshape(L, B, dp)
    dQa, dK, dV = attention_backward(Qt, rb(f["K"]), rb(f["V"]), rb(dO).reshape(L, B, dp),
                                     mem_len, causal)
    dKs = dK[mem_len:].reshape(L * B, dp)                # this segment's keys and values
    dVs = dV[mem_len:].reshape(L * B, dp)
    Qr = rb(Q)
    dWk = matmul(rb(dKs), Qr, a_km=True)
    dWv = matmul(rb(dVs), Qr, a_km=True)
    dQ = dS + dQa.reshape(L * B, dp) + matmul(rb(dKs), Wk) + matmul(rb(dVs), Wv)
    dQt = rb(dQ)
    dWq = matmul(dQt, rb(X), a_km=True)
    dX = matmul(dQt, Wq)
    return {"dX": dX, "dWq": dWq, "dWk": dWk, "dWv": dWv, "dWo": dWo, "dalpha": dalpha,
            "dgamma": dgamma, "dbeta": dbeta, "dR": dR, "dS": dS, "dO": dO, "dQ": dQ,
            "dK": dKs, "dV": dVs, "A": A}


def step(x, W, v, b, c_prev, alpha, round_x: bool):
    """One step of a unidirectional layer (Eq. 1, then Eqs. 2-5 at L = 1):
    x [B, d], W [3d, d], v, b [2, d], c_prev [B, d] or None (zero state).
    Returns (h, c_next), each [B, d]."""
    x = np.asarray(x, np.float32)
    B, d = x.shape
    U = project(x, W, round_x).reshape(1, B, 1, 3, d)
    c0 = np.zeros((1, B, d), np.float32) if c_prev is None else np.asarray(c_prev).reshape(1, B, d)
    fo = forward(U, x.reshape(1, B, d), np.asarray(v).reshape(1, 2, d),
                 np.asarray(b).reshape(1, 2, d), c0, alpha)
    return fo["h"][0, :, 0], fo["c_last"][0]
