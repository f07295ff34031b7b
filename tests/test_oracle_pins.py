"""Pins of the CPU oracle to things other than itself (CPU only).

The pages print no worked numeric example for the recurrence, so every pin here
is one the equations and mathematics fix on their own:

* the projection (Eq. 1 of the SRU++ paper) against numpy's float64 matmul on
  the same bf16-rounded operands, with non-square shapes so a transposed
  operand fails;
* the oracle's bf16 rounding against torch's own fp32 -> bf16 cast;
* saturated gates (f = 0 / 1, r = 0 / 1), where Eqs. 4-5 collapse to
  copies of U's candidate slot, c0, c or alpha * x;
* the exponential-moving-average closed form of Eq. 4 when v = 0 and the
  forget gate is constant, and its time-varying-gate sum form (linear mode);
* brute-force unrolled recurrences at L <= 4, written as explicit nested
  expressions in both directions with every term non-zero;
* central finite differences of a scalar loss for every gradient the
  backward returns (dU, dx, dv, db, dc0, and dX through the projection);
* invariants: direction 1 equals direction 0 on time-reversed inputs, and
  permuting channels or batch rows permutes the outputs (the independence
  remark after Eq. 5).
"""
import math

import numpy as np
import pytest

import oracle


def sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def rand_problem(rng, L, B, d, nd, v_scale=0.5, b_scale=0.5):
    U = rng.standard_normal((L, B, nd, 3, d))
    x = rng.standard_normal((L, B, d)).astype(np.float32).astype(np.float64)
    v = rng.uniform(-v_scale, v_scale, (nd, 2, d))
    b = rng.uniform(-b_scale, b_scale, (nd, 2, d))
    c0 = rng.standard_normal((nd, B, d))
    # the whole-tensor routines take x, v, b, c0 as float32: keep them exactly representable
    v = v.astype(np.float32).astype(np.float64)
    b = b.astype(np.float32).astype(np.float64)
    c0 = c0.astype(np.float32).astype(np.float64)
    return U, x, v, b, c0


# --------------------------------------------------------------------------
# projection and bf16 rounding
# --------------------------------------------------------------------------

def test_round_bf16_matches_torch_cast():
    import torch
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 2000),
        # exact ties between two bf16 neighbours, both parities of the kept bit
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 3.0 + 2 ** -7],
                 np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1e-40, -1e-42], np.float32),
    ]).astype(np.float32)
    ours = oracle.round_bf16(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    nan = oracle.round_bf16(np.array([np.nan], np.float32))
    assert np.isnan(nan[0])


@pytest.mark.parametrize("round_a", [False, True])
def test_project_matches_numpy_matmul(round_a):
    import torch
    rng = np.random.default_rng(3)
    M, N, K = 37, 23, 19
    A = rng.standard_normal((M, K)).astype(np.float32)
    W = rng.standard_normal((N, K)).astype(np.float32)
    At = torch.from_numpy(A).to(torch.bfloat16).to(torch.float32).numpy() if round_a else A
    ref = At.astype(np.float64) @ W.astype(np.float64).T
    got = oracle.project(A, W, round_a)
    assert got.shape == (M, N)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))
    rows, cols = [36, 0, 5], [22, 1]
    sub = oracle.project(A, W, round_a, rows=rows, cols=cols)
    assert np.array_equal(sub, got[np.ix_(rows, cols)])


def test_project_bwd_data_matches_numpy_matmul():
    rng = np.random.default_rng(4)
    M, N, K = 29, 31, 7
    G = rng.standard_normal((M, N))
    W = rng.standard_normal((N, K)).astype(np.float32)
    ref = G @ W.astype(np.float64)
    got = oracle.project_bwd_data(G, W)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("round_x", [False, True])
def test_project_bwd_weight_matches_numpy_matmul(round_x):
    import torch
    rng = np.random.default_rng(8)
    M, N, K = 41, 13, 9
    G = rng.standard_normal((M, N))
    X = rng.standard_normal((M, K)).astype(np.float32)
    Xt = torch.from_numpy(X).to(torch.bfloat16).to(torch.float32).numpy() if round_x else X
    ref = G.T @ Xt.astype(np.float64)
    got = oracle.project_bwd_weight(G, X, round_x)
    assert got.shape == (N, K)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_project_bwd_weight_is_the_weight_derivative_of_the_projection():
    """Independent pin: central differences of sum(U * G) with U = Xt W^T,
    taken through the forward projection oracle.  U is linear in W and the
    perturbed weights are exact in float32, so the difference quotient is the
    derivative up to double rounding."""
    rng = np.random.default_rng(9)
    M, N, K = 11, 5, 4
    X = rng.standard_normal((M, K)).astype(np.float32)
    W = (np.round(rng.standard_normal((N, K)) * 256) / 256).astype(np.float32)
    G = rng.standard_normal((M, N))
    dW = oracle.project_bwd_weight(G, X, True)
    h = 2.0 ** -6
    for n in range(N):
        for q in range(K):
            Wp, Wm = W.copy(), W.copy()
            Wp[n, q] += h
            Wm[n, q] -= h
            fd = (np.sum(oracle.project(X, Wp, True) * G) -
                  np.sum(oracle.project(X, Wm, True) * G)) / (2 * h)
            assert fd == pytest.approx(dW[n, q], rel=1e-11, abs=1e-11)


@pytest.mark.parametrize("a_km,b_nk", [(False, False), (True, False), (False, True),
                                       (True, True)])
def test_matmul_matches_numpy(a_km, b_nk):
    rng = np.random.default_rng(21)
    M, N, K = 7, 5, 9
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    got = oracle.matmul(A.T.copy() if a_km else A, B.T.copy() if b_nk else B, a_km, b_nk)
    np.testing.assert_allclose(got, A @ B, rtol=1e-13, atol=1e-13)


def test_factored_projection_is_one_projection_with_the_product_weight():
    """Closed form (associativity): Wo (Wq X^T) = (Wo Wq) X^T, so without
    rounding the factorised map equals Eq. 1's projection with the weight
    Wo Wq, evaluated here by the Eq. 1 oracle in one product."""
    rng = np.random.default_rng(22)
    M, d, dp, n3 = 13, 8, 3, 24
    # dyadic values with few bits: every product and sum below is exact in
    # double, and Wo Wq is exact in float32 as the Eq. 1 oracle takes it
    X = (rng.integers(-8, 8, (M, d)) / 4).astype(np.float32)
    Wq = rng.integers(-4, 4, (dp, d)) / 8
    Wo = rng.integers(-4, 4, (n3, dp)) / 8
    f = oracle.factored_project(X, Wq, Wo, False)
    Wcomb = (Wo @ Wq).astype(np.float32)
    assert np.array_equal(Wcomb.astype(np.float64), Wo @ Wq)
    assert np.array_equal(f["U"], oracle.project(X, Wcomb, False))
    assert np.array_equal(f["Q"], oracle.project(X, Wq.astype(np.float32), False))


def test_factored_projection_rounds_x_and_q():
    """Hand-computed: with Wq = Wo = [[1]] the map is U = bf16(bf16(x)).
    x = 1 + 2^-9 lies below half an ulp of bf16 at 1 (2^-8) and rounds to 1;
    x = 1 + 3 * 2^-9 lies above it and rounds to 1 + 2^-7."""
    one = np.ones((1, 1))
    for x, want in ((1 + 2 ** -9, 1.0), (1 + 3 * 2 ** -9, 1 + 2 ** -7)):
        X = np.array([[x]], np.float32)
        assert oracle.factored_project(X, one, one, True)["U"][0, 0] == want
        assert oracle.factored_project(X, one, one, False)["U"][0, 0] == np.float32(x)
    # Q rounded between the products: x = 1, Wq = [[1 + 2^-9]] gives Q = 1 + 2^-9,
    # which enters the second product as 1
    f = oracle.factored_project(np.ones((1, 1), np.float32), np.array([[1 + 2 ** -9]]), one, True)
    assert f["Q"][0, 0] == 1 + 2 ** -9 and f["U"][0, 0] == 1.0


def test_factored_projection_backward_finite_differences():
    """Central differences of s = sum(G * U(X, Wq, Wo)) for every entry of X,
    Wq and Wo (no rounding).  U is bilinear in (Wq, Wo) and linear in X, so
    the central quotient is exact up to double rounding."""
    rng = np.random.default_rng(23)
    M, d, dp, n3 = 5, 4, 2, 6
    X = rng.standard_normal((M, d)).astype(np.float32).astype(np.float64)
    Wq = rng.standard_normal((dp, d))
    Wo = rng.standard_normal((n3, dp))
    G = rng.standard_normal((M, n3))
    f = oracle.factored_project(X.astype(np.float32), Wq, Wo, False)
    g = oracle.factored_project_backward(X.astype(np.float32), f["Q"], Wq, Wo, G, False)

    def s_of(X_, Wq_, Wo_):
        # the map written out directly, so the pin does not go through the oracle
        return float(np.sum(G * ((X_ @ Wq_.T) @ Wo_.T)))

    h = 2.0 ** -10
    for name, arr in (("dX", X), ("dWq", Wq), ("dWo", Wo)):
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args_p = [p if a is arr else a for a in (X, Wq, Wo)]
            args_m = [m if a is arr else a for a in (X, Wq, Wo)]
            fd = (s_of(*args_p) - s_of(*args_m)) / (2 * h)
            assert fd == pytest.approx(g[name][idx], rel=1e-9, abs=1e-9), (name, idx)
    # dQ is the gradient with respect to the intermediate Q
    np.testing.assert_allclose(g["dQ"], G @ Wo, rtol=1e-12, atol=1e-12)


def test_sigmoid_values():
    for z in (-800.0, -30.0, -1.5, 0.0, 0.25, 4.0, 40.0, 800.0):
        ref = 1.0 / (1.0 + math.exp(-z)) if z > -700 else 0.0
        assert oracle.sigmoid(z) == pytest.approx(ref, rel=1e-15, abs=1e-300)
    assert oracle.sigmoid(-1e4) == 0.0
    assert oracle.sigmoid(1e4) == 1.0


# --------------------------------------------------------------------------
# saturated gates
# --------------------------------------------------------------------------

@pytest.mark.parametrize("direction", [0, 1])
def test_forget_gate_closed_copies_candidate(direction):
    rng = np.random.default_rng(5)
    L = 9
    uf = np.full(L, -1e4)              # f = 0 exactly in double
    ur = np.full(L, 1e4)               # r = 1 exactly
    ux = rng.standard_normal(L)
    x = rng.standard_normal(L)
    h, c, cl = oracle.chain_forward(uf, ur, ux, x, 0.07, -0.03, 0.1, 0.2, 0.9, 1.7, direction)
    assert np.array_equal(c, ux)                     # c[t] = U[t, 2]
    assert np.array_equal(h, ux)                     # h = c when r = 1
    assert cl == (ux[-1] if direction == 0 else ux[0])
    # r = 0: h = alpha * x
    h2, _, _ = oracle.chain_forward(uf, -ur, ux, x, 0.07, -0.03, 0.1, 0.2, 0.9, 1.7, direction)
    assert np.allclose(h2, 1.7 * x, rtol=0, atol=1e-15)


@pytest.mark.parametrize("direction", [0, 1])
def test_forget_gate_open_keeps_initial_state(direction):
    rng = np.random.default_rng(6)
    L = 7
    uf = np.full(L, 1e4)               # f = 1: c never changes
    ur = np.full(L, 1e4)
    ux = rng.standard_normal(L)
    x = rng.standard_normal(L)
    h, c, cl = oracle.chain_forward(uf, ur, ux, x, 0.05, 0.05, 0.0, 0.0, -0.625, 1.0, direction)
    assert np.all(c == -0.625) and np.all(h == -0.625) and cl == -0.625


# --------------------------------------------------------------------------
# closed forms of the v = 0 recurrence
# --------------------------------------------------------------------------

def test_ema_closed_form_constant_gate():
    rng = np.random.default_rng(7)
    L, a, c0 = 40, 0.8, 1.25
    s = 1.0 / (1.0 + np.exp(-a))
    u = rng.standard_normal(L)
    x = np.zeros(L)
    _, c, _ = oracle.chain_forward(np.full(L, a), np.full(L, 1e4), u, x,
                                   0.0, 0.0, 0.0, 0.0, c0, 1.0)
    t = np.arange(L)
    # c[t] = s^(t+1) c0 + (1 - s) sum_{k<=t} s^(t-k) u[k]
    powers = s ** (t[:, None] - t[None, :]) * (t[:, None] >= t[None, :])
    ref = s ** (t + 1) * c0 + (1 - s) * (powers @ u)
    assert np.max(np.abs(c - ref)) < 1e-14
    # constant candidate: c[t] = u + s^(t+1) (c0 - u)
    _, c2, _ = oracle.chain_forward(np.full(L, a), np.full(L, 1e4), np.full(L, -0.5), x,
                                    0.0, 0.0, 0.0, 0.0, c0, 1.0)
    assert np.max(np.abs(c2 - (-0.5 + s ** (t + 1) * (c0 + 0.5)))) < 1e-14


def test_linear_mode_time_varying_gate_sum_form():
    """v = 0: c[t] = P(0..t) c0 + sum_k P(k+1..t) (1 - a_k) u_k with P a product of gates."""
    rng = np.random.default_rng(8)
    L, c0, alpha = 33, -0.4, 0.6
    uf = rng.standard_normal(L) + 2.0
    ur = rng.standard_normal(L)
    ux = rng.standard_normal(L)
    x = rng.standard_normal(L)
    bf, br = 0.3, -0.2
    h, c, _ = oracle.chain_forward(uf, ur, ux, x, 0.0, 0.0, bf, br, c0, alpha)
    a = 1.0 / (1.0 + np.exp(-(uf + bf)))
    r = 1.0 / (1.0 + np.exp(-(ur + br)))
    ref = np.empty(L)
    for t in range(L):
        total = np.prod(a[: t + 1]) * c0
        for k in range(t + 1):
            total += np.prod(a[k + 1: t + 1]) * (1 - a[k]) * ux[k]
        ref[t] = total
    assert np.max(np.abs(c - ref)) < 1e-13
    assert np.max(np.abs(h - (r * ref + (1 - r) * alpha * x))) < 1e-13


def test_linear_mode_is_the_v0_recurrence_on_finite_input():
    """The linear mode (v None: gates that do not see the state) equals the
    recurrence at v = 0 value for value on finite input, forward and backward."""
    rng = np.random.default_rng(9)
    L, B, d, nd, al = 7, 2, 3, 2, 0.8
    U, x, v, b, c0 = rand_problem(rng, L, B, d, nd)
    z = np.zeros_like(v)
    dh = rng.standard_normal((L, B, nd, d)).astype(np.float32)
    dcl = rng.standard_normal((nd, B, d)).astype(np.float32)
    f0 = oracle.forward(U, x, z, b, c0, al)
    f1 = oracle.forward(U, x, None, b, c0, al)
    for k in f0:
        assert np.array_equal(f0[k], f1[k]), k
    g0 = oracle.backward(U, x, z, b, c0, f0["c"], dh, dcl, al)
    g1 = oracle.backward(U, x, None, b, c0, f1["c"], dh, dcl, al)
    for k in g0:
        assert np.array_equal(g0[k], g1[k]), k


@pytest.mark.parametrize("direction", [0, 1])
def test_linear_mode_gradients_that_do_not_read_the_state(direction):
    """In the linear mode the state adjoint obeys gc[t-1] = f[t] (gc[t] +
    r[t] dh[t]): it, the candidate's gradient dc (1 - f), the highway dx and
    dc0 never read the state.  A NaN initial state (so every state is NaN)
    must leave them exactly as with c0 = 0, while the gate gradients, which
    read the state, turn NaN.  Evaluating v = 0 as a multiplied zero would
    spoil them all through 0 * NaN."""
    rng = np.random.default_rng(10 + direction)
    L, al = 9, 1.1
    uf, ur, ux, x, dh = (rng.standard_normal(L) for _ in range(5))
    bf, br, dcl = 0.2, -0.1, 0.7
    h, c, cl = oracle.chain_forward(uf, ur, ux, x, 0.0, 0.0, bf, br, np.nan, al, direction,
                                    linear=True)
    assert np.isnan(c).all() and np.isnan(h).all() and np.isnan(cl)
    g = oracle.chain_backward(uf, ur, ux, x, 0.0, 0.0, bf, br, np.nan, c, dh, dcl, al,
                              direction, linear=True)
    _, c_ok, _ = oracle.chain_forward(uf, ur, ux, x, 0.0, 0.0, bf, br, 0.0, al, direction,
                                      linear=True)
    g_ok = oracle.chain_backward(uf, ur, ux, x, 0.0, 0.0, bf, br, 0.0, c_ok, dh, dcl, al,
                                 direction, linear=True)
    for k in ("dux", "dx_hw", "dc0"):
        assert np.array_equal(g[k], g_ok[k]) and np.isfinite(g_ok[k]).all(), k
    assert np.isnan(g["duf"]).all() and np.isnan(g["dur"]).all()
    # the general cell at v = 0 carries the NaN state into every gradient
    gv = oracle.chain_backward(uf, ur, ux, x, 0.0, 0.0, bf, br, np.nan, c, dh, dcl, al,
                               direction)
    assert np.isnan(gv["dux"]).any()


# --------------------------------------------------------------------------
# brute force, L <= 4
# --------------------------------------------------------------------------

def _unrolled_L3(uf, ur, ux, x, vf, vr, bf, br, c0, al):
    """Eqs. 2-5 written out for three steps, no loop."""
    f0 = sig(uf[0] + vf * c0 + bf)
    r0 = sig(ur[0] + vr * c0 + br)
    k0 = f0 * c0 + (1 - f0) * ux[0]
    h0 = r0 * k0 + (1 - r0) * al * x[0]
    f1 = sig(uf[1] + vf * k0 + bf)
    r1 = sig(ur[1] + vr * k0 + br)
    k1 = f1 * k0 + (1 - f1) * ux[1]
    h1 = r1 * k1 + (1 - r1) * al * x[1]
    f2 = sig(uf[2] + vf * k1 + bf)
    r2 = sig(ur[2] + vr * k1 + br)
    k2 = f2 * k1 + (1 - f2) * ux[2]
    h2 = r2 * k2 + (1 - r2) * al * x[2]
    return [h0, h1, h2], [k0, k1, k2]


def _unrolled_L4(uf, ur, ux, x, vf, vr, bf, br, c0, al):
    hs, ks = _unrolled_L3(uf, ur, ux, x, vf, vr, bf, br, c0, al)
    k2 = ks[2]
    f3 = sig(uf[3] + vf * k2 + bf)
    r3 = sig(ur[3] + vr * k2 + br)
    k3 = f3 * k2 + (1 - f3) * ux[3]
    h3 = r3 * k3 + (1 - r3) * al * x[3]
    return hs + [h3], ks + [k3]


@pytest.mark.parametrize("L", [1, 2, 3, 4])
@pytest.mark.parametrize("direction", [0, 1])
def test_bruteforce_unrolled(L, direction):
    rng = np.random.default_rng(100 + L + 10 * direction)
    uf, ur, ux, x = (rng.standard_normal(L) for _ in range(4))
    vf, vr, bf, br = rng.uniform(-0.9, 0.9, 4)
    c0, al = 0.7, 1.9
    h, c, cl = oracle.chain_forward(uf, ur, ux, x, vf, vr, bf, br, c0, al, direction)
    order = list(range(L)) if direction == 0 else list(range(L - 1, -1, -1))
    pad = lambda a: np.concatenate([a[order], np.zeros(4 - L)])
    hs, ks = _unrolled_L4(pad(uf), pad(ur), pad(ux), pad(x), vf, vr, bf, br, c0, al)
    for s, t in enumerate(order):
        assert h[t] == pytest.approx(hs[s], rel=1e-15, abs=1e-15)
        assert c[t] == pytest.approx(ks[s], rel=1e-15, abs=1e-15)
    assert cl == pytest.approx(ks[L - 1], rel=1e-15, abs=1e-15)


def test_tensor_routine_layout_matches_chain():
    """The whole-tensor routine places chain (dir, b, j) where the layouts say."""
    rng = np.random.default_rng(9)
    L, B, d, nd = 4, 3, 5, 2
    U, x, v, b, c0 = rand_problem(rng, L, B, d, nd)
    out = oracle.forward(U, x, v, b, c0, 1.1)
    for dl in range(nd):
        for bb in range(B):
            for j in range(d):
                hs, ks = _unrolled_L4(
                    *(a[::-1] if dl else a for a in
                      (U[:, bb, dl, 0, j], U[:, bb, dl, 1, j], U[:, bb, dl, 2, j], x[:, bb, j])),
                    v[dl, 0, j], v[dl, 1, j], b[dl, 0, j], b[dl, 1, j], c0[dl, bb, j], 1.1)
                hs = np.array(hs[::-1] if dl else hs)
                assert np.allclose(out["h"][:, bb, dl, j], hs, rtol=1e-14, atol=1e-14)
                assert out["c_last"][dl, bb, j] == pytest.approx(ks[-1], rel=1e-14)


# --------------------------------------------------------------------------
# gradients by central finite differences
# --------------------------------------------------------------------------

def _loss(U, x, v, b, c0, dh, dcl, al):
    o = oracle.forward(U, x, v, b, c0, al)
    return float(np.sum(o["h"] * dh) + np.sum(o["c_last"] * dcl))


@pytest.mark.parametrize("linear", [False, True])
def test_backward_finite_differences(linear):
    rng = np.random.default_rng(21 if linear else 20)
    L, B, d, nd, al = 6, 2, 3, 2, 1.3
    U, x, v, b, c0 = rand_problem(rng, L, B, d, nd)
    if linear:
        v[:] = 0.0
        U[:, :, :, 0, :] += 2.0
    dh = rng.standard_normal((L, B, nd, d)).astype(np.float32).astype(np.float64)
    dcl = rng.standard_normal((nd, B, d)).astype(np.float32).astype(np.float64)
    fw = oracle.forward(U, x, v, b, c0, al)
    g = oracle.backward(U, x, v, b, c0, fw["c"], dh, dcl, al)
    eps = 1e-6

    def fd(arr, idx, **kw):
        plus = arr.copy(); plus[idx] += eps
        minus = arr.copy(); minus[idx] -= eps
        args = dict(U=U, x=x, v=v, b=b, c0=c0)
        name = kw["name"]
        args[name] = plus
        lp = _loss(args["U"], args["x"], args["v"], args["b"], args["c0"], dh, dcl, al)
        args[name] = minus
        lm = _loss(args["U"], args["x"], args["v"], args["b"], args["c0"], dh, dcl, al)
        return (lp - lm) / (2 * eps)

    # x, v, b, c0 go through float32 inside the whole-tensor routines: perturb with a step
    # that float32 represents and compare at a matching tolerance.
    for idx in np.ndindex(U.shape):
        assert g["dU"][idx] == pytest.approx(fd(U, idx, name="U"), rel=1e-6, abs=1e-8)
    checks = [("x", x, "dx_hw"), ("c0", c0, "dc0"), ("b", b, "db")]
    if not linear:
        checks.append(("v", v, "dv"))
    for name, arr, key in checks:
        for idx in np.ndindex(arr.shape):
            num = _fd32(name, arr, idx, U, x, v, b, c0, dh, dcl, al)
            assert g[key][idx] == pytest.approx(num, rel=2e-3, abs=2e-4), (name, idx)


def _fd32(name, arr, idx, U, x, v, b, c0, dh, dcl, al):
    """Central difference for an input the whole-tensor routine reads as float32."""
    eps = 2.0 ** -10
    args = dict(U=U, x=x, v=v, b=b, c0=c0)
    plus = arr.copy(); plus[idx] += eps
    minus = arr.copy(); minus[idx] -= eps
    args[name] = plus
    lp = _loss(args["U"], args["x"], args["v"], args["b"], args["c0"], dh, dcl, al)
    args[name] = minus
    lm = _loss(args["U"], args["x"], args["v"], args["b"], args["c0"], dh, dcl, al)
    return (lp - lm) / (2 * eps)


def test_chain_backward_finite_differences_double():
    """Per-chain gradients against central differences entirely in double."""
    rng = np.random.default_rng(22)
    L, al = 6, 0.8
    for direction in (0, 1):
        uf, ur, ux, x, dh = (rng.standard_normal(L) for _ in range(5))
        vf, vr, bf, br, c0, dcl = rng.uniform(-0.8, 0.8, 6)
        _, c, _ = oracle.chain_forward(uf, ur, ux, x, vf, vr, bf, br, c0, al, direction)
        g = oracle.chain_backward(uf, ur, ux, x, vf, vr, bf, br, c0, c, dh, dcl, al, direction)

        def loss(uf=uf, ur=ur, ux=ux, x=x, vf=vf, vr=vr, bf=bf, br=br, c0=c0):
            h, _, cl = oracle.chain_forward(uf, ur, ux, x, vf, vr, bf, br, c0, al, direction)
            return float(h @ dh + cl * dcl)

        eps = 1e-6
        for key, name in (("duf", "uf"), ("dur", "ur"), ("dux", "ux"), ("dx_hw", "x")):
            base = dict(uf=uf, ur=ur, ux=ux, x=x)[name]
            for t in range(L):
                p = base.copy(); p[t] += eps
                m = base.copy(); m[t] -= eps
                num = (loss(**{name: p}) - loss(**{name: m})) / (2 * eps)
                assert g[key][t] == pytest.approx(num, rel=1e-6, abs=1e-9)
        for key, name, val in (("dvf", "vf", vf), ("dvr", "vr", vr), ("dbf", "bf", bf),
                               ("dbr", "br", br), ("dc0", "c0", c0)):
            num = (loss(**{name: val + eps}) - loss(**{name: val - eps})) / (2 * eps)
            assert g[key] == pytest.approx(num, rel=1e-6, abs=1e-9)


def test_projection_input_gradient_finite_differences():
    """dX = dU W + dx_hw for the whole layer (U = X W^T, unrounded X)."""
    rng = np.random.default_rng(23)
    L, B, d, nd, al = 4, 2, 3, 2, 0.9
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    W = (rng.standard_normal((nd * 3 * d, d)) * 0.5).astype(np.float32)
    _, _, v, b, c0 = rand_problem(rng, L, B, d, nd)
    dh = rng.standard_normal((L, B, nd, d))
    dcl = np.zeros((nd, B, d))

    def loss(Xv):
        U = oracle.layer_U(Xv, W, False, L, B, nd, d)
        o = oracle.forward(U, Xv, v, b, c0, al)
        return float(np.sum(o["h"] * dh))

    U = oracle.layer_U(X, W, False, L, B, nd, d)
    fw = oracle.forward(U, X, v, b, c0, al)
    g = oracle.backward(U, X, v, b, c0, fw["c"], dh, dcl, al)
    dX = oracle.project_bwd_data(g["dU"].reshape(L * B, nd * 3 * d), W).reshape(L, B, d)
    dX += g["dx_hw"]
    eps = 2.0 ** -10
    for idx in np.ndindex(X.shape):
        p = X.copy(); p[idx] += eps
        m = X.copy(); m[idx] -= eps
        num = (loss(p) - loss(m)) / (2 * eps)
        assert dX[idx] == pytest.approx(num, rel=2e-3, abs=2e-4)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------

def test_bidirectional_is_forward_on_reversed_time():
    rng = np.random.default_rng(30)
    L, B, d = 7, 2, 4
    U, x, v, b, c0 = rand_problem(rng, L, B, d, 2)
    out = oracle.forward(U, x, v, b, c0, 1.4)
    # direction 1 alone, recomputed as a one-direction layer on flipped time
    U1 = U[::-1, :, 1:2].copy()
    ref = oracle.forward(U1, x[::-1].copy(), v[1:2], b[1:2], c0[1:2], 1.4)
    assert np.allclose(out["h"][:, :, 1], ref["h"][::-1, :, 0], rtol=0, atol=1e-15)
    assert np.allclose(out["c_last"][1], ref["c_last"][0], rtol=0, atol=1e-15)
    dh = rng.standard_normal((L, B, 2, d))
    g = oracle.backward(U, x, v, b, c0, out["c"], dh, None, 1.4)
    g1 = oracle.backward(U1, x[::-1].copy(), v[1:2], b[1:2], c0[1:2], ref["c"],
                         dh[::-1, :, 1:2].copy(), None, 1.4)
    assert np.allclose(g["dU"][:, :, 1], g1["dU"][::-1, :, 0], rtol=0, atol=1e-14)
    assert np.allclose(g["dv"][1], g1["dv"][0], rtol=1e-13, atol=1e-14)
    assert np.allclose(g["dc0"][1], g1["dc0"][0], rtol=0, atol=1e-14)


def test_permutation_equivariance():
    rng = np.random.default_rng(31)
    L, B, d, nd = 5, 3, 6, 2
    U, x, v, b, c0 = rand_problem(rng, L, B, d, nd)
    pj = rng.permutation(d)
    pb = rng.permutation(B)
    o = oracle.forward(U, x, v, b, c0, 1.0)
    o2 = oracle.forward(U[:, pb][..., pj], x[:, pb][..., pj], v[..., pj], b[..., pj],
                        c0[:, pb][..., pj], 1.0)
    assert np.array_equal(o2["h"], o["h"][:, pb][..., pj])
    assert np.array_equal(o2["c_last"], o["c_last"][:, pb][..., pj])


# --------------------------------------------------------------------------
# SRU++ attention (the U-producer)
# --------------------------------------------------------------------------

def _attn_inputs(L, B, dp, Lm, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((L, B, dp)), rng.standard_normal((Lm + L, B, dp)),
            rng.standard_normal((Lm + L, B, dp)))


@pytest.mark.parametrize("causal", [False, True])
def test_attention_zero_keys_average_the_visible_values(causal):
    """All scores equal -> uniform weights: A[t] is the mean of the values
    the query may see (all Lm + L, or the first Lm + t + 1 when causal)."""
    L, B, dp, Lm = 6, 3, 5, 2
    Q, K, V = _attn_inputs(L, B, dp, Lm, 30)
    A = oracle.attention(Q, np.zeros_like(K), V, Lm, causal)
    for t in range(L):
        n = Lm + t + 1 if causal else Lm + L
        np.testing.assert_allclose(A[t], V[:n].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_attention_first_causal_query_copies_first_value():
    L, B, dp = 4, 2, 3
    Q, K, V = _attn_inputs(L, B, dp, 0, 31)
    A = oracle.attention(Q, K, V, 0, True)
    np.testing.assert_array_equal(A[0], V[0])


def test_attention_two_keys_closed_form():
    """One query, two keys: weights sigma(s0 - s1) and 1 - sigma(s0 - s1)."""
    q = np.array([[[0.5, -1.0, 2.0, 0.25]]])
    k = np.array([[[1.0, 0.0, 0.5, -2.0]], [[-0.5, 1.5, 0.0, 1.0]]])
    v = np.array([[[2.0, -1.0, 0.0, 3.0]], [[-4.0, 0.5, 1.0, 1.0]]])
    s0, s1 = (q[0, 0] @ k[0, 0]) / 2.0, (q[0, 0] @ k[1, 0]) / 2.0   # sqrt(4) = 2
    w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
    want = w0 * v[0, 0] + (1.0 - w0) * v[1, 0]
    got = oracle.attention(q, k, v, 1, False)          # key 0 is the memory row
    np.testing.assert_allclose(got[0, 0], want, rtol=1e-14, atol=1e-15)
    # causal: the current row (key 1) is the query's own step, so both are seen
    np.testing.assert_allclose(oracle.attention(q, k, v, 1, True)[0, 0], want, rtol=1e-14)


def test_attention_saturated_score_selects_one_value():
    L, B, dp = 3, 1, 4
    Q, K, V = _attn_inputs(L, B, dp, 0, 32)
    K[1, 0] = 200.0 * Q[2, 0]                  # query 2 scores key 1 far above the rest
    A = oracle.attention(Q, K, V, 0, False)
    np.testing.assert_allclose(A[2, 0], V[1, 0], rtol=1e-12, atol=1e-12)


def test_attention_convex_and_key_permutation_invariant():
    L, B, dp, Lm = 5, 2, 6, 3
    Q, K, V = _attn_inputs(L, B, dp, Lm, 33)
    A = oracle.attention(Q, K, V, Lm, False)
    assert np.all(A <= V.max(axis=0)[None] + 1e-12) and np.all(A >= V.min(axis=0)[None] - 1e-12)
    perm = np.random.default_rng(34).permutation(Lm + L)
    np.testing.assert_allclose(oracle.attention(Q, K[perm], V[perm], Lm, False), A,
                               rtol=1e-12, atol=1e-13)
    bperm = np.array([1, 0])
    np.testing.assert_allclose(oracle.attention(Q[:, bperm], K[:, bperm], V[:, bperm], Lm, False),
                               A[:, bperm], rtol=0, atol=0)


def test_attention_rounded_weights_closed_form():
    """Three visible keys with equal scores: each weight 1/3 becomes
    bf16(1/3) = 0.333984375 before the sum."""
    q = np.zeros((1, 1, 2))
    k = np.zeros((3, 1, 2))
    v = np.full((3, 1, 2), 1.5)
    got = oracle.attention(q, k, v, 2, True, round_p=True)
    assert got[0, 0, 0] == 3 * 0.333984375 * 1.5


def test_layernorm_closed_form():
    """[a, b] normalises to [-1, 1] * h / sqrt(h^2 + eps) with h = (b - a) / 2,
    then scale and shift; with unit gain and zero shift every row has mean 0
    and variance var / (var + eps)."""
    eps = 1e-5
    y = oracle.layernorm(np.array([[1.0, 4.0]]), np.array([2.0, 3.0]), np.array([0.5, -1.0]), eps)
    h = 1.5
    n = h / math.sqrt(h * h + eps)
    np.testing.assert_allclose(y[0], [2.0 * -n + 0.5, 3.0 * n - 1.0], rtol=1e-15)
    x = np.random.default_rng(35).standard_normal((4, 9)) * 3 + 1
    z = oracle.layernorm(x, np.ones(9), np.zeros(9), eps)
    np.testing.assert_allclose(z.mean(axis=1), 0.0, atol=1e-14)
    v = x.var(axis=1)
    np.testing.assert_allclose(z.var(axis=1), v / (v + eps), rtol=1e-13)


def test_attention_project_alpha_zero_is_the_factorised_projection():
    """The pages' own special case: with alpha = 0 (its initial value), the
    attention drops out and U = Wo Wq X, the factorised projection."""
    rng = np.random.default_rng(36)
    L, B, d, dp = 4, 3, 8, 4
    X = rng.standard_normal((L * B, d)).astype(np.float32)
    Wq, Wk, Wv = (rng.standard_normal((dp, n)) for n in (d, dp, dp))
    Wo = rng.standard_normal((3 * d, dp))
    for round_ops in (False, True):
        a = oracle.attention_project(X, Wq, Wk, Wv, Wo, L, B, 0.0, round_ops=round_ops)
        f = oracle.factored_project(X, Wq, Wo, round_ops)
        np.testing.assert_array_equal(a["U"], f["U"])
        np.testing.assert_array_equal(a["Q"], f["Q"])


def _uniform_attention_case(seed, L, B, d, dp, Lm):
    """Inputs whose keys are all zero (W_k = 0 and zero context keys), so
    every score is 0 and each query's weights are uniform over the keys it
    may see: the attention is then a plain mean of value rows."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((L * B, d)).astype(np.float32)
    Wq = rng.standard_normal((dp, d))
    Wk = np.zeros((dp, dp))
    Wv = rng.standard_normal((dp, dp))
    Wo = rng.standard_normal((3 * d, dp))
    Kmem = np.zeros((Lm, B, dp))
    Vmem = rng.standard_normal((Lm, B, dp))
    return X, Wq, Wk, Wv, Wo, Kmem, Vmem


def _uniform_attention_by_hand(X, Wq, Wv, Vmem, L, B, Lm, causal):
    """Q = X Wq^T and V = Q Wv^T with numpy; A[t, b] = mean of the visible
    value rows, the context rows first (the previous segment precedes this
    one), so with a causal mask step t sees the Lm context rows and steps
    0..t of its own segment."""
    Q = X.astype(np.float64) @ Wq.T
    V = (Q @ Wv.T).reshape(L, B, -1)
    allv = np.concatenate([Vmem, V])
    A = np.empty_like(V)
    for t in range(L):
        n = Lm + t + 1 if causal else Lm + L
        A[t] = allv[:n].mean(axis=0)
    return Q, V, A.reshape(L * B, -1)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_project_uniform_weights_closed_form(causal):
    """SRU++ section: U = Wo (Q + alpha A) with K = Wk Q and V = Wv Q.  With
    all keys zero, A is a mean of value rows, so the whole composition has a
    closed form at alpha != 0: it fixes the sign of the residual, that V is
    built from Q, and that the context rows come first (causal: a context
    appended after the segment would let step 0 see steps 1.. instead)."""
    L, B, d, dp, Lm, alpha = 3, 2, 6, 4, 2, 0.75
    X, Wq, Wk, Wv, Wo, Kmem, Vmem = _uniform_attention_case(37, L, B, d, dp, Lm)
    a = oracle.attention_project(X, Wq, Wk, Wv, Wo, L, B, alpha, mem_len=Lm, Kmem=Kmem,
                                 Vmem=Vmem, causal=causal)
    Q, V, A = _uniform_attention_by_hand(X, Wq, Wv, Vmem, L, B, Lm, causal)
    R = Q + alpha * A
    np.testing.assert_allclose(a["Q"], Q, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(a["V"][Lm:], V, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(a["V"][:Lm], Vmem)
    np.testing.assert_allclose(a["A"], A, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["R"], R, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["U"], R @ Wo.T, rtol=1e-12, atol=1e-12)


def test_attention_project_layernorm_before_the_output_projection():
    """The layer-norm variant normalises the residual sum Q + alpha A over
    its d' features (biased variance, gain, shift) and only then applies Wo
    (SRU++ section).  Closed form as above; the normalisation by hand with
    numpy's mean and variance."""
    L, B, d, dp, Lm, alpha, eps = 3, 2, 6, 4, 2, -1.25, 1e-5
    X, Wq, Wk, Wv, Wo, Kmem, Vmem = _uniform_attention_case(38, L, B, d, dp, Lm)
    rng = np.random.default_rng(39)
    gamma = rng.uniform(0.5, 1.5, dp)
    beta = rng.uniform(-0.5, 0.5, dp)
    a = oracle.attention_project(X, Wq, Wk, Wv, Wo, L, B, alpha, mem_len=Lm, Kmem=Kmem,
                                 Vmem=Vmem, causal=True, ln=(gamma, beta, eps))
    Q, _, A = _uniform_attention_by_hand(X, Wq, Wv, Vmem, L, B, Lm, True)
    S = Q + alpha * A
    mu = S.mean(axis=1, keepdims=True)
    var = S.var(axis=1, keepdims=True)
    R = (S - mu) / np.sqrt(var + eps) * gamma + beta
    np.testing.assert_allclose(a["R"], R, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(a["U"], R @ Wo.T, rtol=1e-11, atol=1e-11)


def test_attention_project_rounding_points_by_hand():
    """The bf16 path: K and V are products of the rounded Q~, not of Q, and
    the residual adds the unrounded Q.  One step, one key, d = 2, d' = 1:
      Q  = 1 * 1 + 1 * 2^-9 = 1.001953125, Q~ = bf16(Q) = 1 (spacing 2^-7);
      K  = Q~ * 0.5 = 0.5;  V = Q~ * 3 = 3 (3.005859375 from unrounded Q);
      the single visible key has weight 1, so A = bf16(V) = 3;
      R  = Q + 0.5 * A = 2.501953125, R~ = 2.5 (spacing 2^-6);
      U  = R~ * Wo = 2.5 * [1, 2, -1, 0.5, 4, -2]."""
    X = np.array([[1.0, 1.0]], np.float32)
    Wq = np.array([[1.0, 2.0 ** -9]])
    Wk = np.array([[0.5]])
    Wv = np.array([[3.0]])
    Wo = np.array([[1.0], [2.0], [-1.0], [0.5], [4.0], [-2.0]])
    a = oracle.attention_project(X, Wq, Wk, Wv, Wo, 1, 1, 0.5, causal=True, round_ops=True)
    assert a["Q"][0, 0] == 1.001953125
    assert a["K"][0, 0, 0] == 0.5
    assert a["V"][0, 0, 0] == 3.0
    assert a["A"][0, 0] == 3.0
    assert a["R"][0, 0] == 2.501953125
    np.testing.assert_array_equal(a["U"][0], 2.5 * Wo[:, 0])


# --------------------------------------------------------------------------
# decoding step
# --------------------------------------------------------------------------

def test_steps_reproduce_the_sequence_forward():
    """Carrying c through L single steps gives the sequence forward (Eqs. 1-5
    over all L at once) step for step.  The step takes its state as fp32 (as
    stored between calls), so each step starts from the fp64 state rounded to
    fp32: 1e-6 covers that rounding."""
    rng = np.random.default_rng(40)
    L, B, d, alpha = 6, 3, 8, 0.7
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    W = rng.uniform(-0.3, 0.3, (3 * d, d)).astype(np.float32)
    v = rng.uniform(-0.5, 0.5, (2, d)).astype(np.float32)
    b = rng.uniform(-0.5, 0.5, (2, d)).astype(np.float32)
    c0 = rng.standard_normal((B, d)).astype(np.float32)
    U = oracle.project(X.reshape(L * B, d), W, False).reshape(L, B, 1, 3, d)
    fo = oracle.forward(U, X, v.reshape(1, 2, d), b.reshape(1, 2, d), c0.reshape(1, B, d), alpha)
    c = c0.astype(np.float64)
    for t in range(L):
        h, c = oracle.step(X[t], W, v, b, c.astype(np.float32), alpha, False)
        np.testing.assert_allclose(h, fo["h"][t, :, 0], rtol=1e-6, atol=1e-6)
        np.testing.assert_allclose(c, fo["c"][t, :, 0], rtol=1e-6, atol=1e-6)


def test_step_closed_gate_copies_candidate():
    """f = 0 and r = 1 (saturated through b): c_next = u_cand = x W_cand^T and
    h = c_next, whatever the state."""
    rng = np.random.default_rng(41)
    B, d = 2, 4
    x = rng.standard_normal((B, d)).astype(np.float32)
    W = rng.uniform(-0.5, 0.5, (3 * d, d)).astype(np.float32)
    v = np.zeros((2, d), np.float32)
    b = np.stack([np.full(d, -1e4), np.full(d, 1e4)]).astype(np.float32)
    h, c = oracle.step(x, W, v, b, rng.standard_normal((B, d)).astype(np.float32), 1.0, False)
    ucand = x.astype(np.float64) @ W[2 * d:].astype(np.float64).T
    np.testing.assert_allclose(c, ucand, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h, ucand, rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------
# SRU++ attention: backward
# --------------------------------------------------------------------------

def _central_difference(f, arr, h=1e-6):
    """d f / d arr by central differences, element by element (arr is
    perturbed in place and restored)."""
    g = np.empty_like(arr, dtype=np.float64)
    for idx in np.ndindex(arr.shape):
        keep = arr[idx]
        arr[idx] = keep + h
        fp = f()
        arr[idx] = keep - h
        fm = f()
        arr[idx] = keep
        g[idx] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("causal,ln,Lm", [(True, False, 0), (True, True, 2), (False, True, 1),
                                          (False, False, 2)])
def test_attention_backward_finite_differences(causal, ln, Lm):
    """Every gradient of the attention U-producer against central differences
    of the scalar sum(dU * U): X, Wq, Wk, Wv, Wo, alpha and (layer norm on)
    gamma, beta.  The context rows are constants; perturbing them is not a
    parameter of the loss."""
    rng = np.random.default_rng(60 + Lm + 3 * causal + 7 * ln)
    L, B, d, dp = 3, 2, 4, 3
    P = {"X": rng.standard_normal((L * B, d)),
         "Wq": rng.standard_normal((dp, d)) * 0.6,
         "Wk": rng.standard_normal((dp, dp)) * 0.6,
         "Wv": rng.standard_normal((dp, dp)) * 0.6,
         "Wo": rng.standard_normal((3 * d, dp)) * 0.6,
         "alpha": np.array(0.7),
         "gamma": rng.uniform(0.5, 1.5, dp),
         "beta": rng.uniform(-0.5, 0.5, dp)}
    Kmem = rng.standard_normal((Lm, B, dp))
    Vmem = rng.standard_normal((Lm, B, dp))
    dU = rng.standard_normal((L * B, 3 * d))
    eps = 1e-3

    def loss():
        lnp = (P["gamma"], P["beta"], eps) if ln else None
        U = oracle.attention_project(P["X"], P["Wq"], P["Wk"], P["Wv"], P["Wo"], L, B,
                                     float(P["alpha"]), Lm, Kmem, Vmem, causal, lnp)["U"]
        return float(np.sum(dU * U))

    g = oracle.attention_project_backward(P["X"], P["Wq"], P["Wk"], P["Wv"], P["Wo"], L, B,
                                          float(P["alpha"]), dU, Lm, Kmem, Vmem, causal,
                                          (P["gamma"], P["beta"], eps) if ln else None)
    names = ["X", "Wq", "Wk", "Wv", "Wo", "alpha"] + (["gamma", "beta"] if ln else [])
    for n in names:
        num = _central_difference(loss, P[n])
        got = np.asarray(g["d" + n], np.float64)
        scale = max(1.0, float(np.max(np.abs(num))))
        np.testing.assert_allclose(got, num, rtol=1e-6, atol=1e-7 * scale, err_msg=n)


def test_attention_backward_single_key_closed_form():
    """One query that sees one key: A = V, so dV = dA, and the weight is
    constant 1, so no gradient reaches Q or K."""
    rng = np.random.default_rng(70)
    Q, K, V, dA = (rng.standard_normal((1, 2, 3)) for _ in range(4))
    dQ, dK, dV = oracle.attention_backward(Q, K, V, dA, 0, True)
    np.testing.assert_array_equal(dV, dA)
    np.testing.assert_allclose(dQ, 0.0, atol=1e-15)
    np.testing.assert_allclose(dK, 0.0, atol=1e-15)


def test_layernorm_backward_closed_form():
    """d/dx of layernorm with unit gain: the gradient sums to zero over a row
    (shifting a row does not change its normalisation), its projection on xh
    is sum(dy xh) eps / ((var + eps) sqrt(var + eps)) (only eps keeps the
    scale direction alive), and dbeta, dgamma are the column sums of dy and
    dy * xh."""
    rng = np.random.default_rng(71)
    x = rng.standard_normal((5, 7)) * 2 + 1
    dy = rng.standard_normal((5, 7))
    eps = 1e-2
    dx, dg, db = oracle.layernorm_backward(x, np.ones(7), eps, dy)
    var = x.var(1)
    xh = (x - x.mean(1, keepdims=True)) / np.sqrt(var[:, None] + eps)
    np.testing.assert_allclose(dx.sum(1), 0.0, atol=1e-12)
    want = (dy * xh).sum(1) * eps / ((var + eps) * np.sqrt(var + eps))
    np.testing.assert_allclose((dx * xh).sum(1), want, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(db, dy.sum(0), rtol=1e-14)
    np.testing.assert_allclose(dg, (dy * xh).sum(0), rtol=1e-12)
