"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Tolerances (normwise relative error, max|gpu - oracle| / max|oracle|, per
output tensor):
  * 1e-5 for everything computed from fp32 (or exactly-widened bf16) inputs
    by the fp32 recurrence, and for the fp32 projection;
  * 2e-2 for anything downstream of a bf16-input projection when compared
    with the oracle evaluated on the UNROUNDED fp32 input (the bar for
    bf16-input projections);
  * 1e-4 for the same outputs compared with the oracle evaluated on the
    bf16-rounded input the kernel actually multiplies: the only difference
    left is the GEMM's fp32 accumulation (K <= 3072 terms, unit roundoff
    2^-24: K u = 1.8e-4 worst case, ~sqrt(K) u = 3e-6 typical);
  * 1e-2 for dX = dU W against the unrounded oracle at the tight stage: the
    backward-data GEMM rounds dU to bf16 (relative 2^-9 = 2e-3 per element);
    the same for the weight gradient dW = dU^T X at the workload sizes.
  * the weight gradient reduces over K = L*B terms (<= 2048 in the small
    cases here): 1e-4 against the oracle on the same bf16 operands (K u =
    1.2e-4 worst case, sqrt(K) u = 3e-6 typical), 1e-5 with fp32 arithmetic.
Inputs are drawn by the seeded generators in
parallelizable_recurrent_units_amd/workloads.py; no oracle input or expected
value comes from the GPU.
"""
import numpy as np
import pytest

import oracle
from parallelizable_recurrent_units_amd import (SRU_PROJ_BWD_DATA, SRU_PROJ_FWD, SruShape,
                                                layer, sru_project, workloads)
from tests.gpu_util import check, dev_inputs, host

pytestmark = pytest.mark.gpu

TIGHT = 1e-5
BF16_BAR = 2e-2
GEMM_ACC = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    yield
    torch.cuda.synchronize()


def run_fwd_bwd(shape, t, keep=True, with_bwd=True):
    h, c_seq, c_last = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t.get("c0"),
                                     keep_c_seq=keep)
    out = {"h": h, "c_seq": c_seq, "c_last": c_last}
    if with_bwd:
        dU, dx, dv, db, dc0 = layer.backward(shape, t["U"], t["x"], t["v"], t["b"], t.get("c0"),
                                             c_seq, t["dh"], t.get("dc_last"))
        out.update(dU=dU, dx=dx, dv=dv, db=db, dc0=dc0)
    return out


def oracle_fwd_bwd(inp, alpha, with_bwd=True, U=None):
    U = inp["U"] if U is None else U
    fo = oracle.forward(U, inp["x"], inp["v"], inp["b"], inp.get("c0"), alpha)
    if not with_bwd:
        return fo, None
    bo = oracle.backward(U, inp["x"], inp["v"], inp["b"], inp.get("c0"), fo["c"], inp["dh"],
                         inp.get("dc_last"), alpha)
    return fo, bo


# ---------------------------------------------------------------------------
# recurrence on a given U (fp32), small shapes: fast and generic paths, odd L,
# both directions, c0, dc_last, b, alpha all non-trivial
# ---------------------------------------------------------------------------
CASES_F32 = [
    # L, B, d, ndir
    (1, 1, 1, 1),
    (5, 3, 7, 2),
    (2, 2, 64, 2),
    (33, 2, 64, 1),
    (17, 3, 128, 2),
    (40, 1, 192, 1),
    (64, 2, 200, 2),
    (100, 2, 64, 1),
    (300, 1, 128, 2),
    (131, 2, 64, 1),
    # two directions from 65 to 128 fp32 steps: one streaming launch per
    # direction, the second adding its highway dx to the first's
    (65, 3, 64, 2),
    (100, 2, 128, 2),
    (128, 1, 192, 2),
    # the chunked backward scan (fp32 from 129 steps): chunks of 64 with a
    # ragged last chunk, many chunks, both directions
    (129, 2, 64, 2),
    (640, 1, 64, 1),
    (1000, 2, 128, 2),
]


@pytest.mark.parametrize("L,B,d,nd", CASES_F32)
def test_recurrence_fp32_given_u(L, B, d, nd):
    w = workloads.custom(L, B, d, ndir=nd, alpha=1.7, mode="given_u", c0="normal0.1")
    inp = workloads.make_inputs(w, seed=1000 + L + d, dc_last=True, v_scale=0.5, b_scale=0.3)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    print(f"case L={L} B={B} d={d} ndir={nd}", flush=True)
    g = run_fwd_bwd(shape, dev_inputs(inp))
    fo, bo = oracle_fwd_bwd(inp, w.alpha)
    for k in ("h", "c_last"):
        check(k, host(g[k]), fo[k], TIGHT)
    check("c_seq", host(g["c_seq"]), fo["c"], TIGHT)
    check("dU", host(g["dU"]), bo["dU"], TIGHT)
    check("dx", host(g["dx"]), bo["dx_hw"], TIGHT)
    for k in ("dv", "db", "dc0"):
        check(k, host(g[k]), bo[k], TIGHT)


# saturated gates: |U_f|, |U_r| drawn in [20, 120] with random signs, so the
# gates are exactly 0 or 1 in fp32 for most steps and e^(-z) exceeds the fp32
# range for some (the kernels cap the exponent; reading s19).  Forward and
# every backward kernel: streaming (L = 40), chunked scan (L = 300), generic
# (d = 37).
@pytest.mark.parametrize("L,B,d,nd", [(40, 3, 128, 2), (300, 2, 128, 1), (20, 2, 37, 2)])
def test_recurrence_saturated_gates(L, B, d, nd):
    w = workloads.custom(L, B, d, ndir=nd, alpha=1.3, mode="given_u", c0="normal0.1")
    inp = workloads.make_inputs(w, seed=4000 + L + d, dc_last=True, v_scale=0.5, b_scale=0.3)
    rng = np.random.default_rng(4100 + L)
    for gate in (0, 1):
        mag = rng.uniform(20.0, 120.0, inp["U"][:, :, :, gate].shape)
        sign = np.where(rng.random(mag.shape) < 0.5, -1.0, 1.0)
        inp["U"][:, :, :, gate] = (sign * mag).astype(np.float32)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    print(f"case L={L} B={B} d={d} ndir={nd} (saturated gates)", flush=True)
    g = run_fwd_bwd(shape, dev_inputs(inp))
    fo, bo = oracle_fwd_bwd(inp, w.alpha)
    for k in ("h", "c_last"):
        check(k, host(g[k]), fo[k], TIGHT)
    check("c_seq", host(g["c_seq"]), fo["c"], TIGHT)
    check("dU", host(g["dU"]), bo["dU"], TIGHT)
    check("dx", host(g["dx"]), bo["dx_hw"], TIGHT)
    for k in ("dv", "db", "dc0"):
        check(k, host(g[k]), bo[k], TIGHT)
    for k in ("h", "dU", "dx"):
        assert np.isfinite(host(g[k])).all(), k


@pytest.mark.parametrize("L,B,d,nd,xdt", [(37, 2, 128, 1, "bf16"), (8, 3, 64, 2, "bf16"),
                                          (9, 2, 70, 1, "bf16"), (12, 2, 64, 1, "f32"),
                                          (257, 1, 64, 2, "bf16"), (65, 1, 64, 1, "bf16"),
                                          (130, 2, 128, 2, "f32"), (1, 2, 64, 2, "bf16"),
                                          (2, 1, 128, 2, "bf16"), (3, 2, 64, 1, "f32")])
def test_recurrence_bf16_u(L, B, d, nd, xdt):
    """bf16 U (and x): the fast two-steps-per-packet path and the generic one;
    the chunked backward scan down to one step."""
    w = workloads.custom(L, B, d, ndir=nd, alpha=1.3, mode="given_u", u_dtype="bf16",
                         x_dtype=xdt, c0="normal0.1")
    inp = workloads.make_inputs(w, seed=2000 + L, dc_last=True, v_scale=0.4, b_scale=0.2)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    print(f"case L={L} B={B} d={d} ndir={nd} x={xdt}", flush=True)
    g = run_fwd_bwd(shape, dev_inputs(inp))
    fo, bo = oracle_fwd_bwd(inp, w.alpha)
    check("h", host(g["h"]), fo["h"], TIGHT)
    check("c_seq", host(g["c_seq"]), fo["c"], TIGHT)
    check("c_last", host(g["c_last"]), fo["c_last"], TIGHT)
    check("dU", host(g["dU"]), bo["dU"], TIGHT)
    check("dx", host(g["dx"]), bo["dx_hw"], TIGHT)
    check("dv", host(g["dv"]), bo["dv"], TIGHT)


@pytest.mark.parametrize("L,B,d,nd,dt", [(9, 64, 1024, 1, "f32"), (21, 32, 1024, 2, "bf16"),
                                         (3, 64, 1024, 1, "bf16"), (13, 1, 64, 2, "f32"),
                                         (70, 3, 128, 1, "bf16"), (16, 2, 64, 1, "bf16"),
                                         (1, 2, 64, 2, "f32"), (1, 1, 64, 1, "bf16"),
                                         (3, 2, 128, 2, "bf16"), (2, 1, 64, 2, "bf16")])
def test_forward_both_kernels(L, B, d, nd, dt):
    """Forward: one wave per 64 channels (1024+ waves) and the two-wave split
    (fewer), ragged group tails and sequences shorter than a group, down to
    sequences shorter than one packet (fp32 packets hold 2 steps, bf16 4)."""
    w = workloads.custom(L, B, d, ndir=nd, alpha=0.8, mode="given_u", u_dtype=dt, x_dtype=dt,
                         c0="normal0.1", backward=False)
    inp = workloads.make_inputs(w, seed=3000 + L + B, v_scale=0.5, b_scale=0.3)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    print(f"case L={L} B={B} d={d} ndir={nd} {dt}", flush=True)
    t = dev_inputs(inp)
    h, c_seq, c_last = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"],
                                     keep_c_seq=True)
    fo, _ = oracle_fwd_bwd(inp, w.alpha, with_bwd=False)
    check("h", host(h), fo["h"], TIGHT)
    check("c_seq", host(c_seq), fo["c"], TIGHT)
    check("c_last", host(c_last), fo["c_last"], TIGHT)


def test_forward_without_state_outputs():
    """c_seq and c_last may be NULL (inference): h is unchanged."""
    import torch
    w = workloads.custom(21, 2, 128, ndir=2, alpha=1.0, mode="given_u", backward=False,
                         c0="zero")
    inp = workloads.make_inputs(w, seed=5)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, True, 1.0)
    h = torch.empty((w.L, w.B, 2, w.d), device="cuda")
    from parallelizable_recurrent_units_amd import sru_forward
    sru_forward(shape, t["U"], t["x"], t["v"], t["b"], None, h, None, None)
    fo, _ = oracle_fwd_bwd(inp, 1.0, with_bwd=False)
    check("h", host(h), fo["h"], TIGHT)


@pytest.mark.parametrize("L,B,d,nd", [(33, 2, 64, 1), (17, 3, 128, 2), (5, 3, 7, 2),
                                      (200, 2, 64, 2), (150, 1, 128, 1)])
def test_backward_bf16_copy_of_dU(L, B, d, nd):
    """The optional bf16 dU equals dU rounded to nearest even, bit for bit."""
    import torch
    w = workloads.custom(L, B, d, ndir=nd, alpha=1.1, mode="given_u", c0="normal0.1")
    inp = workloads.make_inputs(w, seed=7000 + L, dc_last=True, v_scale=0.5, b_scale=0.3)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    h, c_seq, _ = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], keep_c_seq=True)
    out = layer.backward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], c_seq, t["dh"],
                         t["dc_last"], bf16_copy=True)
    dU, dU_lp = out[0], out[5]
    ref = dU.to(torch.bfloat16)
    assert torch.equal(dU_lp.view(torch.int16), ref.view(torch.int16))
    plain = layer.backward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], c_seq, t["dh"],
                           t["dc_last"])
    for a, b in zip(out[:5], plain):
        assert torch.equal(a, b)


@pytest.mark.parametrize("L", [50, 300])
def test_backward_is_deterministic(L):
    w = workloads.custom(L, 8, 128, ndir=2, alpha=1.0, mode="given_u")
    inp = workloads.make_inputs(w, seed=6)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, True, 1.0)
    a = run_fwd_bwd(shape, t)
    b = run_fwd_bwd(shape, t)
    for k in ("h", "dU", "dx", "dv", "db", "dc0"):
        assert np.array_equal(host(a[k]), host(b[k])), k


@pytest.mark.parametrize("L", [1, 37, 64])
@pytest.mark.parametrize("tiny_dh", [False, True])
def test_two_direction_dx_is_the_sum_of_each_direction(L, tiny_dh):
    """Up to 64 steps both directions run in one launch and add their highway
    dx terms into shared rows.  dx must equal, bit for bit, the fp32 sum of
    what each direction gives on its own (direction 1 as a one-direction
    layer on time-reversed inputs), whichever direction adds first; with
    tiny_dh half of dh is scaled by 2^-130, so many terms and sums are fp32
    denormals, which must be kept."""
    import torch
    B, d, alpha = 4, 128, 1.3
    w = workloads.custom(L, B, d, ndir=2, alpha=alpha, mode="given_u", c0="normal0.1")
    inp = workloads.make_inputs(w, seed=7600 + L, dc_last=True, v_scale=0.5, b_scale=0.3)
    if tiny_dh:
        rng = np.random.default_rng(7700 + L)
        inp["dh"] = np.where(rng.random(inp["dh"].shape) < 0.5,
                             inp["dh"] * np.float32(2.0 ** -130), inp["dh"]).astype(np.float32)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, True, alpha)
    _, c_seq, _ = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], keep_c_seq=True)
    both = layer.backward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], c_seq, t["dh"],
                          t["dc_last"])
    one = SruShape(L, B, d, False, alpha)
    parts = []
    for k in (0, 1):
        def sel(a, time_axis=True):
            a = a.narrow(2 if time_axis else 0, k, 1)
            return (a.flip(0) if (k and time_axis) else a).contiguous()
        x = t["x"].flip(0).contiguous() if k else t["x"]
        out = layer.backward(one, sel(t["U"]), x, sel(t["v"], False), sel(t["b"], False),
                             sel(t["c0"], False), sel(c_seq), sel(t["dh"]),
                             sel(t["dc_last"], False))
        dx = out[1].cpu().numpy()                   # fp32 as computed
        parts.append(dx[::-1] if k else dx)
    torch.cuda.synchronize()
    want = parts[0] + parts[1]                      # numpy fp32: IEEE, denormals kept
    got = both[1].cpu().numpy()
    assert got.dtype == np.float32 and want.dtype == np.float32
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    if tiny_dh:
        assert (np.abs(want[want != 0]) < np.finfo(np.float32).tiny).sum() > 100


# ---------------------------------------------------------------------------
# projection GEMM
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("d,nd,dt", [(64, 1, "bf16"), (100, 2, "bf16"), (512, 2, "bf16"),
                                     (8, 1, "bf16"), (1000, 1, "bf16"), (36, 2, "bf16"),
                                     (100, 1, "f32")])
def test_transpose_weight_exact(d, nd, dt):
    """W^T bit for bit: 16-byte path (partial tiles included) and element path."""
    import torch
    g = torch.Generator().manual_seed(d * 10 + nd)
    W = torch.randn(nd * 3 * d, d, generator=g)
    W = (W.to(torch.bfloat16) if dt == "bf16" else W).cuda()
    shape = SruShape(1, 1, d, nd == 2, 1.0)
    Wt = layer.transpose_weight(shape, W)
    ref = W.t().contiguous()
    view = torch.int16 if dt == "bf16" else torch.int32
    assert torch.equal(Wt.view(view).cpu(), ref.view(view).cpu())


@pytest.mark.parametrize("L,B,d,nd", [(3, 5, 64, 1), (7, 19, 100, 2), (2, 3, 37, 1),
                                      (64, 4, 256, 2), (1, 1, 8, 1)])
def test_projection_bf16(L, B, d, nd):
    import torch
    rng = np.random.default_rng(3000 + d)
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    W_bits, W = workloads.to_bf16(rng.uniform(-0.1, 0.1, (nd * 3 * d, d)).astype(np.float32))
    Xd = torch.from_numpy(X).cuda()
    Wd = torch.from_numpy(W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    shape = SruShape(L, B, d, nd == 2, 1.0)
    print(f"case M={L*B} N={nd*3*d} K={d}", flush=True)
    U = layer.project(shape, Xd, Wd)
    X2 = X.reshape(L * B, d)
    check("U vs rounded-X oracle", host(U).reshape(L * B, -1), oracle.project(X2, W, True),
          GEMM_ACC)
    check("U vs fp32-X oracle", host(U).reshape(L * B, -1), oracle.project(X2, W, False),
          BF16_BAR)
    # bf16 X in HBM takes the same path without the cast
    Xb_bits, Xb = workloads.to_bf16(X)
    Ub = layer.project(shape, torch.from_numpy(Xb_bits.view(np.int16)).cuda().view(torch.bfloat16),
                       Wd)
    check("U (bf16 X)", host(Ub).reshape(L * B, -1), oracle.project(Xb.reshape(L * B, d), W, False),
          GEMM_ACC)
    # backward-data with accumulation: dX = C0 + dU W
    G = rng.standard_normal((L, B, nd, 3, d)).astype(np.float32)
    C0 = rng.standard_normal((L, B, d)).astype(np.float32)
    dX = torch.from_numpy(C0.copy()).cuda()
    layer.project_bwd_data(shape, torch.from_numpy(G).cuda(), Wd, dX, accumulate=True)
    G2 = G.reshape(L * B, -1).astype(np.float64)
    ref = oracle.project_bwd_data(G2, W) + C0.reshape(L * B, d)
    check("dX vs exact", host(dX).reshape(L * B, d), ref, 1e-2)
    Gr = oracle.round_bf16(G).reshape(L * B, -1)
    ref_r = oracle.project_bwd_data(Gr, W) + C0.reshape(L * B, d)
    check("dX vs bf16(dU) oracle", host(dX).reshape(L * B, d), ref_r, GEMM_ACC)
    # the same product through the transposed weights (K-contiguous path)
    Wt = layer.transpose_weight(shape, Wd)
    assert np.array_equal(host(Wt), W.T.astype(np.float64))
    dX2 = torch.from_numpy(C0.copy()).cuda()
    layer.project_bwd_data(shape, torch.from_numpy(G).cuda(), Wd, dX2, accumulate=True, Wt=Wt)
    check("dX (transposed W) vs bf16(dU) oracle", host(dX2).reshape(L * B, d), ref_r, GEMM_ACC)


# fp32 X on the register-staged kernel's large tiles: 256 x 192 where 256 x 256
# would leave the last round part-empty (d = 1024 at M = 8100, d = 512 at
# M = 16200: 512 tiles for 384), 256 x 256 otherwise (d = 960); ragged M;
# sampled rows (the last ragged row tile included), every column.  bf16(X)
# multiplied on the LDS-copy path gives the same bits.
@pytest.mark.parametrize("L,B,d", [(90, 90, 1024), (90, 90, 960), (90, 180, 512)])
def test_projection_fp32_x_large_ragged(L, B, d):
    import torch
    rng = np.random.default_rng(3200 + d)
    M = L * B
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    W_bits, W = workloads.to_bf16(rng.uniform(-0.05, 0.05, (3 * d, d)).astype(np.float32))
    Wd = torch.from_numpy(W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    shape = SruShape(L, B, d, False, 1.0)
    print(f"case M={M} N={3 * d} K={d}", flush=True)
    Xd = torch.from_numpy(X).cuda()
    U = layer.project(shape, Xd, Wd)
    rows = np.unique(np.concatenate([np.arange(M - 140, M), np.arange(0, 16),
                                     rng.integers(0, M, 40)]))
    want = oracle.project(X.reshape(M, d)[rows], W, True)
    check("U (fp32 X; sampled rows)", host(U).reshape(M, -1)[rows], want, GEMM_ACC)
    Ub = layer.project(shape, layer.round_bf16(Xd), Wd)
    torch.cuda.synchronize()
    assert torch.equal(U.view(torch.int32), Ub.view(torch.int32))


# bf16 X on grids of 256 x 256 tiles (operands straight into LDS): ragged M,
# and ragged M and N (sampled rows, the last ragged row tile included, every
# column).  X rounded by sru_round_bf16 and then multiplied gives U bit for
# bit equal to fp32 X rounded while the tiles are staged by the other kernel
# (same bf16 operands, same k order, same MFMA).
@pytest.mark.parametrize("L,B,d", [(100, 80, 1024), (60, 100, 1088)])
def test_projection_bf16_x_large(L, B, d):
    import torch
    rng = np.random.default_rng(3100 + d)
    M = L * B
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    W_bits, W = workloads.to_bf16(rng.uniform(-0.05, 0.05, (3 * d, d)).astype(np.float32))
    Wd = torch.from_numpy(W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    shape = SruShape(L, B, d, False, 1.0)
    print(f"case M={M} N={3 * d} K={d}", flush=True)
    Xd = torch.from_numpy(X).cuda()
    Xb = layer.round_bf16(Xd)
    U = layer.project(shape, Xb, Wd)
    rows = np.unique(np.concatenate([np.arange(M - 120, M), np.arange(0, 16),
                                     rng.integers(0, M, 40)]))
    want = oracle.project(oracle.round_bf16(X.reshape(M, d)), W, False, rows=rows)
    check("U (bf16 X; sampled rows)", host(U).reshape(M, -1)[rows], want, GEMM_ACC)
    U32 = layer.project(shape, Xd, Wd)
    torch.cuda.synchronize()
    assert torch.equal(U.view(torch.int32), U32.view(torch.int32))


# weight gradient dW = dU^T X: (L, B, d, nd) spanning no split (K = L*B not a
# multiple of the 64-deep k-tile, or too short), split reductions on the fast
# path, and a split on the bounds-checked path (d = 37: rows of dW not
# 4-aligned).
WGRAD_CASES = [(3, 5, 64, 1), (7, 19, 100, 2), (2, 3, 37, 1), (1, 1, 8, 1), (64, 4, 256, 2),
               (128, 16, 128, 1), (64, 32, 128, 2), (256, 8, 64, 2), (32, 64, 100, 1),
               (64, 32, 37, 2), (16, 64, 512, 1)]


@pytest.mark.parametrize("L,B,d,nd", WGRAD_CASES)
def test_projection_bwd_weight(L, B, d, nd):
    import torch
    from parallelizable_recurrent_units_amd import SRU_WS_BWD_WEIGHT, sru_workspace_size
    rng = np.random.default_rng(5000 + 7 * d + L)
    M = L * B
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    G = rng.standard_normal((L, B, nd, 3, d)).astype(np.float32)
    C0 = rng.standard_normal((nd * 3 * d, d)).astype(np.float32)
    shape = SruShape(L, B, d, nd == 2, 1.0)
    print(f"case K={M} M={nd*3*d} N={d} ws={sru_workspace_size(shape, SRU_WS_BWD_WEIGHT)}",
          flush=True)
    X2, G2 = X.reshape(M, d), G.reshape(M, -1).astype(np.float64)
    Gb_bits, Gb = workloads.to_bf16(G)
    Xb_bits, Xb = workloads.to_bf16(X)
    Gd, Xd = torch.from_numpy(G).cuda(), torch.from_numpy(X).cuda()
    Gbd = torch.from_numpy(Gb_bits.view(np.int16)).cuda().view(torch.bfloat16)
    Xbd = torch.from_numpy(Xb_bits.view(np.int16)).cuda().view(torch.bfloat16)
    exact = oracle.project_bwd_weight(G2, X2, False)
    rounded = oracle.project_bwd_weight(Gb.reshape(M, -1), X2, True)
    # bf16 MFMA, every operand dtype: the kernel multiplies bf16(dU) and bf16(X)
    for gd, xd, tag in ((Gd, Xd, "f32 dU, f32 X"), (Gbd, Xd, "bf16 dU, f32 X"),
                        (Gd, Xbd, "f32 dU, bf16 X"), (Gbd, Xbd, "bf16 dU, bf16 X")):
        dW = layer.project_bwd_weight(shape, gd, xd)
        check(f"dW ({tag}) vs bf16-operand oracle", host(dW), rounded, GEMM_ACC)
        check(f"dW ({tag}) vs exact oracle", host(dW), exact, BF16_BAR)
    # accumulate onto an existing gradient
    dW = torch.from_numpy(C0.copy()).cuda()
    layer.project_bwd_weight(shape, Gbd, Xd, dW, accumulate=True)
    check("dW (+=) vs bf16-operand oracle", host(dW), rounded + C0, GEMM_ACC)
    # fp32 arithmetic
    dW = layer.project_bwd_weight(shape, Gd, Xd, f32_math=True)
    check("dW (fp32 math) vs exact oracle", host(dW), exact, TIGHT)
    dW = torch.from_numpy(C0.copy()).cuda()
    layer.project_bwd_weight(shape, Gbd, Xbd, dW, accumulate=True, f32_math=True)
    check("dW (fp32 math, bf16 inputs, +=)", host(dW),
          oracle.project_bwd_weight(Gb.reshape(M, -1), Xb.reshape(M, d), False) + C0, TIGHT)


# 256 x 256 tiles: split 16 ways (ragged M = 1800 and N = 300, K = 8192), and
# unsplit (M = 7800, N = 1300, K = 2048).  With bf16 X and M, N multiples of 8
# the product copies both K-major operands into LDS and reads them back
# transposed: split 16 ways (M = 1536, N = 512, K = 8192), 3 ways with ragged
# tiles (M = 3288, N = 1096, K = 2048) and unsplit (M = 6144, N = 2048,
# K = 1024).  Sampled rows of dW (the first and last ragged tiles included)
# against the oracle on the bf16 operands, with and without accumulation;
# the split sums are deterministic.
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("L,B,d,nd", [(128, 64, 300, 2), (64, 32, 1300, 2), (128, 64, 512, 1),
                                      (64, 32, 1096, 1), (32, 32, 2048, 1)])
def test_projection_bwd_weight_large_tiles(L, B, d, nd, xdt):
    import torch
    rng = np.random.default_rng(5500 + d)
    M, n3 = L * B, nd * 3 * d
    shape = SruShape(L, B, d, nd == 2, 1.0)
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    Gb_bits, Gb = workloads.to_bf16(rng.standard_normal((L, B, nd, 3, d)).astype(np.float32))
    Gbd = torch.from_numpy(Gb_bits.view(np.int16)).cuda().view(torch.bfloat16)
    if xdt == "bf16":
        Xb_bits, _ = workloads.to_bf16(X)
        Xd = torch.from_numpy(Xb_bits.view(np.int16)).cuda().view(torch.bfloat16)
    else:
        Xd = torch.from_numpy(X).cuda()
    print(f"case K={M} M={n3} N={d} X {xdt}", flush=True)
    rows = np.unique(np.concatenate([np.arange(0, 8), np.arange(n3 - 40, n3),
                                     rng.integers(0, n3, 24)]))
    G2 = Gb.reshape(M, n3)
    want = oracle.matmul(np.ascontiguousarray(G2[:, rows]), oracle.round_bf16(X.reshape(M, d)),
                         a_km=True)
    dW = layer.project_bwd_weight(shape, Gbd, Xd)
    check(f"dW (bf16 dU, {xdt} X; sampled rows)", host(dW)[rows], want, GEMM_ACC)
    C0 = rng.standard_normal((n3, d)).astype(np.float32)
    dW2 = torch.from_numpy(C0.copy()).cuda()
    layer.project_bwd_weight(shape, Gbd, Xd, dW2, accumulate=True)
    check("dW (+=; sampled rows)", host(dW2)[rows], want + C0[rows], GEMM_ACC)
    dW3 = layer.project_bwd_weight(shape, Gbd, Xd)
    torch.cuda.synchronize()
    assert torch.equal(dW.view(torch.int32), dW3.view(torch.int32))
    if xdt == "f32" and d % 8 == 0 and n3 % 8 == 0:
        # fp32 X is rounded into the workspace and takes the same kernel as a
        # bf16 X of the same values: the same bits
        Xb_bits, _ = workloads.to_bf16(X)
        Xbd = torch.from_numpy(Xb_bits.view(np.int16)).cuda().view(torch.bfloat16)
        dWb = layer.project_bwd_weight(shape, Gbd, Xbd)
        torch.cuda.synchronize()
        assert torch.equal(dW.view(torch.int32), dWb.view(torch.int32))


def test_projection_bwd_weight_is_deterministic():
    """The split reduction adds its partial sums in a fixed order."""
    import torch
    shape = SruShape(128, 16, 128, True, 1.0)
    g = torch.Generator().manual_seed(77)
    dU = torch.randn(128 * 16, 6 * 128, generator=g).cuda()
    X = torch.randn(128 * 16, 128, generator=g).cuda()
    a = layer.project_bwd_weight(shape, dU, X)
    b = layer.project_bwd_weight(shape, dU, X)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# bf16 dU times the transposed bf16 weights: the products whose operands go
# straight to LDS (whole 64-deep k-tiles), at ragged M and N, one k-tile up to
# long reductions, with accumulation; (100, 164, 1024) and (100, 140, 1088)
# take the 256 x 256 tiles, ragged in M and in both M and N, and the last two
# the 256 x 128 three-stage tiles (N = 512, and N = 448 with M ragged)
# (sampled rows, the last ragged tile included).
@pytest.mark.parametrize("L,B,d,nd", [(3, 5, 64, 1), (7, 19, 128, 2), (64, 4, 256, 2),
                                      (33, 3, 64, 1), (1, 1, 64, 1), (40, 50, 512, 2),
                                      (100, 164, 1024, 1), (100, 140, 1088, 1),
                                      (128, 128, 512, 1), (92, 177, 448, 1)])
def test_bwd_data_bf16_dU_transposed_weight(L, B, d, nd):
    import torch
    rng = np.random.default_rng(6000 + d + L)
    M = L * B
    shape = SruShape(L, B, d, nd == 2, 1.0)
    W_bits, W = workloads.to_bf16(rng.uniform(-0.1, 0.1, (nd * 3 * d, d)).astype(np.float32))
    G_bits, G = workloads.to_bf16(rng.standard_normal((L, B, nd, 3, d)).astype(np.float32))
    C0 = rng.standard_normal((L, B, d)).astype(np.float32)
    Wd = torch.from_numpy(W_bits.view(np.int16)).cuda().view(torch.bfloat16)
    Gd = torch.from_numpy(G_bits.view(np.int16)).cuda().view(torch.bfloat16)
    Wt = layer.transpose_weight(shape, Wd)
    dX = torch.from_numpy(C0.copy()).cuda()
    print(f"case M={M} N={d} K={nd * 3 * d}", flush=True)
    layer.project_bwd_data(shape, Gd, Wd, dX, accumulate=True, Wt=Wt)
    G2 = G.reshape(M, -1)
    if M * d * nd * 3 * d <= 1 << 31:
        want = oracle.project_bwd_data(G2, W) + C0.reshape(M, d)
        check("dX (bf16 dU, W^T)", host(dX).reshape(M, d), want, GEMM_ACC)
    else:
        rows = np.unique(np.concatenate([np.arange(M - 130, M), np.arange(0, 40),
                                         rng.integers(0, M, 60)]))
        want = oracle.project_bwd_data(G2, W, rows=rows) + C0.reshape(M, d)[rows]
        check("dX (bf16 dU, W^T; sampled rows)", host(dX).reshape(M, d)[rows], want, GEMM_ACC)
    # the same product without accumulation
    dX1 = layer.project_bwd_data(shape, Gd, Wd, Wt=Wt)
    check("dX == accumulated - C0", host(dX1).reshape(M, d), host(dX).reshape(M, d) - C0.reshape(M, d),
          1e-6)
    # W untransposed ([K, N], read back by transposing LDS reads when d is a
    # multiple of 8): the same bf16 operands in the same k order, so the
    # same bits as the transposed weights
    dX2 = layer.project_bwd_data(shape, Gd, Wd)
    torch.cuda.synchronize()
    if d % 8 == 0:
        assert torch.equal(dX2.view(torch.int32), dX1.view(torch.int32))
    else:
        check("dX (W untransposed)", host(dX2).reshape(M, d), host(dX1).reshape(M, d), 1e-6)


@pytest.mark.parametrize("n", [1, 3, 4, 5, 4096, 12289, 1000003, 40000003])
def test_round_bf16_exact(n):
    """sru_round_bf16 bit for bit against the oracle's rounding (ties, both
    parities of the kept bit, infinities, tiny and huge values, NaN).  The
    sizes cover one whole block step (4096), a ragged last step, and more
    elements than one pass of the capped grid (8192 blocks of 4096)."""
    import torch
    rng = np.random.default_rng(n)
    x = (rng.standard_normal(n) * 10.0 ** rng.integers(-30, 30, n)).astype(np.float32)
    special = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), np.inf, -np.inf,
                        3.3895314e38, 1e-40, 0.0, -0.0], np.float32)
    x[:min(n, special.size)] = special[:min(n, special.size)]
    got = layer.round_bf16(torch.from_numpy(x).cuda())
    want = oracle.round_bf16(x)
    g = got.float().cpu().numpy()
    assert np.array_equal(g.view(np.uint32), want.view(np.uint32))
    if n > 10:
        x[7] = np.nan
        g = layer.round_bf16(torch.from_numpy(x).cuda()).float().cpu().numpy()
        assert np.isnan(g[7])


def test_projection_fp32_config1():
    """Workload 1 (fp32 throughout): projection + forward at the 1e-5 bar."""
    w = workloads.WORKLOADS[1]
    inp = workloads.make_inputs(w, seed=1)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, False, w.alpha)
    U = layer.project(shape, t["x"], t["W"])
    h, _, c_last = layer.forward(shape, U, t["x"], t["v"], t["b"], t["c0"])
    Uo = oracle.layer_U(inp["x"], inp["W"], False, w.L, w.B, w.ndir, w.d)
    fo = oracle.forward(Uo, inp["x"], inp["v"], inp["b"], inp["c0"], w.alpha)
    check("U", host(U), Uo, TIGHT)
    check("h", host(h), fo["h"], TIGHT)
    check("c_last", host(c_last), fo["c_last"], TIGHT)


# ---------------------------------------------------------------------------
# linear mode (v = 0): chunked scan == sequential oracle for every chunk size
# ---------------------------------------------------------------------------
def linear_case(L, B, d, nd, chunk, seed, uf_shift=2.0, dt="f32"):
    w = workloads.custom(L, B, d, ndir=nd, alpha=0.8, mode="given_u", linear=True,
                         uf_shift=uf_shift, c0="normal0.1", u_dtype=dt, x_dtype=dt)
    inp = workloads.make_inputs(w, seed=seed, dc_last=True, b_scale=0.3)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    print(f"case L={L} B={B} d={d} ndir={nd} chunk={chunk} uf_shift={uf_shift}", flush=True)
    h, c_seq, c_last = layer.linear_forward(shape, chunk, t["U"], t["x"], t["b"], t["c0"])
    dU, dx, db, dc0 = layer.linear_backward(shape, chunk, t["U"], t["x"], t["b"], t["c0"], c_seq,
                                            t["dh"], t["dc_last"])
    fo, bo = oracle_fwd_bwd(inp, w.alpha)
    check("h", host(h), fo["h"], TIGHT)
    check("c_seq", host(c_seq), fo["c"], TIGHT)
    check("c_last", host(c_last), fo["c_last"], TIGHT)
    check("dU", host(dU), bo["dU"], TIGHT)
    check("dx", host(dx), bo["dx_hw"], TIGHT)
    check("db", host(db), bo["db"], TIGHT)
    check("dc0", host(dc0), bo["dc0"], TIGHT)


@pytest.mark.parametrize("chunk", [1, 7, 64, 256, 300, 1000])
def test_linear_scan_chunk_sizes(chunk):
    linear_case(300, 2, 64, 1, chunk, seed=4000 + chunk)


def test_linear_scan_bidirectional_ragged():
    linear_case(50, 2, 33, 2, 8, seed=4100)


@pytest.mark.parametrize("L,B,d,nd,dt", [(700, 2, 64, 2, "f32"), (1000, 1, 128, 1, "f32"),
                                         (520, 1, 128, 1, "bf16"), (256, 1, 64, 1, "f32"),
                                         (3, 2, 64, 1, "f32"), (1, 1, 64, 2, "bf16")])
def test_linear_scan_single_pass_chunk256(L, B, d, nd, dt):
    """chunk 256 with d % 64 == 0 takes the single-pass look-back kernels."""
    linear_case(L, B, d, nd, 256, seed=4500 + L, dt=dt)


def test_linear_scan_carry_stress():
    """U_f ~ N(8, 1): the product of forget gates over a chunk of 256 stays
    near 0.9, so the carries between chunks dominate the result."""
    linear_case(1024, 2, 64, 1, 256, seed=4200, uf_shift=8.0)


def test_linear_matches_nonlinear_kernel_at_v0():
    """The linear scan and the sequential kernel agree when v = 0."""
    w = workloads.custom(96, 2, 128, ndir=1, alpha=1.0, mode="given_u", linear=True,
                         uf_shift=2.0, c0="normal0.1")
    inp = workloads.make_inputs(w, seed=4300)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, False, 1.0)
    h1, c1, _ = layer.linear_forward(shape, 16, t["U"], t["x"], t["b"], t["c0"])
    h2, c2, _ = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], keep_c_seq=True)
    check("h", host(h1), host(h2), TIGHT)
    check("c", host(c1), host(c2), TIGHT)
