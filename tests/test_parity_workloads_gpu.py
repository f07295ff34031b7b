"""GPU parity at the five specified workload sizes, in the launch configuration
the benchmark times.

* workload 1 (fp32, L=32 B=4 d=64): every output element (test_parity_gpu).
* workload 2 (bidirectional, L=64 B=128 d=512): every output element of the
  whole training step (projection, forward, backward, dv/db, dX), and 52
  sampled rows of the weight gradient dW.
* workload 3 (given bf16 U, L=1024 B=16 d=2048): 48 sampled chains.
* workload 4 (training step, L=512 B=32 d=1024): every chain of 3 sampled
  batch rows; dv and db of 16 sampled channels against the oracle run on all
  32 batch rows of each, plus size-independent properties for all of dv and
  db; sampled rows of dW (each needs the oracle's dU of every batch row for
  its column).
* workload 5 (linear mode, L=16384 B=4 d=4096, chunk 256): 24 sampled chains;
  db of 16 sampled channels against the oracle on all 4 batch rows, plus
  size-independent properties for all of db.
* beyond 2 GiB per tensor (L=4096 B=16 d=4096, fp32 U of 3.2 GB): the forward
  and backward on their large-tensor paths, 6 sampled chains.
Tolerances are explained in test_parity_gpu.py.
"""
import numpy as np
import pytest

import oracle
from parallelizable_recurrent_units_amd import SruShape, layer, workloads
from tests.gpu_util import check, dev_inputs, host

pytestmark = pytest.mark.gpu

TIGHT = 1e-5
BF16_BAR = 2e-2
GEMM_ACC = 1e-4


def _sum_bound_check(name, gpu, terms_sum, terms_abs_sum, n_terms):
    """|gpu - exact| <= n u sum|terms| (fp32 summation of n terms, u = 2^-24)."""
    bound = n_terms * 2.0 ** -24 * terms_abs_sum + 1e-30
    err = np.abs(gpu - terms_sum)
    worst = float(np.max(err / bound))
    print(f"  {name}: max err / (n u sum|terms|) = {worst:.3f}", flush=True)
    assert worst <= 1.0, name


def training_step(w, t):
    """The step as the benchmark runs it, plus the weight gradient (which the
    benchmark times beside the step)."""
    shape = SruShape(w.L, w.B, w.d, w.ndir == 2, w.alpha)
    U = layer.project(shape, t["x"], t["W"])
    h, c_seq, c_last = layer.forward(shape, U, t["x"], t["v"], t["b"], t["c0"], keep_c_seq=True)
    dU, dx, dv, db, dc0, dU_lp = layer.backward(shape, U, t["x"], t["v"], t["b"], t["c0"], c_seq,
                                                t["dh"], t["dc_last"], bf16_copy=True)
    layer.project_bwd_data(shape, dU_lp, t["W"], dx, accumulate=True)   # W as stored
    dW = layer.project_bwd_weight(shape, dU_lp, t["x"])
    return dict(U=U, h=h, c_seq=c_seq, c_last=c_last, dU=dU, dX=dx, dv=dv, db=db, dc0=dc0,
                dW=dW)


def dw_rows(w, seed, n_random):
    """Rows of dW to sample: the first and last of every gate block, plus random ones."""
    n3 = w.ndir * 3 * w.d
    rng = np.random.default_rng(seed)
    edges = [k * w.d for k in range(w.ndir * 3)] + [k * w.d - 1 for k in range(1, w.ndir * 3 + 1)]
    return np.unique(np.concatenate([edges, rng.integers(0, n3, n_random)]))


def oracle_dU_columns(w, inp, cols, round_x):
    """The oracle's dU [L*B, len(cols)] at columns ``cols`` (index (dir, gate, j)
    of the [ndir, 3, d] slot), every (t, b): one chain per (dir, j, b)."""
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    G = np.empty((L, B, cols.size))
    chains = {}
    for k, n in enumerate(cols):
        dr, rem = divmod(int(n), 3 * d)
        gate, j = divmod(rem, d)
        chains.setdefault((dr, j), []).append((k, gate))
    for (dr, j), ks in chains.items():
        v, bias = inp["v"][dr, :, j], inp["b"][dr, :, j]
        for b in range(B):
            uf, ur, ux = oracle.chain_inputs_from_projection(inp["x"], inp["W"], round_x, L, B, d,
                                                             nd, dr, b, j)
            x = inp["x"][:, b, j]
            c0 = inp["c0"][dr, b, j]
            _, c, _ = oracle.chain_forward(uf, ur, ux, x, v[0], v[1], bias[0], bias[1], c0,
                                           w.alpha, direction=dr)
            gb = oracle.chain_backward(uf, ur, ux, x, v[0], v[1], bias[0], bias[1], c0, c,
                                       inp["dh"][:, b, dr, j], inp["dc_last"][dr, b, j], w.alpha,
                                       direction=dr)
            for k, gate in ks:
                G[:, b, k] = gb[("duf", "dur", "dux")[gate]]
    return G.reshape(L * B, cols.size)


def oracle_rows(w, inp, bs, round_x):
    """Oracle for every chain of batch rows ``bs`` (projection included)."""
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    X2 = inp["x"].reshape(L * B, d)
    res = []
    for b in bs:
        rows = np.arange(L) * B + b
        U = oracle.project(X2, inp["W"], round_x, rows=rows).reshape(L, 1, nd, 3, d)
        sl = lambda a: np.ascontiguousarray(a[:, b:b + 1])
        fo = oracle.forward(U, sl(inp["x"]), inp["v"], inp["b"], sl(inp["c0"]), w.alpha)
        bo = oracle.backward(U, sl(inp["x"]), inp["v"], inp["b"], sl(inp["c0"]), fo["c"],
                             sl(inp["dh"]), sl(inp["dc_last"]), w.alpha)
        dX = oracle.project_bwd_data(bo["dU"].reshape(L, -1), inp["W"]) + bo["dx_hw"][:, 0]
        res.append(dict(U=U[:, 0], h=fo["h"][:, 0], c_last=fo["c_last"][:, 0],
                        dU=bo["dU"][:, 0], dc0=bo["dc0"][:, 0], dX=dX))
    return res


def param_grad_channels(w, seed, n_random):
    """Channels whose dv, db are compared with the oracle: both edges of the
    first and last 64-channel tile, plus random ones."""
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 63, 64, w.d - 1], rng.integers(0, w.d, n_random)]))


def oracle_param_grads(w, U, inp, js, linear=False):
    """The oracle's dv, db [2, len(js)] of direction 0 for channels ``js``:
    every batch row's chain run forward and backward (U [L, B, 3, len(js)]
    holds those channels' gate inputs), its per-chain sums over t added over
    b.  ``linear``: v = 0 (the linear mode has no dv)."""
    dv = np.zeros((2, js.size))
    db = np.zeros((2, js.size))
    for k, j in enumerate(js):
        vf, vr = (0.0, 0.0) if linear else (inp["v"][0, 0, j], inp["v"][0, 1, j])
        bf, br = inp["b"][0, 0, j], inp["b"][0, 1, j]
        for b in range(w.B):
            uf, ur, ux = U[:, b, 0, k], U[:, b, 1, k], U[:, b, 2, k]
            x = inp["x"][:, b, j]
            c0 = float(inp["c0"][0, b, j])
            _, c, _ = oracle.chain_forward(uf, ur, ux, x, vf, vr, bf, br, c0, w.alpha)
            g = oracle.chain_backward(uf, ur, ux, x, vf, vr, bf, br, c0, c, inp["dh"][:, b, 0, j],
                                      float(inp["dc_last"][0, b, j]), w.alpha)
            dv[:, k] += (g["dvf"], g["dvr"])
            db[:, k] += (g["dbf"], g["dbr"])
    return dv, db


def test_workload2_full():
    import torch
    w = workloads.WORKLOADS[2]
    inp = workloads.make_inputs(w, seed=2)
    print(f"workload {w.name}", flush=True)
    g = training_step(w, dev_inputs(inp))
    torch.cuda.synchronize()
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    for round_x, tol, tag in ((True, GEMM_ACC, "bf16-X oracle"), (False, BF16_BAR, "fp32-X oracle")):
        Uo = oracle.layer_U(inp["x"], inp["W"], round_x, L, B, nd, d)
        fo = oracle.forward(Uo, inp["x"], inp["v"], inp["b"], inp["c0"], w.alpha)
        bo = oracle.backward(Uo, inp["x"], inp["v"], inp["b"], inp["c0"], fo["c"], inp["dh"],
                             inp["dc_last"], w.alpha)
        dXo = oracle.project_bwd_data(bo["dU"].reshape(L * B, -1), inp["W"]).reshape(L, B, d)
        dXo += bo["dx_hw"]
        print(f" vs {tag}", flush=True)
        check("U", host(g["U"]), Uo, tol)
        check("h", host(g["h"]), fo["h"], tol)
        check("c_seq", host(g["c_seq"]), fo["c"], tol)
        check("c_last", host(g["c_last"]), fo["c_last"], tol)
        check("dU", host(g["dU"]), bo["dU"], tol)
        check("dv", host(g["dv"]), bo["dv"], tol)
        check("db", host(g["db"]), bo["db"], tol)
        check("dc0", host(g["dc0"]), bo["dc0"], tol)
        check("dX", host(g["dX"]), dXo, max(tol, 1e-2))
        rows = dw_rows(w, 22, 40)
        Gs = np.ascontiguousarray(bo["dU"].reshape(L * B, -1)[:, rows])
        dWo = oracle.project_bwd_weight(Gs, inp["x"].reshape(L * B, d), round_x)
        check(f"dW ({rows.size} sampled rows)", host(g["dW"])[rows], dWo, max(tol, 1e-2))


def test_workload3_sampled_chains():
    import torch
    w = workloads.WORKLOADS[3]
    inp = workloads.make_inputs(w, seed=3)
    print(f"workload {w.name}", flush=True)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, False, w.alpha)
    h, _, c_last = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"])
    rng = np.random.default_rng(33)
    chains = [(0, 0), (w.B - 1, w.d - 1), (0, w.d - 1), (w.B - 1, 0)]
    chains += [(int(b), int(j)) for b, j in zip(rng.integers(0, w.B, 44), rng.integers(0, w.d, 44))]
    bi = torch.tensor([b for b, _ in chains], device="cuda")
    ji = torch.tensor([j for _, j in chains], device="cuda")
    hg = host(h[:, bi, 0, ji])            # [L, n]
    cg = host(c_last[0, bi, ji])
    ho = np.empty_like(hg)
    co = np.empty_like(cg)
    U, x = inp["U"], inp["x"]
    for n, (b, j) in enumerate(chains):
        hh, _, cl = oracle.chain_forward(U[:, b, 0, 0, j], U[:, b, 0, 1, j], U[:, b, 0, 2, j],
                                         x[:, b, j], inp["v"][0, 0, j], inp["v"][0, 1, j],
                                         inp["b"][0, 0, j], inp["b"][0, 1, j], 0.0, w.alpha)
        ho[:, n] = hh
        co[n] = cl
    check("h (48 chains)", hg, ho, TIGHT)
    check("c_last (48 chains)", cg, co, TIGHT)


def test_workload4_sampled_rows_and_properties():
    import torch
    w = workloads.WORKLOADS[4]
    inp = workloads.make_inputs(w, seed=4)
    print(f"workload {w.name}", flush=True)
    g = training_step(w, dev_inputs(inp))
    torch.cuda.synchronize()
    bs = [0, w.B - 1, 13]
    for round_x, tol, tag in ((True, GEMM_ACC, "bf16-X oracle"), (False, BF16_BAR, "fp32-X oracle")):
        print(f" vs {tag}, batch rows {bs}", flush=True)
        for b, o in zip(bs, oracle_rows(w, inp, bs, round_x)):
            check(f"U[b={b}]", host(g["U"][:, b]), o["U"], tol)
            check(f"h[b={b}]", host(g["h"][:, b]), o["h"], tol)
            check(f"c_last[b={b}]", host(g["c_last"][:, b]), o["c_last"], tol)
            check(f"dU[b={b}]", host(g["dU"][:, b]), o["dU"], tol)
            check(f"dc0[b={b}]", host(g["dc0"][:, b]), o["dc0"], tol)
            check(f"dX[b={b}]", host(g["dX"][:, b]), o["dX"], max(tol, 1e-2))
    # dW sums over every (t, b): its sampled rows need the oracle's dU of every
    # batch row for those columns only, i.e. one chain per (b, row) pair
    rows = dw_rows(w, 44, 10)
    X2 = inp["x"].reshape(w.L * w.B, w.d)
    for round_x, tol in ((True, 1e-2), (False, BF16_BAR)):
        Gs = oracle_dU_columns(w, inp, rows, round_x)
        check(f"dW ({rows.size} sampled rows, round_x={round_x})", host(g["dW"])[rows],
              oracle.project_bwd_weight(Gs, X2, round_x), tol)
    # dv, db against the oracle: for sampled channels, every batch row's chain
    # (the chunked backward's per-(chunk, row) partial sums and their fixed-order
    # reduction over all 8 chunks x 32 rows).  Fed the kernel's own U, the
    # recurrence bar applies; fed the oracle's projection from unrounded X,
    # the bf16 bar.
    js = param_grad_channels(w, 45, 12)
    jt = torch.from_numpy(js).cuda()
    Ug = host(g["U"][:, :, 0][..., jt])                  # [L, B, 3, len(js)]
    dvo, dbo = oracle_param_grads(w, Ug, inp, js)
    check(f"dv ({js.size} channels, all {w.B} rows, kernel's U)", host(g["dv"][0][:, jt]), dvo,
          TIGHT)
    check(f"db ({js.size} channels, all {w.B} rows, kernel's U)", host(g["db"][0][:, jt]), dbo,
          TIGHT)
    Uo = np.empty_like(Ug)
    for k, j in enumerate(js):
        for b in range(w.B):
            Uo[:, b, :, k] = np.stack(oracle.chain_inputs_from_projection(
                inp["x"], inp["W"], False, w.L, w.B, w.d, 1, 0, b, int(j)), axis=1)
    dvo, dbo = oracle_param_grads(w, Uo, inp, js)
    check(f"dv ({js.size} channels, fp32-X oracle)", host(g["dv"][0][:, jt]), dvo, BF16_BAR)
    check(f"db ({js.size} channels, fp32-X oracle)", host(g["db"][0][:, jt]), dbo, BF16_BAR)
    # dv, db: exact sums of the per-step terms the kernel produced
    dU = g["dU"].double()
    c_seq = g["c_seq"].double()
    c_prev = torch.cat([torch.from_numpy(inp["c0"]).cuda().double()[None, :, :, :].permute(
        0, 2, 1, 3), c_seq[:-1]], dim=0)           # [L, B, 1, d]
    n = w.L * w.B
    for gate, name in ((0, "f"), (1, "r")):
        dz = dU[:, :, 0, gate, :]
        _sum_bound_check(f"db_{name}", host(g["db"][0, gate]), host(dz.sum((0, 1))),
                         host(dz.abs().sum((0, 1))), n)
        terms = dz * c_prev[:, :, 0, :]
        _sum_bound_check(f"dv_{name}", host(g["dv"][0, gate]), host(terms.sum((0, 1))),
                         host(terms.abs().sum((0, 1))), n)


def test_workload5_linear_sampled_chains():
    import torch
    w = workloads.WORKLOADS[5]
    print(f"workload {w.name} (generating inputs)", flush=True)
    inp = workloads.make_inputs(w, seed=5)
    t = dev_inputs(inp)
    shape = SruShape(w.L, w.B, w.d, False, w.alpha)
    h, c_seq, c_last = layer.linear_forward(shape, w.chunk, t["U"], t["x"], t["b"], t["c0"])
    dU, dx, db, dc0 = layer.linear_backward(shape, w.chunk, t["U"], t["x"], t["b"], t["c0"],
                                            c_seq, t["dh"], t["dc_last"])
    torch.cuda.synchronize()
    print(" GPU done", flush=True)
    rng = np.random.default_rng(55)
    chains = [(0, 0), (w.B - 1, w.d - 1)]
    chains += [(int(b), int(j)) for b, j in zip(rng.integers(0, w.B, 22), rng.integers(0, w.d, 22))]
    U, x, dh = inp["U"], inp["x"], inp["dh"]
    errs = {}
    out = {k: [] for k in ("h", "c", "cl", "dU", "dx", "dc0")}
    ref = {k: [] for k in out}
    for b, j in chains:
        uf, ur, ux = U[:, b, 0, 0, j], U[:, b, 0, 1, j], U[:, b, 0, 2, j]
        bf, br = inp["b"][0, 0, j], inp["b"][0, 1, j]
        hh, cc, cl = oracle.chain_forward(uf, ur, ux, x[:, b, j], 0.0, 0.0, bf, br, 0.0, w.alpha)
        gb = oracle.chain_backward(uf, ur, ux, x[:, b, j], 0.0, 0.0, bf, br, 0.0, cc,
                                   dh[:, b, 0, j], 0.0, w.alpha)
        ref["h"].append(hh)
        ref["c"].append(cc)
        ref["cl"].append([cl])
        ref["dU"].append(np.stack([gb["duf"], gb["dur"], gb["dux"]]))
        ref["dx"].append(gb["dx_hw"])
        ref["dc0"].append([gb["dc0"]])
        out["h"].append(host(h[:, b, 0, j]))
        out["c"].append(host(c_seq[:, b, 0, j]))
        out["cl"].append(host(c_last[0, b, j:j + 1]))
        out["dU"].append(host(dU[:, b, 0, :, j]).T)
        out["dx"].append(host(dx[:, b, j]))
        out["dc0"].append(host(dc0[0, b, j:j + 1]))
    for k in out:
        check(f"{k} (24 chains)", np.array(out[k]), np.array(ref[k]), TIGHT, errs)
    # db against the oracle for sampled channels over all 4 batch rows (the
    # fused backward's per-(chunk, chain) partials over 64 chunks, then
    # lin_db_reduce)
    js = param_grad_channels(w, 56, 12)
    _, dbo = oracle_param_grads(w, U[:, :, 0][..., js], inp, js, linear=True)
    check(f"db ({js.size} channels, all {w.B} rows)", host(db[0][:, torch.from_numpy(js).cuda()]),
          dbo, TIGHT)
    n = w.L * w.B
    for gate, name in ((0, "f"), (1, "r")):
        dz = dU[:, :, 0, gate, :].double()
        _sum_bound_check(f"db_{name}", host(db[0, gate]), host(dz.sum((0, 1))),
                         host(dz.abs().sum((0, 1))), n)


def test_recurrence_beyond_2gib_sampled_chains():
    """fp32 U of 3.2 GB (every fast-path tensor limit is 2 GiB): the forward
    takes the generic kernel, the backward the segmented chunked scan.
    Inputs are drawn on the device from a seeded generator; the sampled
    chains' inputs are copied to the host for the oracle, which runs its own
    forward for the states its backward needs."""
    import torch
    L, B, d, alpha = 4096, 16, 4096, 1.0
    gen = torch.Generator(device="cuda").manual_seed(2024)
    f32 = dict(device="cuda", dtype=torch.float32)
    U = torch.randn((L, B, 1, 3, d), generator=gen, **f32)
    x = torch.randn((L, B, d), generator=gen, **f32)
    v = (torch.rand((1, 2, d), generator=gen, **f32) - 0.5) * 0.2
    b = (torch.rand((1, 2, d), generator=gen, **f32) - 0.5) * 0.2
    c0 = 0.1 * torch.randn((1, B, d), generator=gen, **f32)
    dh = torch.randn((L, B, 1, d), generator=gen, **f32)
    assert U.numel() * 4 > 2 ** 31
    shape = SruShape(L, B, d, False, alpha)
    print(f"L={L} B={B} d={d}: U {U.numel() * 4 / 2 ** 30:.2f} GiB", flush=True)
    h, c_seq, c_last = layer.forward(shape, U, x, v, b, c0, keep_c_seq=True)
    dU, dx, _, _, dc0 = layer.backward(shape, U, x, v, b, c0, c_seq, dh)
    torch.cuda.synchronize()
    chains = [(0, 0), (B - 1, d - 1), (5, 1234), (11, 3000), (2, 4095), (15, 64)]
    vh, bh = host(v)[0], host(b)[0]
    for bb, j in chains:
        u = host(U[:, bb, 0, :, j])                      # [L, 3]
        xs, dhs = host(x[:, bb, j]), host(dh[:, bb, 0, j])
        cz = float(host(c0[0, bb, j]))
        hh, cc, cl = oracle.chain_forward(u[:, 0], u[:, 1], u[:, 2], xs, vh[0, j], vh[1, j],
                                          bh[0, j], bh[1, j], cz, alpha)
        g = oracle.chain_backward(u[:, 0], u[:, 1], u[:, 2], xs, vh[0, j], vh[1, j], bh[0, j],
                                  bh[1, j], cz, cc, dhs, 0.0, alpha)
        tag = f"chain (b={bb}, j={j})"
        check(f"h {tag}", host(h[:, bb, 0, j]), hh, TIGHT)
        check(f"c_last {tag}", host(c_last[0, bb, j]), cl, TIGHT)
        check(f"dU {tag}", host(dU[:, bb, 0, :, j]), np.stack([g["duf"], g["dur"], g["dux"]], 1),
              TIGHT)
        check(f"dx {tag}", host(dx[:, bb, j]), g["dx_hw"], TIGHT)
        check(f"dc0 {tag}", host(dc0[0, bb, j]), g["dc0"], TIGHT)
