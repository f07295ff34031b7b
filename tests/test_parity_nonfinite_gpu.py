"""GPU parity of the recurrence on non-finite input: NaN entries in U, x, dh
and c0 propagate as IEEE arithmetic propagates them in the oracle.

The gates are sigma(z) of Eqs. 2-3 of Lei, "When Attention Meets Fast
Recurrence" (SRU background section), and sigma(NaN) is NaN; every later
state of a chain whose forget gate, candidate or state is NaN is NaN, a NaN
reset gate or x spoils that step's h, and the backward carries a NaN state
adjoint to every earlier step.  The kernels cap the gate's exponent with a
NaN-propagating minimum, so they must put NaN in exactly the oracle's places:
the test compares the NaN masks of every output exactly and the finite
entries to the fp32 bar (1e-5, normwise).

In the linear mode the gates do not see the state, so the state adjoint,
the candidate's gradient, the highway dx and dc0 never read a NaN state: the
oracle's linear mode forms no v * c terms (v = 0 is structural, not a
multiplied zero), and the linear scans leave those gradients finite exactly
where it does.

Each case poisons one (batch row, direction, channel) chain per input kind
at a step inside the sequence, each kind on its own chain, so that a kernel
that drops or invents a NaN shows up in the mask of that chain.  Every
backward kernel is covered: the two-direction streaming kernel (L <= 64),
the chunked scan (L > 128, fp32), the generic kernel (odd d), the bf16
paths, and the linear mode's single-pass and three-phase scans.
"""
import numpy as np
import pytest

import oracle
from parallelizable_recurrent_units_amd import SruShape, layer, workloads
from tests.gpu_util import dev_inputs, host

pytestmark = pytest.mark.gpu

TIGHT = 1e-5
BF16_NAN = np.uint16(0x7FC0)


def poison(inp, nd, seed, linear=False):
    """Put one NaN per input kind on a chain of its own; returns the list of
    (kind, t, b, dir, j)."""
    L, B, _, _, d = inp["U"].shape
    rng = np.random.default_rng(seed)
    kinds = ["U_f", "U_r", "U_cand", "x", "dh", "c0"]
    chains = rng.choice(B * nd * d, size=len(kinds), replace=False)
    out = []
    for kind, ch in zip(kinds, chains):
        b, rest = divmod(int(ch), nd * d)
        dr, j = divmod(rest, d)
        t = int(rng.integers(L // 3, L - L // 3)) if L > 2 else 0
        if kind.startswith("U_"):
            g = ("U_f", "U_r", "U_cand").index(kind)
            inp["U"][t, b, dr, g, j] = np.nan
            if "U_bits" in inp:
                inp["U_bits"][t, b, dr, g, j] = BF16_NAN
        elif kind == "x":
            inp["x"][t, b, j] = np.nan
            if "x_bits" in inp:
                inp["x_bits"][t, b, j] = BF16_NAN
        elif kind == "dh":
            inp["dh"][t, b, dr, j] = np.nan
        else:
            inp["c0"][dr, b, j] = np.nan
        out.append((kind, t, b, dr, j))
    return out


def compare(name, gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    gm, rm = np.isnan(gpu), np.isnan(ref)
    bad = np.argwhere(gm != rm)
    assert bad.size == 0, (f"{name}: NaN masks differ at {len(bad)} places, first "
                           f"{bad[:5].tolist()} (gpu NaN {gm.sum()}, oracle NaN {rm.sum()})")
    fin = ~rm
    assert np.isfinite(gpu[fin]).all(), f"{name}: non-finite where the oracle is finite"
    scale = np.max(np.abs(ref[fin])) if fin.any() else 0.0
    err = np.max(np.abs(gpu[fin] - ref[fin])) if fin.any() else 0.0
    e = err / scale if scale > 0 else err
    print(f"  {name}: {int(rm.sum())} NaN (masks equal), finite normwise err {e:.3e}",
          flush=True)
    assert e <= TIGHT, f"{name}: {e} > {TIGHT}"
    return int(rm.sum())


def oracle_fwd_bwd(inp, alpha, linear=False):
    v = None if linear else inp["v"]
    fo = oracle.forward(inp["U"], inp["x"], v, inp["b"], inp["c0"], alpha)
    bo = oracle.backward(inp["U"], inp["x"], v, inp["b"], inp["c0"], fo["c"],
                         inp["dh"], inp["dc_last"], alpha)
    return fo, bo


# (L, B, d, ndir, dtype): streaming two-direction backward, chunked scan
# (fp32 from 129 steps, one and two directions), generic (d = 37), bf16
# packets (fast and generic), the two-wave forward split
CASES = [(40, 3, 128, 2, "f32"), (300, 2, 128, 1, "f32"), (200, 2, 64, 2, "f32"),
         (20, 2, 37, 2, "f32"), (37, 2, 128, 1, "bf16"), (9, 3, 70, 2, "bf16"),
         (21, 32, 1024, 2, "bf16")]


@pytest.mark.parametrize("L,B,d,nd,dt", CASES)
def test_nan_propagates_as_in_the_oracle(L, B, d, nd, dt):
    w = workloads.custom(L, B, d, ndir=nd, alpha=1.3, mode="given_u", u_dtype=dt, x_dtype=dt,
                         c0="normal0.1")
    inp = workloads.make_inputs(w, seed=6000 + L + d, dc_last=True, v_scale=0.5, b_scale=0.3)
    sites = poison(inp, nd, seed=6100 + L)
    print(f"case L={L} B={B} d={d} ndir={nd} {dt} NaN at {sites}", flush=True)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    h, c_seq, c_last = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"],
                                     keep_c_seq=True)
    dU, dx, dv, db, dc0 = layer.backward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], c_seq,
                                         t["dh"], t["dc_last"])
    fo, bo = oracle_fwd_bwd(inp, w.alpha)
    n = compare("h", host(h), fo["h"])
    assert n > 0
    compare("c_seq", host(c_seq), fo["c"])
    compare("c_last", host(c_last), fo["c_last"])
    assert compare("dU", host(dU), bo["dU"]) > 0
    compare("dx", host(dx), bo["dx_hw"])
    compare("dv", host(dv), bo["dv"])
    compare("db", host(db), bo["db"])
    compare("dc0", host(dc0), bo["dc0"])


@pytest.mark.parametrize("L,B,d,nd,chunk,dt", [(700, 2, 64, 2, 256, "f32"),
                                               (300, 2, 64, 1, 64, "f32"),
                                               (520, 1, 128, 1, 256, "bf16")])
def test_nan_propagates_in_the_linear_scan(L, B, d, nd, chunk, dt):
    w = workloads.custom(L, B, d, ndir=nd, alpha=0.8, mode="given_u", linear=True,
                         uf_shift=2.0, c0="normal0.1", u_dtype=dt, x_dtype=dt)
    inp = workloads.make_inputs(w, seed=6500 + L, dc_last=True, b_scale=0.3)
    sites = poison(inp, nd, seed=6600 + L)
    print(f"case linear L={L} B={B} d={d} ndir={nd} chunk={chunk} {dt} NaN at {sites}",
          flush=True)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    h, c_seq, c_last = layer.linear_forward(shape, chunk, t["U"], t["x"], t["b"], t["c0"])
    dU, dx, db, dc0 = layer.linear_backward(shape, chunk, t["U"], t["x"], t["b"], t["c0"], c_seq,
                                            t["dh"], t["dc_last"])
    fo, bo = oracle_fwd_bwd(inp, w.alpha, linear=True)
    assert compare("h", host(h), fo["h"]) > 0
    compare("c_seq", host(c_seq), fo["c"])
    compare("c_last", host(c_last), fo["c_last"])
    assert compare("dU", host(dU), bo["dU"]) > 0
    compare("dx", host(dx), bo["dx_hw"])
    compare("db", host(db), bo["db"])
    compare("dc0", host(dc0), bo["dc0"])
