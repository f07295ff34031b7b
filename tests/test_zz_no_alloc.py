"""sru_backward_static (the backward with the library's static scratch, for
callers that cannot allocate) against sru_backward with a caller workspace:
the same kernels in the same order, so every output must be the same bits.
Two calls in a row on the one static array, the second on a smaller input
(and another kernel path), each compared with its own workspace call."""
import numpy as np
import pytest

from parallelizable_recurrent_units_amd import SruShape, _binding as Bd, layer, workloads
from tests.gpu_util import dev_inputs

pytestmark = pytest.mark.gpu


def _case(L, B, d, ndir, seed, u_dtype="f32"):
    w = workloads.custom(L=L, B=B, d=d, ndir=ndir, alpha=0.8, mode="given_u", u_dtype=u_dtype,
                         x_dtype=u_dtype)
    inp = workloads.make_inputs(w, seed=seed, dc_last=True, b_scale=0.2)
    t = dev_inputs(inp)
    shape = SruShape(L, B, d, ndir == 2, w.alpha)
    _, c_seq, _ = layer.forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], keep_c_seq=True)
    return shape, t, c_seq


def _outputs(shape, U):
    import torch
    s = shape
    f32 = dict(device="cuda", dtype=torch.float32)
    return dict(dU=torch.full((s.L, s.B, s.ndir, 3, s.d), float("nan"), **f32),
                dU_lp=torch.zeros((s.L, s.B, s.ndir, 3, s.d), device="cuda", dtype=torch.bfloat16),
                dx=torch.full((s.L, s.B, s.d), float("nan"), **f32),
                dv=torch.full((s.ndir, 2, s.d), float("nan"), **f32),
                db=torch.full((s.ndir, 2, s.d), float("nan"), **f32),
                dc0=torch.full((s.ndir, s.B, s.d), float("nan"), **f32))


def _run(shape, t, c_seq, static, err=None):
    o = _outputs(shape, t["U"])
    args = (shape, t["U"], t["x"], t["v"], t["b"], t["c0"], c_seq, t["dh"], t["dc_last"],
            o["dU"], o["dx"], o["dv"], o["db"], o["dc0"])
    if static:
        Bd.sru_backward_static(*args, dU_lp=o["dU_lp"], error_word=err)
    else:
        ws = layer.workspace(shape, Bd.SRU_WS_BACKWARD)
        Bd.sru_backward(*args, ws, dU_lp=o["dU_lp"])
        o["ws"] = ws
    return o


def _same_bits(a, b, name):
    import torch
    assert a.shape == b.shape
    va = a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32)
    vb = b.view(torch.int16 if b.dtype == torch.bfloat16 else torch.int32)
    n = int((va != vb).sum())
    print(f"  {name}: {n} differing elements of {a.numel()}", flush=True)
    assert n == 0, name


def test_static_scratch_backward_matches_the_workspace_call_twice():
    import torch
    err = torch.full((1,), 7, device="cuda", dtype=torch.int32)   # must be cleared by the call
    # first: a long sequence (the chunked scan with look-back, 5 chunks);
    # second: smaller, two directions, short (the streaming two-direction kernel)
    for (L, B, d, ndir, seed) in ((300, 4, 256, 1, 81), (40, 3, 128, 2, 82)):
        shape, t, c_seq = _case(L, B, d, ndir, seed)
        need = Bd.sru_workspace_size(shape, Bd.SRU_WS_BACKWARD)
        print(f"case L={L} B={B} d={d} ndir={ndir}: scratch {need} bytes", flush=True)
        assert need <= Bd.SRU_BACKWARD_STATIC_SCRATCH_BYTES
        ref = _run(shape, t, c_seq, static=False)
        got = _run(shape, t, c_seq, static=True, err=err)
        torch.cuda.synchronize()
        assert Bd.workspace_error_word(ref["ws"]) == 0
        assert int(err.item()) == 0
        for k in ("dU", "dU_lp", "dx", "dv", "db", "dc0"):
            _same_bits(got[k], ref[k], k)
