"""HIP graph capture of the hot path.

The training step (projection, forward, the chunked-scan backward with its
bf16 dU copy, backward-data) and the linear scan's forward and backward are
captured once in a HIP graph and replayed three times, with eager work and
synchronisation between the replays.  Every replay must give the eager
results bit for bit.  The chunked scans keep tickets and published states in
their workspace; each call clears them with a kernel of its own (no memset),
so a replayed graph starts every call from a clean workspace.
"""
import numpy as np
import pytest

from parallelizable_recurrent_units_amd import SruShape, layer, workloads
from tests.gpu_util import dev_inputs, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    yield
    torch.cuda.synchronize()


def replay_matches_eager(run, n_replays=3):
    """Run eagerly, capture, then replay n times; every output tensor of every
    replay equals the eager one bit for bit."""
    import torch
    eager = [host(t) for t in run()]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = run()
    for rep in range(n_replays):
        for t in outs:
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, (t, e) in enumerate(zip(outs, eager)):
            g = host(t)
            assert g.shape == e.shape and np.array_equal(g, e), (rep, k)
    return len(outs)


def test_training_step_graph_replay():
    """L = 300 fp32 with d = 128: the backward runs as the chunked scan."""
    import torch
    L, B, d = 300, 8, 128
    w = workloads.custom(L, B, d, ndir=2, mode="layer")
    t = dev_inputs(workloads.make_inputs(w, 5))
    shape = SruShape(L, B, d, True, 1.0)
    Wt = layer.transpose_weight(shape, t["W"])
    torch.cuda.synchronize()

    def run():
        U = layer.project(shape, t["x"], t["W"])
        h, c_seq, c_last = layer.forward(shape, U, t["x"], t["v"], t["b"], t["c0"],
                                         keep_c_seq=True)
        dU, dx, dv, db, dc0, dU_lp = layer.backward(shape, U, t["x"], t["v"], t["b"], t["c0"],
                                                    c_seq, t["dh"], t["dc_last"], bf16_copy=True)
        layer.project_bwd_data(shape, dU_lp, t["W"], dx, accumulate=True, Wt=Wt)
        return [U, h, c_seq, c_last, dU, dx, dv, db, dc0, dU_lp]

    print("training step L=300 B=8 d=128 bidirectional", flush=True)
    assert replay_matches_eager(run) == 10


def test_linear_scan_graph_replay():
    """Linear mode, chunk 256 over 1000 steps (a ragged last chunk)."""
    import torch
    L, B, d, chunk = 1000, 2, 128, 256
    w = workloads.custom(L, B, d, ndir=1, mode="given_u", linear=True, chunk=chunk,
                         uf_shift=2.0)
    t = dev_inputs(workloads.make_inputs(w, 6))
    shape = SruShape(L, B, d, False, 1.0)
    torch.cuda.synchronize()

    def run():
        h, c_seq, c_last = layer.linear_forward(shape, chunk, t["U"], t["x"], t["b"], t["c0"])
        dU, dx, db, dc0 = layer.linear_backward(shape, chunk, t["U"], t["x"], t["b"], t["c0"],
                                                c_seq, t["dh"], t["dc_last"])
        return [h, c_seq, c_last, dU, dx, db, dc0]

    print("linear scan L=1000 B=2 d=128 chunk 256", flush=True)
    assert replay_matches_eager(run) == 7
