"""GPU parity of the decoding step (sru_step: Eq. 1 and Eqs. 2-5 for one
time step, state carried between calls) against the CPU oracle.

Tolerances (normwise): fp32 W, and bf16 W against the oracle on the same
bf16-rounded x, differ only by the order of the fp32 sums over d products:
about sqrt(d) 2^-24 relative to a gate input, so 4 sqrt(d) 2^-24 (at least
1e-5) for one step; a chain of steps carries it in the state, so twice that.
bf16 W against the oracle on unrounded x: the 2e-2 bar.
"""
import math

import numpy as np
import pytest

import oracle
from parallelizable_recurrent_units_amd import SruShape, layer, workloads
from tests.gpu_util import check, host

pytestmark = pytest.mark.gpu

BF16_BAR = 2e-2


def acc_tol(d):
    return max(1e-5, 4 * math.sqrt(d) * 2.0 ** -24)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU parity tests need a GPU"
    yield
    torch.cuda.synchronize()


def dev(a, bits=None):
    import torch
    if bits is not None:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def params(d, seed, w_dtype):
    rng = np.random.default_rng(seed)
    bound = math.sqrt(6.0 / (4 * d))
    W = rng.uniform(-bound, bound, (3 * d, d)).astype(np.float32)
    v = rng.uniform(-0.1, 0.1, (2, d)).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, (2, d)).astype(np.float32)
    if w_dtype == "bf16":
        bits, W = workloads.to_bf16(W)
        return W, dev(W, bits), v, b
    return W, dev(W), v, b


# (B, d): every kernel variant: d <= 512, 1024, 2048 with the W rows in
# registers, 4096 streamed, d not a multiple of 8 (element path), B up to 100
CASES = [(1, 64), (3, 100), (4, 512), (2, 1024), (5, 2048), (1, 4096), (64, 256), (7, 37),
         # bf16 W from 8 rows on, d % 32 == 0, d <= 2048: the MFMA kernels.
         # 16 x 16 blocks (reduction in 1, 2 or 4 parts; whole and ragged
         # 16-row batch groups, d from 96 to 2048), and 32 x 32 blocks on
         # batches that fill the chip with them (4 and 2 parts, ragged)
         (8, 96), (32, 1024), (33, 512), (16, 2048), (100, 128), (20, 320),
         (512, 256), (700, 96)]


@pytest.mark.parametrize("B,d", CASES)
@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
def test_step(B, d, w_dtype):
    import torch
    rng = np.random.default_rng(B * 1000 + d)
    W, Wd, v, b = params(d, d + B, w_dtype)
    x = rng.standard_normal((B, d)).astype(np.float32)
    c = (0.5 * rng.standard_normal((B, d))).astype(np.float32)
    shape = SruShape(1, B, d, False, 0.8)
    print(f"case B={B} d={d} W={w_dtype}", flush=True)
    rounded = w_dtype == "bf16"
    for x_dtype in ("f32", "bf16"):
        xv = x
        xd = dev(x)
        if x_dtype == "bf16":
            bits, xv = workloads.to_bf16(x)
            xd = dev(xv, bits)
        for state in ("given", "zero"):
            cd = dev(c) if state == "given" else None
            h, cn = layer.step(shape, xd, Wd, dev(v), dev(b), cd)
            h_o, c_o = oracle.step(xv, W, v, b, c if state == "given" else None, 0.8, rounded)
            check(f"h ({x_dtype} x, {state} state)", host(h), h_o, acc_tol(d))
            check(f"c_next ({x_dtype} x, {state} state)", host(cn), c_o, acc_tol(d))
            if rounded:
                h_e, _ = oracle.step(xv, W, v, b, c if state == "given" else None, 0.8, False)
                check("h vs unrounded x", host(h), h_e, BF16_BAR)
    torch.cuda.synchronize()


@pytest.mark.parametrize("B", [3, 20])
@pytest.mark.parametrize("w_dtype", ["bf16", "f32"])
def test_steps_follow_the_sequence(w_dtype, B):
    """40 steps, state updated in place, against the oracle's sequence forward
    (U from the projection oracle on the same x, rounded as the kernel does);
    B = 20 with bf16 W takes the matrix-core kernel."""
    L, d, alpha = 40, 256, 1.0
    W, Wd, v, b = params(d, 77, w_dtype)
    rng = np.random.default_rng(78)
    X = rng.standard_normal((L, B, d)).astype(np.float32)
    c0 = (0.1 * rng.standard_normal((B, d))).astype(np.float32)
    shape = SruShape(1, B, d, False, alpha)
    c = dev(c0.copy())
    hs = []
    for t in range(L):
        h, c = layer.step(shape, dev(X[t]), Wd, dev(v), dev(b), c)
        hs.append(host(h))
    U = oracle.project(X.reshape(L * B, d), W, w_dtype == "bf16").reshape(L, B, 1, 3, d)
    fo = oracle.forward(U, X, v.reshape(1, 2, d), b.reshape(1, 2, d), c0.reshape(1, B, d), alpha)
    check("h over 40 steps", np.stack(hs), fo["h"][:, :, 0], 2 * acc_tol(d))
    check("final state", host(c), fo["c_last"][0], 2 * acc_tol(d))


def test_steps_replayed_from_a_graph():
    """Eight steps captured in a HIP graph: every replay (with eager work and
    synchronisation between replays) gives the eager results bit for bit."""
    import torch
    B, d = 4, 512
    W, Wd, v, b = params(d, 91, "bf16")
    rng = np.random.default_rng(92)
    X = dev(rng.standard_normal((8, B, d)).astype(np.float32))
    c0 = dev((0.1 * rng.standard_normal((B, d))).astype(np.float32))
    vd, bd = dev(v), dev(b)
    shape = SruShape(1, B, d, False, 1.0)
    c = c0.clone()
    hs = [torch.empty((B, d), device="cuda") for _ in range(8)]

    def steps():
        for i in range(8):
            layer.step(shape, X[i], Wd, vd, bd, c, h=hs[i])

    steps()
    torch.cuda.synchronize()
    eager = [host(h) for h in hs] + [host(c)]
    graph = torch.cuda.CUDAGraph()
    c.copy_(c0)
    with torch.cuda.graph(graph):
        steps()
    for rep in range(3):
        c.copy_(c0)
        for h in hs:
            h.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(h) for h in hs] + [host(c)]
        for k, (g, e) in enumerate(zip(got, eager)):
            assert np.array_equal(g, e), (rep, k)
