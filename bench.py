"""Benchmark of the SRU layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-extras] [--workload 2]

One step = one pass of the whole hot path over one batch: projection GEMM
(U = X~ W^T), forward recurrence, backward recurrence with the fused dv/db
reduction (which also writes dU rounded to bf16), and the backward-data GEMM
(W transposed once, then dX = bf16(dU) W + highway dx).  The headline
workload is the bidirectional layer L=64, B=128, d=512 (fp32 activations,
bf16 W).  Inputs are seeded synthetic draws (no dataset), resident in HBM
before the timed region; several input/output sets rotate so consecutive steps
do not reuse cached data.

Printed: one JSON line.  ``value`` is the step's algorithmic HBM bytes (every
tensor of every row counted once at its dtype) divided by the step time, in
GB/s; per-row times (HIP events recorded on the stream the kernels run on),
their roofline fractions, the dominant row's roofline object, the CPU oracle
baseline on a bounded sample, and measurements of the other rows at the other
workload sizes (given-U bf16 forward, the L=512 training step, the linear-mode
chunked scan) are included.  ``beyond_step`` times, after the step and on its
buffers, rows that are not part of the step: the projection's weight gradient
dW = bf16(dU)^T X~, and the factorised projection U = Wo (Wq X~) with d' = d/4
(SRU++ paper, Fig. 2(b)), forward and backward; at the given-U workload, the
SRU++ attention that would produce that U (causal, previous segment as
context, layer norm); for unidirectional layers, 32 consecutive decoding
steps (sru_step) at B = 1 and at the layer's B.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
METRIC = "SRU fwd+bwd recurrence GB/s and L·B·d steps/s; % HBM peak; GEMM % MFMA"
KERNEL_SOURCES = ["gemm.hip", "recurrence.hip", "backward_scan.hip", "linear_scan.hip",
                  "device_common.h", "scan_common.h"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5],
                   help="2, 4: training step; 3: given-U forward; 5: linear mode fwd+bwd")
    p.add_argument("--sets", type=int, default=4, help="rotating input/output sets")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-beyond", action="store_true",
                   help="skip the rows timed beyond the step (counter runs use this, so "
                        "that every dispatch of a kernel belongs to a step row)")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="also run one torch copy of this many MiB (counter calibration)")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, "
                        "then WRITE_SIZE, each with --copy-probe-mib) into profiles/traffic.json")
    return p.parse_args()


def source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "parallelizable_recurrent_units_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# algorithmic work of each row (every tensor counted once at its dtype)
# ---------------------------------------------------------------------------
def row_work(w):
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    LB = L * B
    xs = 2 if w.x_dtype == "bf16" else 4
    us = 2 if w.u_dtype == "bf16" else 4
    n3 = nd * 3 * d
    rows = {}
    if w.mode == "layer":
        rows["a1_projection"] = dict(flops=2 * LB * n3 * d,
                                     bytes=LB * d * xs + n3 * d * 2 + LB * n3 * 4)
        # bf16(dU) x bf16 W, plus the highway dx read and dX written
        rows["a5_projection_bwd_data"] = dict(flops=2 * LB * d * n3,
                                              bytes=LB * n3 * 2 + n3 * d * 2 + 2 * LB * d * 4)
    fwd = LB * n3 * us + LB * d * xs + LB * nd * d * 4 * (2 if w.backward else 1)
    if w.linear:
        rows["a6_linear_forward"] = dict(bytes=fwd)
    else:
        rows["a2_forward"] = dict(bytes=fwd)
    if w.backward:
        bwd = (LB * n3 * us + LB * d * xs + 2 * LB * nd * d * 4 + LB * n3 * 4 + LB * d * 4)
        rows["a7_linear_backward" if w.linear else "a3_a4_backward"] = dict(bytes=bwd)
    return rows


def next_row_work(w):
    """Rows timed beside the step, not part of it: the weight gradient of
    the projection, dW = bf16(dU)^T X~ (dU's bf16 copy and X read once, dW
    written once)."""
    if w.mode != "layer":
        return attention_work(w) if not w.linear else {}
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    LB, n3 = L * B, nd * 3 * d
    xs = 2 if w.x_dtype == "bf16" else 4
    di = factored_inner(w)
    fwd_flops = 2 * LB * d * di + 2 * LB * di * n3
    fwd_bytes = (LB * d * xs + di * d * 2 + LB * di * 4          # Q = X Wq^T
                 + LB * di * 4 + n3 * di * 2 + LB * n3 * 4)     # U = Q Wo^T
    bwd_flops = 4 * LB * n3 * di + 4 * LB * di * d
    bwd_bytes = (LB * n3 * 2 + n3 * di * 2 + LB * di * 4         # dQ = bf16(dU) Wo
                 + LB * di * 4 + di * d * 2 + 2 * LB * d * 4    # dX += dQ Wq
                 + LB * di * 4 + LB * d * xs + di * d * 4       # dWq = dQ^T X
                 + LB * n3 * 2 + LB * di * 4 + n3 * di * 4)     # dWo = bf16(dU)^T Q
    rows = {"f1_projection_bwd_weight": dict(flops=2 * LB * n3 * d,
                                             bytes=LB * n3 * 2 + LB * d * xs + n3 * d * 4),
            "f3_factored_forward": dict(flops=fwd_flops, bytes=fwd_bytes),
            "f3_factored_backward": dict(flops=bwd_flops, bytes=bwd_bytes)}
    if nd == 1:   # decoding steps (unidirectional layers only)
        ws = 2 if w.w_dtype == "bf16" else 4
        for bb in sorted({1, B}):
            rows[f"f4_decode_step_B{bb}"] = dict(
                flops=DECODE_STEPS * 2 * bb * 3 * d * d,
                bytes=DECODE_STEPS * (3 * d * d * ws + 4 * d * 4 + bb * d * (xs + 3 * 4)))
    return rows


DECODE_STEPS = 32   # consecutive single-step calls per timed decode row


ATTN_CONTEXT = 1.0   # previous-segment context length, in units of L


def attention_work(w):
    """The SRU++ attention producing this workload's U: d' = d / 4, causal,
    the previous segment (L steps) as context.  Flops count the visible
    (query, key) pairs only; bytes count X, the weights, Q, the keys and
    values (written once for this segment, read once for all Lm + L steps),
    R and U (bf16, the U the given-U recurrence takes), not the scores the
    kernels keep in a workspace."""
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    dp, Lm, n3, LB = max(1, d // 4), int(ATTN_CONTEXT * L), nd * 3 * d, L * B
    pairs = B * (L * Lm + L * (L + 1) // 2)
    flops = (2 * LB * d * dp + 2 * LB * dp * 2 * dp + 4 * pairs * dp + 2 * LB * dp * n3)
    byts = (LB * d * 4 + (dp * d + 2 * dp * dp + n3 * dp) * 2 + LB * dp * 4
            + LB * 2 * dp * 2 + (Lm + L) * B * 2 * dp * 2 + LB * dp * 4 + LB * n3 * 2)
    return {"f2_attention_forward": dict(flops=flops, bytes=byts)}


def factored_inner(w):
    """Inner dimension of the factorised projection: d / 4, the proportion of
    the SRU++ paper's Fig. 2 (d = 2048, d' = 512)."""
    return max(1, w.d // 4)


def roofline_of(name, work, seconds):
    if "flops" in work:
        t_mfma = work["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        t_hbm = work["bytes"] / (HBM_PEAK_GBS * 1e9)
        if t_mfma >= t_hbm:
            a = work["flops"] / seconds / 1e12
            return dict(bound="mfma", achieved=a, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=a / MFMA_BF16_PEAK_TFLOPS)
    a = work["bytes"] / seconds / 1e9
    return dict(bound="hbm", achieved=a, peak=HBM_PEAK_GBS, unit="GB/s", frac=a / HBM_PEAK_GBS)


# ---------------------------------------------------------------------------
# device buffers for one training-step set
# ---------------------------------------------------------------------------
def device_set(w, seed):
    import numpy as np
    import torch
    from parallelizable_recurrent_units_amd import (SRU_WS_BACKWARD, SRU_WS_BWD_WEIGHT,
                                                    SRU_WS_FACTORED_WEIGHT, SruShape,
                                                    sru_workspace_size)
    from parallelizable_recurrent_units_amd.workloads import make_inputs
    inp = make_inputs(w, seed=seed)
    dev = {}
    for k, v in inp.items():
        if k.endswith("_bits"):
            continue
        if k + "_bits" in inp:
            dev[k] = torch.from_numpy(inp[k + "_bits"].view(np.int16)).cuda().view(torch.bfloat16)
        else:
            dev[k] = torch.from_numpy(v).cuda()
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    f32 = dict(device="cuda", dtype=torch.float32)
    shape = SruShape(L, B, d, nd == 2, w.alpha)
    dev.update(U=torch.empty((L, B, nd, 3, d), **f32), h=torch.empty((L, B, nd, d), **f32),
               c_seq=torch.empty((L, B, nd, d), **f32), c_last=torch.empty((nd, B, d), **f32),
               dU=torch.empty((L, B, nd, 3, d), **f32), dx=torch.empty((L, B, d), **f32),
               dU_lp=torch.empty((L, B, nd, 3, d), device="cuda", dtype=torch.bfloat16),
               dv=torch.empty((nd, 2, d), **f32), db=torch.empty((nd, 2, d), **f32),
               dc0=torch.empty((nd, B, d), **f32),
               Wt=torch.empty((d, nd * 3 * d), device="cuda", dtype=dev["W"].dtype),
               ws=torch.empty(sru_workspace_size(shape, SRU_WS_BACKWARD), device="cuda",
                              dtype=torch.uint8),
               dW=torch.empty((nd * 3 * d, d), **f32))
    nw = sru_workspace_size(shape, SRU_WS_BWD_WEIGHT)
    dev["ws_w"] = torch.empty(nw, device="cuda", dtype=torch.uint8) if nw else None
    # factorised projection (timed beyond the step): weights ~ U(-0.05, 0.05) in bf16
    di = factored_inner(w)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev["Wq"] = ((torch.rand((di, d), generator=g, **f32) - 0.5) * 0.1).to(torch.bfloat16)
    dev["Wo"] = ((torch.rand((nd * 3 * d, di), generator=g, **f32) - 0.5) * 0.1).to(torch.bfloat16)
    dev.update(Q=torch.empty((L * B, di), **f32), dQ=torch.empty((L * B, di), **f32),
               dWq=torch.empty((di, d), **f32), dWo=torch.empty((nd * 3 * d, di), **f32))
    nf = sru_workspace_size(shape, SRU_WS_FACTORED_WEIGHT, di)
    dev["ws_f"] = torch.empty(nf, device="cuda", dtype=torch.uint8) if nf else None
    return shape, dev


def training_step_rows(shape, t):
    """The four row calls of one training step (C-ABI entry points).  The
    projection reads fp32 X and rounds it to bf16 as it stages it: at these
    shapes that is faster than rounding X into a bf16 copy first."""
    from parallelizable_recurrent_units_amd import (SRU_PROJ_BWD_DATA_WT, SRU_PROJ_FWD,
                                                    sru_backward, sru_forward, sru_project,
                                                    sru_transpose_weight)

    def bwd_data():
        sru_transpose_weight(shape, t["W"], t["Wt"])
        sru_project(shape, SRU_PROJ_BWD_DATA_WT, t["dU_lp"], t["Wt"], t["dx"], True)

    return [
        ("a1_projection", lambda: sru_project(shape, SRU_PROJ_FWD, t["x"], t["W"], t["U"])),
        ("a2_forward", lambda: sru_forward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"], t["h"],
                                           t["c_seq"], t["c_last"])),
        ("a3_a4_backward", lambda: sru_backward(shape, t["U"], t["x"], t["v"], t["b"], t["c0"],
                                                t["c_seq"], t["dh"], t["dc_last"], t["dU"],
                                                t["dx"], t["dv"], t["db"], t["dc0"], t["ws"],
                                                t["dU_lp"])),
        ("a5_projection_bwd_data", bwd_data),
    ]


def next_rows(shape, t):
    """The rows beyond the step, run on a step's buffers (dU_lp as the step
    left it): the weight gradient, and the factorised projection's forward
    (writing U) and backward (adding to dx)."""
    from parallelizable_recurrent_units_amd import (SRU_BF16, SRU_FACT_BWD_Q, SRU_FACT_BWD_X,
                                                    SRU_FACT_Q, SRU_FACT_U, SRU_FACT_WGRAD_O,
                                                    SRU_FACT_WGRAD_Q, sru_project_bwd_weight,
                                                    sru_project_factored,
                                                    sru_project_factored_bwd_weight)
    di = t["Q"].shape[1]

    def fact_fwd():
        sru_project_factored(shape, di, SRU_FACT_Q, t["x"], t["Wq"], t["Q"])
        sru_project_factored(shape, di, SRU_FACT_U, t["Q"], t["Wo"], t["U"])

    def fact_bwd():
        sru_project_factored(shape, di, SRU_FACT_BWD_Q, t["dU_lp"], t["Wo"], t["dQ"])
        sru_project_factored(shape, di, SRU_FACT_BWD_X, t["dQ"], t["Wq"], t["dx"], True)
        sru_project_factored_bwd_weight(shape, di, SRU_FACT_WGRAD_Q, t["dQ"], t["x"], t["dWq"],
                                        SRU_BF16, False, t["ws_f"])
        sru_project_factored_bwd_weight(shape, di, SRU_FACT_WGRAD_O, t["dU_lp"], t["Q"],
                                        t["dWo"], SRU_BF16, False, t["ws_f"])

    rows = [("f1_projection_bwd_weight",
             lambda: sru_project_bwd_weight(shape, t["dU_lp"], t["x"], t["dW"], SRU_BF16,
                                            False, t["ws_w"])),
            ("f3_factored_forward", fact_fwd),
            ("f3_factored_backward", fact_bwd)]
    if not shape.bidirectional:
        rows += decode_rows(shape, t)
    return rows


def decode_rows(shape, t):
    """DECODE_STEPS single-step calls (sru_step) with the state carried in
    place, the inputs of step i being row i of the layer's x; at B = 1 and at
    the layer's B.  The steps are captured once in a HIP graph and the row
    replays it (a decoding loop issues its steps that way; launched one by
    one from Python, the host's launch rate would be measured instead)."""
    import torch
    from parallelizable_recurrent_units_amd import SruShape, sru_step
    out = []
    for bb in sorted({1, shape.B}):
        s1 = SruShape(1, bb, shape.d, False, shape.alpha)
        xs = [t["x"][i, :bb] for i in range(DECODE_STEPS)]
        h = torch.empty((bb, shape.d), device="cuda", dtype=torch.float32)
        c = torch.zeros((bb, shape.d), device="cuda", dtype=torch.float32)

        def steps(s1=s1, xs=xs, h=h, c=c):
            for x in xs:
                sru_step(s1, x, t["W"], t["v"], t["b"], c, h, c)

        steps()                                   # once outside capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            steps()
        out.append((f"f4_decode_step_B{bb}", graph.replay))
    return out


def time_rows(row_sets, steps, warmup):
    """Run ``steps`` passes (rotating sets), HIP events between the rows.

    Returns (ms per step, {row: mean seconds})."""
    import torch
    nsets = len(row_sets)
    for i in range(warmup):
        for _, fn in row_sets[i % nsets]:
            fn()
    torch.cuda.synchronize()
    names = [n for n, _ in row_sets[0]]
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        ev = evs[i]
        ev[0].record()
        for k, (_, fn) in enumerate(row_sets[i % nsets]):
            fn()
            ev[k + 1].record()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    per_row = {n: 0.0 for n in names}
    for ev in evs:
        for k, n in enumerate(names):
            per_row[n] += ev[k].elapsed_time(ev[k + 1]) / 1e3 / steps
    return total_ms / steps, per_row


def attention_rows(w, shape, g):
    """The SRU++ attention that would produce this workload's U (one buffer
    set): X ~ N(0, 1), bf16 weights ~ U(-0.05, 0.05), layer norm on, the
    previous segment's keys and values ~ N(0, 1) in front; U written in
    bf16, as the given-U recurrence takes it."""
    import torch
    from parallelizable_recurrent_units_amd import (SruAttnCfg, sru_attention_forward,
                                                    sru_attention_workspace_size)
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    dp, Lm = max(1, d // 4), int(ATTN_CONTEXT * L)
    f32 = dict(device="cuda", dtype=torch.float32)
    wt = lambda r, c: ((torch.rand((r, c), generator=g, **f32) - 0.5) * 0.1).to(torch.bfloat16)
    cfg = SruAttnCfg(dp, Lm, True, True, 1.0, 1e-5)
    X = torch.randn((L * B, d), generator=g, **f32)
    Wq, Wkv, Wo = wt(dp, d), wt(2 * dp, dp), wt(nd * 3 * d, dp)
    gamma, beta = torch.ones(dp, **f32), torch.zeros(dp, **f32)
    KV = torch.randn((Lm + L, B, 2 * dp), generator=g, **f32).to(torch.bfloat16)
    Q, R = torch.empty((L * B, dp), **f32), torch.empty((L * B, dp), **f32)
    U = torch.empty((L, B, nd, 3, d), device="cuda", dtype=torch.bfloat16)
    ws = torch.empty(sru_attention_workspace_size(shape, cfg), device="cuda", dtype=torch.uint8)
    return [("f2_attention_forward",
             lambda: sru_attention_forward(shape, cfg, X, Wq, Wkv, Wo, gamma, beta, Q, KV, R, U,
                                           ws))]


class RowSet(list):
    """One set's step rows [(row, fn)], plus ``beyond``: rows timed after the
    step on the same buffers."""
    beyond = ()


def row_sets_for(w, nsets, seed0):
    """Rotating sets of the rows of workload ``w`` (each set: list of (row, fn))."""
    import torch
    from parallelizable_recurrent_units_amd import (SRU_BWD, SRU_FWD, SRU_WS_LINEAR_BWD,
                                                    SRU_WS_LINEAR_FWD, SruShape, sru_forward,
                                                    sru_linear_scan, sru_workspace_size)
    f32 = dict(device="cuda", dtype=torch.float32)
    if w.mode == "layer":
        out = []
        for i in range(nsets):
            shape, t = device_set(w, seed0 + i)
            out.append(RowSet(training_step_rows(shape, t)))
            out[-1].beyond = next_rows(shape, t)
        return out
    g = torch.Generator(device="cuda")
    g.manual_seed(seed0)
    s = SruShape(w.L, w.B, w.d, w.ndir == 2, w.alpha)
    if not w.linear:
        # given U (bf16), forward only: U ~ N(0,1), x ~ N(0,1), v ~ U(-0.1, 0.1), b = 0
        out = []
        for _ in range(nsets):
            U = torch.randn((w.L, w.B, 1, 3, w.d), generator=g, **f32).to(torch.bfloat16)
            x = torch.randn((w.L, w.B, w.d), generator=g, **f32).to(torch.bfloat16)
            v = (torch.rand((1, 2, w.d), generator=g, **f32) - 0.5) * 0.2
            b = torch.zeros((1, 2, w.d), **f32)
            h = torch.empty((w.L, w.B, 1, w.d), **f32)
            cl = torch.empty((1, w.B, w.d), **f32)
            out.append(RowSet([("a2_forward", (lambda U=U, x=x, v=v, b=b, h=h, cl=cl:
                                               sru_forward(s, U, x, v, b, None, h, None, cl)))]))
        out[0].beyond = attention_rows(w, s, g)
        return out
    # linear mode, chunk 256: U_f ~ N(2,1), U_r, U_x, x, dh ~ N(0,1), b = 0, c0 = 0.
    # One set: a single call's working set (>= 6 GB) is far beyond every cache.
    U = torch.randn((w.L, w.B, 1, 3, w.d), generator=g, **f32)
    U[:, :, :, 0] += 2.0
    x = torch.randn((w.L, w.B, w.d), generator=g, **f32)
    dh = torch.randn((w.L, w.B, 1, w.d), generator=g, **f32)
    b = torch.zeros((1, 2, w.d), **f32)
    h = torch.empty((w.L, w.B, 1, w.d), **f32)
    c_seq = torch.empty_like(h)
    cl = torch.empty((1, w.B, w.d), **f32)
    dU = torch.empty_like(U)
    dx = torch.empty_like(x)
    dbv = torch.empty((1, 2, w.d), **f32)
    dc0 = torch.empty((1, w.B, w.d), **f32)
    wsf = torch.empty(sru_workspace_size(s, SRU_WS_LINEAR_FWD, w.chunk), device="cuda",
                      dtype=torch.uint8)
    wsb = torch.empty(sru_workspace_size(s, SRU_WS_LINEAR_BWD, w.chunk), device="cuda",
                      dtype=torch.uint8)
    return [[("a6_linear_forward", lambda: sru_linear_scan(s, SRU_FWD, w.chunk, U, x, b, None, h=h,
                                                           c_seq=c_seq, c_last=cl, workspace=wsf)),
             ("a7_linear_backward", lambda: sru_linear_scan(s, SRU_BWD, w.chunk, U, x, b, None,
                                                            c_seq=c_seq, dh=dh, dU=dU, dx=dx,
                                                            db=dbv, dc0=dc0, workspace=wsb))]]


def measure(w, nsets, steps, warmup, seed0):
    """(ms per step, {row: measurement}) for workload ``w``."""
    import torch
    sets = row_sets_for(w, nsets, seed0)
    ms, rows = time_rows(sets, steps, warmup)
    work = row_work(w)
    per_row = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    beyond = time_beyond(w, sets, steps, warmup)
    if beyond:
        per_row["beyond_step"] = beyond
    del sets
    torch.cuda.empty_cache()
    return ms, per_row


def time_beyond(w, sets, steps, warmup):
    """{row: measurement} of the rows beyond the step (after the step has run
    on every set, so their inputs hold a step's results)."""
    beyond = [s.beyond for s in sets if getattr(s, "beyond", ())]
    if not beyond:
        return {}
    _, rows = time_rows(beyond, steps, warmup)
    work = next_row_work(w)
    out = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    for n, r in out.items():
        if n.startswith("f4_decode_step_B"):
            bb = int(n[len("f4_decode_step_B"):])
            r["us_per_step"] = r["us"] / DECODE_STEPS
            r["tokens_per_s"] = bb * DECODE_STEPS / rows[n]
    return out


def extras(main_id, steps):
    """Rows at the other workload sizes, each workload timed on its own."""
    from parallelizable_recurrent_units_amd.workloads import WORKLOADS
    out = {}
    for wid in (2, 3, 4, 5):
        if wid == main_id:
            continue
        w = WORKLOADS[wid]
        linear = w.linear
        ms, per_row = measure(w, 1 if linear else 4, max(3, steps // 5) if linear else steps,
                              2 if linear else 3, 40 + 10 * wid)
        out[w.name] = dict(per_row, ms_per_step=ms)
    return out


def cpu_baseline(w, budget_s=10.0):
    """The CPU oracle (as written) on a bounded sample of the same training
    step: batch rows in order, repeating the whole batch if it finishes early,
    until about ``budget_s`` seconds of work."""
    import numpy as np
    import oracle
    from parallelizable_recurrent_units_amd.workloads import make_inputs
    inp = make_inputs(w, seed=2)
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    X2 = inp["x"].reshape(L * B, d)
    t0 = time.perf_counter()
    done = 0
    while True:
        b = done % B
        rows = np.arange(L) * B + b
        U = oracle.project(X2, inp["W"], True, rows=rows).reshape(L, 1, nd, 3, d)
        sl = lambda a: np.ascontiguousarray(a[:, b:b + 1])
        fo = oracle.forward(U, sl(inp["x"]), inp["v"], inp["b"], sl(inp["c0"]), w.alpha)
        bo = oracle.backward(U, sl(inp["x"]), inp["v"], inp["b"], sl(inp["c0"]), fo["c"],
                             sl(inp["dh"]), sl(inp["dc_last"]), w.alpha)
        oracle.project_bwd_data(bo["dU"].reshape(L, -1), inp["W"])
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    secs = time.perf_counter() - t0
    step_bytes = sum(r["bytes"] for r in row_work(w).values())
    frac = done / B
    return {"value": step_bytes * frac / secs / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "elem_steps_per_s": w.elem_steps * frac / secs,
            "sample": f"{done} batch rows ({frac:.2f} passes over the {B} rows) of the same "
                      f"training step (projection, forward, backward, dX) in double precision, "
                      f"{secs:.1f} s; algorithmic bytes scaled by {frac:.4f}"}


# kernel launches of one call of each row (what its event-timed span covers)
ROW_LAUNCHES = {
    "a1_projection": ["gemm_bf16_mfma (A = fp32 X, rounded to bf16 while staged)"],
    "a2_forward": ["fwd_fast (both directions in one grid)"],
    "a3_a4_backward": ["bwd_fast (fp32 inputs, up to 128 steps; both directions in one "
                       "launch when bidirectional and L <= 64, else one per direction, the "
                       "last one first) or scan_clear + bwd_scan per direction",
                       "param_reduce (dv, db)"],
    "a5_projection_bwd_data": ["transpose16 (W -> W^T)",
                               "gemm_lds (bf16 dU copy x bf16 W, operands copied straight into LDS)"],
    "a6_linear_forward": ["scan_clear", "lin_fwd_fused"],
    "a7_linear_backward": ["scan_clear", "lin_bwd_fused", "lin_db_reduce"],
    "f1_projection_bwd_weight": ["gemm_bf16_mfma (A = bf16 dU copy and B = fp32 X, both read "
                                 "along L*B; the reduction split over blocks)",
                                 "split_reduce (partial sums added in split order)"],
    "f3_factored_forward": ["gemm_bf16_mfma (Q = X Wq^T)", "gemm_bf16_mfma (U = Q Wo^T)"],
    "f4_decode_step_B1": [f"step_cell x {DECODE_STEPS} (one call per step, state in place, "
                          "replayed from a HIP graph)"],
    "f2_attention_forward": ["gemm_bf16_mfma (Q = X Wq^T)", "gemm_bf16_mfma ([K|V] = Q Wkv^T, "
                             "bf16 out)", "gemm_bf16_mfma (scores, one batch per sequence)",
                             "attn_softmax", "gemm_bf16_mfma (weights x V, batched)",
                             "attn_residual (R = layernorm(Q + alpha A))",
                             "gemm_bf16_mfma (U = R Wo^T)"],
    "f3_factored_backward": ["gemm_bf16_mfma (dQ = bf16(dU) Wo)", "gemm_bf16_mfma (dx += dQ Wq)",
                             "gemm_bf16_mfma + split_reduce (dWq = dQ^T X)",
                             "gemm_bf16_mfma + split_reduce (dWo = bf16(dU)^T Q)"],
}

# kernels of each training-step row (rocprofv3 kernel names), and the one
# kernel that runs exactly once per call of the row
ROW_KERNELS = {
    "a1_projection": ([r"gemm_bf16_mfma<.*>, float, false, "],
                      r"gemm_bf16_mfma<.*>, float, false, "),
    "a2_forward": ([r"fwd_fast<"], r"fwd_fast<"),
    "a3_a4_backward": ([r"bwd_scan<", r"bwd_fast<", r"scan_clear", r"param_reduce"],
                       r"param_reduce"),
    "a5_projection_bwd_data": ([r"transpose16", r"gemm_lds<.*LdsCfg<128, 128, 4, 2, 4, 1>"],
                               r"transpose16"),
}


def _per_dispatch(run_dir, counter):
    """{dispatch id: (kernel name, counter summed over its hardware instances)}
    from the rocpd database(s) a rocprofv3 --pmc run wrote under ``run_dir``."""
    import glob
    import sqlite3
    files = glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True)
    if not files:
        raise SystemExit(f"no rocpd database under {run_dir}")
    per = {}
    for f in files:
        db = sqlite3.connect(f)
        q = "select dispatch_id, name, counter_value from pmc_events where counter_name = ?"
        for did, name, v in db.execute(q, (counter,)):
            key = (f, did)
            n, acc = per.get(key, (name, 0.0))
            per[key] = (n, acc + float(v))
        db.close()
    return per


def write_traffic(fetch_dir, write_dir, copy_bytes):
    """profiles/traffic.json: HBM bytes per call of each row.  FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) are each scaled by the factor that makes the
    calibration copy (the largest torch copy kernel of the run, which moves
    ``copy_bytes`` in and out) read and write exactly its size."""
    import re
    rows = {}
    factors = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _per_dispatch(run_dir, counter)
        copies = [v for n, v in per.values() if "copyBuffer" in n]
        if not copies:
            raise SystemExit(f"{counter}: no calibration copy kernel under {run_dir}")
        factors[counter] = copy_bytes / (max(copies) * 1024.0)
        for row, (pats, anchor) in ROW_KERNELS.items():
            calls = sum(1 for n, _ in per.values() if re.search(anchor, n))
            if not calls:
                continue
            kib = sum(v for n, v in per.values() if any(re.search(q, n) for q in pats))
            r = rows.setdefault(row, {"calls": calls})
            r[counter.lower() + "_bytes"] = kib * 1024.0 * factors[counter] / calls
    for r in rows.values():
        if "fetch_size_bytes" in r and "write_size_bytes" in r:
            r["bytes"] = r["fetch_size_bytes"] + r["write_size_bytes"]
    rec = {"source_digest": source_digest(), "copy_probe_bytes": copy_bytes,
           "calibration_factors": factors,
           "rows": {k: v["bytes"] for k, v in rows.items() if "bytes" in v},
           "detail": rows}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def copy_ceiling(gib=2, reps=10):
    """HBM bandwidth of a plain device copy (torch copy_, read + write), the
    practical ceiling the recurrence rows are compared with (context only;
    the roofline fractions use the published peak)."""
    import torch
    n = int(gib * (1 << 30)) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    secs = e0.elapsed_time(e1) / 1e3 / reps
    del src, dst
    torch.cuda.empty_cache()
    return {"GB/s": 2 * n * 4 / secs / 1e9, "kind": f"torch device copy of {gib} GiB (read + write)"}


def traffic_for(kernel_row, digest):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != digest:
        return None
    return rec.get("rows", {}).get(kernel_row)


def main():
    args = parse()
    if args.write_traffic:
        if not args.copy_probe_mib:
            raise SystemExit("--write-traffic needs the --copy-probe-mib the runs used")
        write_traffic(*args.write_traffic, copy_bytes=args.copy_probe_mib * (1 << 20))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the "
              "kernels run on one GPU's share of the work and are not sharded (how they "
              "would shard is described in the design notes).", file=sys.stderr)
        sys.exit(2)
    import torch
    import parallelizable_recurrent_units_amd as sru
    from parallelizable_recurrent_units_amd.workloads import WORKLOADS
    sru.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = WORKLOADS[args.workload]
    nsets = 1 if w.linear else args.sets
    print(f"[bench] workload {w.name}: building {nsets} input sets", file=sys.stderr, flush=True)
    row_sets = row_sets_for(w, nsets, 100)
    print("[bench] timing", file=sys.stderr, flush=True)
    ms, rows = time_rows(row_sets, args.steps, args.warmup)
    beyond = {} if args.no_beyond else time_beyond(w, row_sets, args.steps, args.warmup)
    del row_sets
    torch.cuda.empty_cache()
    work = row_work(w)
    per_row = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    dominant = max(rows, key=lambda n: rows[n])
    digest = source_digest()
    roof = dict(roofline_of(dominant, work[dominant], rows[dominant]))
    roof["kernel"] = dominant
    roof["launches_per_call"] = ROW_LAUNCHES.get(dominant)
    roof["traffic"] = traffic_for(dominant, digest)
    step_bytes = sum(r["bytes"] for r in work.values())
    line = {
        "metric": METRIC,
        "value": step_bytes / (ms / 1e3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": "recurrences in fp32; projection GEMMs take bf16 operands on MFMA with "
                      "fp32 accumulation",
        "data": "synthetic (seeded Gaussian/uniform draws of the workload's shapes)",
        "config": {"workload": w.name, "L": w.L, "B": w.B, "d": w.d,
                   "bidirectional": w.ndir == 2, "alpha": w.alpha,
                   "x": w.x_dtype, "W": w.w_dtype, "parallelism": "single GPU"},
        "elem_steps_per_s": w.elem_steps / (ms / 1e3),
        "step_algorithmic_bytes": step_bytes,
        "rows": per_row,
        "beyond_step": beyond,
        "roofline": roof,
        "source_digest": digest,
    }
    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_probe_bytes"] = n * 4
    # the metric's two parts: the recurrence (forward + backward rows) in GB/s
    # and element-steps/s, and the projection GEMMs against their roofline
    rec_rows = [n for n in per_row if n in ("a2_forward", "a3_a4_backward",
                                            "a6_linear_forward", "a7_linear_backward")]
    if rec_rows:
        rb = sum(work[n]["bytes"] for n in rec_rows)
        rt = sum(rows[n] for n in rec_rows)
        line["recurrence_fwd_bwd"] = {"GB/s": rb / rt / 1e9, "frac_of_hbm_peak": rb / rt / 1e9 / HBM_PEAK_GBS,
                                      "elem_steps_per_s": w.elem_steps / rt, "rows": rec_rows}
    # counter runs (--copy-probe-mib) skip the ceiling: its 2 GiB copies would
    # be taken for the calibration copy
    ceil = None if args.copy_probe_mib else copy_ceiling()
    line["copy_ceiling"] = ceil
    for r in per_row.values():
        if ceil and r["unit"] == "GB/s":
            r["frac_of_copy_ceiling"] = r["achieved"] / ceil["GB/s"]
    if not args.no_extras:
        print("[bench] other workloads", file=sys.stderr, flush=True)
        line["other_workloads"] = extras(args.workload, max(10, args.steps // 2))
        for rows_w in line["other_workloads"].values():
            for r in rows_w.values():
                if ceil and isinstance(r, dict) and r.get("unit") == "GB/s":
                    r["frac_of_copy_ceiling"] = r["achieved"] / ceil["GB/s"]
    if not args.no_cpu_baseline and w.mode == "layer":
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
