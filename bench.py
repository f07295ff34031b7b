"""Benchmark of the SRU layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-extras] [--workload 4]

One step = one pass of the whole hot path over one batch: projection GEMM
(U = X~ W^T), forward recurrence, backward recurrence with the fused dv/db
reduction (which also writes dU rounded to bf16), and the backward-data GEMM
(W transposed once, then dX = bf16(dU) W + highway dx).  The headline
workload is the full layer training step L=512, B=32, d=1024 (fp32
activations, bf16 W), the largest configuration that carries every part of
the metric.  Inputs are seeded synthetic draws (no dataset), resident in HBM
before the timed region; several input/output sets rotate so consecutive
steps do not reuse cached data.

Printed: one JSON line.  ``value`` is the metric's first part, the forward +
backward recurrence's algorithmic HBM bytes (every tensor of the two rows
counted once at its dtype) divided by the two rows' event-timed time, in
GB/s; ``elem_steps_per_s`` is L*B*d*ndir over the same time; the projection
GEMMs' fraction of the bf16 MFMA peak is ``gemm_frac_of_mfma_peak``.  Also:
per-row times (HIP events recorded on the stream the kernels run on), their
roofline fractions, the dominant row's roofline object, the CPU oracle
baseline on a bounded sample (single-threaded and on every core), and
measurements at the other workload sizes (the bidirectional L=64 step, the
given-U bf16 forward, the linear-mode chunked scan).  ``beyond_step`` times,
after the step and on its buffers, rows that are not part of the step: the
projection's weight gradient dW = bf16(dU)^T X~, and the factorised
projection U = Wo (Wq X~) with d' = d/4 (SRU++ paper, Fig. 2(b)), forward and
backward; at the given-U workload, the SRU++ attention that would produce
that U (causal, previous segment as context, layer norm); for
unidirectional layers, 32 consecutive decoding steps (sru_step) at B = 1 and
at the layer's B.  After every timed region the error word of each scan
workspace is read; a set word aborts the run before anything is printed.
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
    p.add_argument("--workload", type=int, default=4, choices=[2, 3, 4, 5],
                   help="2, 4: training step; 3: given-U forward; 5: linear mode fwd+bwd")
    p.add_argument("--sets", type=int, default=4, help="rotating input/output sets")
    p.add_argument("--x-copy", choices=sorted(X_ROUNDED_COPY), default="auto",
                   help="projection of fp32 X: round X into a bf16 copy first (on), round it "
                        "while staging (off), or by size (auto)")
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
def row_work(w, x_copy=False):
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    LB = L * B
    xs = 2 if w.x_dtype == "bf16" else 4
    us = 2 if w.u_dtype == "bf16" else 4
    n3 = nd * 3 * d
    rows = {}
    if w.mode == "layer":
        if x_copy:   # X~ = bf16(X) made first (its own row), the GEMM reads X~
            rows["a1_round_x"] = dict(bytes=LB * d * (xs + 2))
        rows["a1_projection"] = dict(flops=2 * LB * n3 * d,
                                     bytes=LB * d * (2 if x_copy else xs) + n3 * d * 2 + LB * n3 * 4)
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
        if w.mode == "layer":
            bwd += LB * n3 * 2       # the bf16 copy of dU the backward-data GEMM reads
        rows["a7_linear_backward" if w.linear else "a3_a4_backward"] = dict(bytes=bwd)
    return rows


GEMM_ROWS = ("a1_projection", "a5_projection_bwd_data")
RECURRENCE_ROWS = ("a2_forward", "a3_a4_backward", "a6_linear_forward", "a7_linear_backward")


def next_row_work(w, x_copy=False):
    """Rows timed beside the step, not part of it: the weight gradient of
    the projection, dW = bf16(dU)^T X~ (dU's bf16 copy and X read once, dW
    written once)."""
    if w.mode != "layer":
        return attention_work(w) if not w.linear else {}
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    LB, n3 = L * B, nd * 3 * d
    xs = 2 if (w.x_dtype == "bf16" or x_copy) else 4   # X~ when the step made it
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
    # backward: the forward's three attention products again (recomputed),
    # then dR = dU Wo, dWo = dU^T R, dP = dO V^T, dQ += dS' K, dK = dS'^T Q,
    # dV = P^T dO (visible pairs), dWkv = dKV^T Q, dQ += dKV Wkv, dWq = dQ^T X,
    # dX = dQ Wq; bytes: X, the weights, Q, KV, R, dU (bf16) and dX read or
    # written once, the weight gradients written once
    seg = B * (L * (L + 1) // 2)                                # pairs within the segment
    bflops = (4 * pairs * dp                                   # S and A recomputed
              + 4 * LB * n3 * dp                               # dR, dWo
              + 4 * pairs * dp + 4 * seg * dp                  # dP, dQ; dK, dV (segment keys)
              + 8 * LB * dp * dp                               # dWkv, dQ += dKV Wkv
              + 4 * LB * dp * d)                               # dWq, dX
    bbytes = (LB * d * 4 + (dp * d + 2 * dp * dp + n3 * dp) * 2 + 2 * LB * dp * 4
              + (Lm + L) * B * 2 * dp * 2 + LB * n3 * 2 + LB * d * 4
              + (dp * d + 2 * dp * dp + n3 * dp) * 4)
    return {"f2_attention_forward": dict(flops=flops, bytes=byts),
            "f2_attention_backward": dict(flops=bflops, bytes=bbytes)}


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
def device_set(w, seed, x_copy=False):
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
               ws=torch.empty(sru_workspace_size(shape, SRU_WS_BACKWARD), device="cuda",
                              dtype=torch.uint8),
               dW=torch.empty((nd * 3 * d, d), **f32))
    dev["xb"] = torch.empty((L, B, d), device="cuda", dtype=torch.bfloat16) if x_copy else None
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


X_ROUNDED_COPY = {"auto": None, "on": True, "off": False}


def rounds_x_first(w, mode):
    """Whether the step's projection first rounds X into a bf16 copy X~
    (sru_round_bf16) and multiplies that, rather than rounding fp32 X as it
    stages it.  The copy halves the operand bytes the GEMM streams per k-tile
    (the stream the projection is bound by) for one extra pass over X; it
    pays once the GEMM is long (the L = 512, B = 32, d = 1024 step), and the
    weight gradient then reads X~ as well."""
    if X_ROUNDED_COPY[mode] is not None:
        return X_ROUNDED_COPY[mode]
    return w.x_dtype == "f32" and w.L * w.B * w.d >= (1 << 24)


def training_step_rows(shape, t):
    """The row calls of one training step (C-ABI entry points).  With
    t["xb"] present a row of its own rounds X into that bf16 copy and the
    projection multiplies the copy; otherwise the projection reads fp32 X and
    rounds it to bf16 as it stages it."""
    from parallelizable_recurrent_units_amd import (SRU_PROJ_BWD_DATA, SRU_PROJ_FWD,
                                                    sru_backward, sru_forward, sru_project,
                                                    sru_round_bf16)

    def bwd_data():
        # W as stored ([ndir 3d, d], K-major for this product): the kernel reads
        # it back transposed from LDS, so no W^T pass is needed
        sru_project(shape, SRU_PROJ_BWD_DATA, t["dU_lp"], t["W"], t["dx"], True)

    xb = t.get("xb")
    first = [("a1_round_x", lambda: sru_round_bf16(t["x"], xb))] if xb is not None else []
    return first + [
        ("a1_projection", lambda: sru_project(shape, SRU_PROJ_FWD, t["x"] if xb is None else xb,
                                              t["W"], t["U"])),
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
    (writing U) and backward (adding to dx).  Where the step made the bf16
    copy X~, the products that read X read X~ (the values they would round X
    to as they load it)."""
    from parallelizable_recurrent_units_amd import (SRU_BF16, SRU_FACT_BWD_Q, SRU_FACT_BWD_X,
                                                    SRU_FACT_Q, SRU_FACT_U, SRU_FACT_WGRAD_O,
                                                    SRU_FACT_WGRAD_Q, sru_project_bwd_weight,
                                                    sru_project_factored,
                                                    sru_project_factored_bwd_weight)
    di = t["Q"].shape[1]
    xs = t["xb"] if t.get("xb") is not None else t["x"]

    def fact_fwd():
        sru_project_factored(shape, di, SRU_FACT_Q, xs, t["Wq"], t["Q"])
        sru_project_factored(shape, di, SRU_FACT_U, t["Q"], t["Wo"], t["U"])

    def fact_bwd():
        sru_project_factored(shape, di, SRU_FACT_BWD_Q, t["dU_lp"], t["Wo"], t["dQ"])
        sru_project_factored(shape, di, SRU_FACT_BWD_X, t["dQ"], t["Wq"], t["dx"], True)
        sru_project_factored_bwd_weight(shape, di, SRU_FACT_WGRAD_Q, t["dQ"], xs, t["dWq"],
                                        SRU_BF16, False, t["ws_f"])
        sru_project_factored_bwd_weight(shape, di, SRU_FACT_WGRAD_O, t["dU_lp"], t["Q"],
                                        t["dWo"], SRU_BF16, False, t["ws_f"])

    rows = [("f1_projection_bwd_weight",
             lambda: sru_project_bwd_weight(shape, t["dU_lp"], xs, t["dW"], SRU_BF16,
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


def time_rows(row_sets, steps, warmup, min_warm_s=0.0):
    """Run ``steps`` passes (rotating sets), HIP events between the rows,
    after ``warmup`` untimed passes (continued until ``min_warm_s`` seconds
    have gone by, so a GPU that sat idle reaches its working clock first).

    Returns (ms per step, {row: mean seconds})."""
    import torch
    nsets = len(row_sets)
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        for _, fn in row_sets[i % nsets]:
            fn()
        i += 1
        if i >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    names = [n for n, _ in row_sets[0]]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if len(names) == 1:
        # a step of one row: its launches back to back between the two events
        # (events between the steps would add a marker's drain to every launch)
        torch.cuda.synchronize()
        start.record()
        for i in range(steps):
            for _, fn in row_sets[i % nsets]:
                fn()
        end.record()
        torch.cuda.synchronize()
        total_ms = start.elapsed_time(end)
        return total_ms / steps, {names[0]: total_ms / 1e3 / steps}
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(steps)]
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
    from parallelizable_recurrent_units_amd import (SruAttnCfg, sru_attention_backward,
                                                    sru_attention_backward_workspace_size,
                                                    sru_attention_forward,
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
    # the backward takes this forward's Q, KV and R, and dU ~ N(0, 1) in bf16:
    # the copy the recurrence's backward writes for the products (the kernels
    # round an fp32 dU to bf16 as they load it, so the result is the same)
    dU = torch.randn((L * B, nd * 3 * d), generator=g, **f32).to(torch.bfloat16)
    dX = torch.empty((L * B, d), **f32)
    grads = [torch.empty(n, **f32) for n in (dp * d, 2 * dp * dp, nd * 3 * d * dp, 1, dp, dp)]
    wsb = torch.empty(sru_attention_backward_workspace_size(shape, cfg), device="cuda",
                      dtype=torch.uint8)
    return [("f2_attention_forward",
             lambda: sru_attention_forward(shape, cfg, X, Wq, Wkv, Wo, gamma, beta, Q, KV, R, U,
                                           ws)),
            ("f2_attention_backward",
             lambda: sru_attention_backward(shape, cfg, X, Wq, Wkv, Wo, gamma, Q, KV, R, dU, dX,
                                            *grads, wsb))]


class RowSet(list):
    """One set's step rows [(row, fn)], plus ``beyond``: rows timed after the
    step on the same buffers, and ``workspaces``: the scan workspaces whose
    error words are read after timing."""
    beyond = ()
    workspaces = ()


def check_error_words(sets):
    """Raise if any scan workspace of ``sets`` has its error word set (a
    bounded wait between chunks ran out: that call's outputs are invalid)."""
    from parallelizable_recurrent_units_amd import check_workspace
    for rs in sets:
        for name, ws in getattr(rs, "workspaces", ()):
            check_workspace(ws, name)


def row_sets_for(w, nsets, seed0, x_copy_mode="auto"):
    """Rotating sets of the rows of workload ``w`` (each set: list of (row, fn))."""
    import torch
    from parallelizable_recurrent_units_amd import (SRU_BWD, SRU_FWD, SRU_WS_LINEAR_BWD,
                                                    SRU_WS_LINEAR_FWD, SruShape, sru_forward,
                                                    sru_linear_scan, sru_workspace_size)
    f32 = dict(device="cuda", dtype=torch.float32)
    if w.mode == "layer":
        out = []
        for i in range(nsets):
            shape, t = device_set(w, seed0 + i, rounds_x_first(w, x_copy_mode))
            out.append(RowSet(training_step_rows(shape, t)))
            out[-1].beyond = next_rows(shape, t)
            out[-1].workspaces = [("sru_backward", t["ws"])]
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
    rs = RowSet([("a6_linear_forward", lambda: sru_linear_scan(s, SRU_FWD, w.chunk, U, x, b, None,
                                                               h=h, c_seq=c_seq, c_last=cl,
                                                               workspace=wsf)),
                 ("a7_linear_backward", lambda: sru_linear_scan(s, SRU_BWD, w.chunk, U, x, b, None,
                                                                c_seq=c_seq, dh=dh, dU=dU, dx=dx,
                                                                db=dbv, dc0=dc0, workspace=wsb))])
    rs.workspaces = [("linear scan forward", wsf), ("linear scan backward", wsb)]
    return [rs]


# the untimed warm-up of every timed set of rows lasts at least this long (and
# at least the requested number of steps): a GPU that has idled, or has only
# generated inputs, runs below its working clock for the first milliseconds
EXTRA_WARM_S = 0.2


def measure(w, nsets, steps, warmup, seed0):
    """(ms per step, {row: measurement}) for workload ``w``."""
    import torch
    sets = row_sets_for(w, nsets, seed0)
    ms, rows = time_rows(sets, steps, warmup, EXTRA_WARM_S)
    check_error_words(sets)
    work = row_work(w, w.mode == "layer" and rounds_x_first(w, "auto"))
    per_row = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    beyond = time_beyond(w, sets, steps, warmup, w.mode == "layer" and rounds_x_first(w, "auto"))
    if beyond:
        per_row["beyond_step"] = beyond
    del sets
    torch.cuda.empty_cache()
    return ms, per_row


def time_beyond(w, sets, steps, warmup, x_copy=False):
    """{row: measurement} of the rows beyond the step (after the step has run
    on every set, so their inputs hold a step's results)."""
    beyond = [s.beyond for s in sets if getattr(s, "beyond", ())]
    if not beyond:
        return {}
    _, rows = time_rows(beyond, steps, warmup, EXTRA_WARM_S)
    work = next_row_work(w, x_copy)
    out = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    for n, r in out.items():
        if n.startswith("f4_decode_step_B"):
            bb = int(n[len("f4_decode_step_B"):])
            r["us_per_step"] = r["us"] / DECODE_STEPS
            r["tokens_per_s"] = bb * DECODE_STEPS / rows[n]
    return out


def extras(main_id, steps, cpu_s=0.0):
    """Rows at the other workload sizes, each workload timed on its own."""
    from parallelizable_recurrent_units_amd.workloads import WORKLOADS
    out = {}
    others = [(wid, WORKLOADS[wid]) for wid in (2, 3, 4, 5) if wid != main_id]
    for wid, w in others:                 # every GPU measurement before the CPU ones
        linear = w.linear
        ms, per_row = measure(w, 1 if linear else 4, max(3, steps // 5) if linear else steps,
                              2 if linear else 3, 40 + 10 * wid)
        out[w.name] = dict(per_row, ms_per_step=ms)
    if cpu_s > 0:
        for _, w in others:
            print(f"[bench] CPU oracle baseline, {w.name}", file=sys.stderr, flush=True)
            out[w.name]["cpu_baseline"] = cpu_baseline(w, cpu_s)
    return out


CPU_BLOCK = 512   # channels per CPU-sample unit of the given-U workloads


def cpu_baseline_run(w, budget_s, threads):
    """The CPU oracle (as written, double precision) on a bounded sample of
    workload ``w``: units of one batch row (and, where U is given rather than
    projected, CPU_BLOCK channels), drawn with the workload's distributions,
    run through the same rows as the GPU step, repeated until about
    ``budget_s`` seconds.  Each row is timed on its own, so the recurrence
    rate (the metric's first part) and the whole step's are both reported,
    scaled by the fraction of the workload the sample covered."""
    import dataclasses
    import numpy as np
    import oracle
    from parallelizable_recurrent_units_amd.workloads import make_inputs
    oracle.set_num_threads(threads)
    dd = w.d if w.mode == "layer" else min(w.d, CPU_BLOCK)
    unit = dataclasses.replace(w, B=1, d=dd)
    inp = make_inputs(unit, seed=2)
    L, nd = w.L, w.ndir
    frac_unit = dd / (w.B * w.d)
    times = {}

    def timed(row, fn):
        t0 = time.perf_counter()
        r = fn()
        times[row] = times.get(row, 0.0) + time.perf_counter() - t0
        return r

    t_start = time.perf_counter()
    done = 0
    while True:
        if w.mode == "layer":
            U = timed("a1_projection", lambda: oracle.project(
                inp["x"].reshape(L, dd), inp["W"], True)).reshape(L, 1, nd, 3, dd)
        else:
            U = inp["U"]
        fwd_row = "a6_linear_forward" if w.linear else "a2_forward"
        fo = timed(fwd_row, lambda: oracle.forward(U, inp["x"], inp["v"], inp["b"], inp["c0"],
                                                   w.alpha))
        if w.backward:
            bwd_row = "a7_linear_backward" if w.linear else "a3_a4_backward"
            bo = timed(bwd_row, lambda: oracle.backward(U, inp["x"], inp["v"], inp["b"], inp["c0"],
                                                        fo["c"], inp["dh"], inp["dc_last"],
                                                        w.alpha))
            if w.mode == "layer":
                timed("a5_projection_bwd_data",
                      lambda: oracle.project_bwd_data(bo["dU"].reshape(L, -1), inp["W"]))
        done += 1
        if time.perf_counter() - t_start > budget_s:
            break
    frac = done * frac_unit
    work = row_work(w)
    rec = [n for n in times if n in RECURRENCE_ROWS]
    rec_bytes = sum(work[n]["bytes"] for n in rec) * frac
    rec_s = sum(times[n] for n in rec)
    step_s = sum(times.values())
    what = ("batch rows" if w.mode == "layer" else f"(batch row, {dd}-channel block) units")
    return {"value": rec_bytes / rec_s / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "elem_steps_per_s": w.elem_steps * frac / rec_s,
            "step_GB_per_s": sum(r["bytes"] for r in work.values()) * frac / step_s / 1e9,
            "step_ms_extrapolated": step_s / frac * 1e3,
            "row_seconds": times,
            "sample": f"{done} {what} = {frac:.4f} of the workload, rows {sorted(times)} in "
                      f"double precision, {step_s:.1f} s; algorithmic bytes and element-steps "
                      f"scaled by {frac:.4f}; value = the recurrence rows' bytes over their time"}


def cpu_baseline(w, budget_s=10.0):
    """The oracle on every host core (OpenMP over chains and GEMM rows), with
    the same sample single-threaded beside it."""
    import oracle
    every = oracle.num_threads()
    out = cpu_baseline_run(w, budget_s, every)
    out["single_thread"] = cpu_baseline_run(w, budget_s, 1)
    oracle.set_num_threads(every)
    return out


# kernel launches of one call of each row (what its event-timed span covers)
ROW_LAUNCHES = {
    "a1_round_x": ["round_bf16_kernel (X~ = bf16(X))"],
    "a1_projection": ["gemm_lds (X~ x W, operands copied straight into LDS; 256x256 tiles of "
                      "16 waves) after a1_round_x, or gemm_bf16_mfma (A = fp32 X, rounded to "
                      "bf16 while staged); see config.projection_x"],
    "a2_forward": ["fwd_fast (both directions in one grid)"],
    "a3_a4_backward": ["bwd_fast (fp32 inputs, up to 128 steps; both directions in one "
                       "launch when bidirectional and L <= 64, else one per direction, the "
                       "last one first) or scan_clear + bwd_scan per direction",
                       "param_reduce (dv, db)"],
    "a5_projection_bwd_data": ["gemm_lds (bf16 dU copy x bf16 W as stored, K-major: both "
                               "operands copied straight into LDS, W read back by transposing "
                               "LDS reads)"],
    "a6_linear_forward": ["scan_clear", "lin_fwd_fused"],
    "a7_linear_backward": ["scan_clear", "lin_bwd_fused", "lin_db_reduce"],
    "f1_projection_bwd_weight": ["gemm_lds_t (A = bf16 dU copy and B = bf16 X~, both read "
                                 "along L*B, copied straight into LDS and read back transposed) "
                                 "or gemm_bf16_mfma (fp32 X); the reduction split over blocks",
                                 "split_reduce (partial sums added in split order)"],
    "f3_factored_forward": ["gemm_bf16_mfma (Q = X Wq^T)", "gemm_bf16_mfma (U = Q Wo^T)"],
    "f4_decode_step_B1": [f"step_cell x {DECODE_STEPS} (one call per step, state in place, "
                          "replayed from a HIP graph)"],
    "f2_attention_forward": ["gemm_bf16_mfma (Q = X Wq^T)", "gemm_bf16_mfma ([K|V] = Q Wkv^T, "
                             "bf16 out)", "attn_v_transpose (V^T tiles)",
                             "attn_fwd_fused (scores, online softmax, weights x V, "
                             "R = layernorm(Q + alpha A) and its bf16 copy R~)",
                             "gemm_lds (U = R~ Wo^T, operands copied straight into LDS)"],
    "f2_attention_backward": ["the forward's scores, softmax and A again (3 launches)",
                              "transpose16 (Wo^T) + gemm_lds (dR = dU Wo, bf16 dU; 256x128 "
                              "tiles in three stages)",
                              "gemm + split_reduce (dWo)",
                              "attn_residual_bwd + attn_part_reduce", "gemm (dP = dO V^T)",
                              "attn_softmax_bwd", "gemm (dQ += dS' K)", "gemm TN (dK, dV, bf16 out)",
                              "gemm + split_reduce (dWkv)", "gemm (dQ += dKV Wkv)",
                              "round_bf16 (dQ~)", "gemm + split_reduce (dWq = dQ~^T X)",
                              "gemm (dX = dQ~ Wq)"],
    "f3_factored_backward": ["gemm_bf16_mfma (dQ = bf16(dU) Wo)", "gemm_bf16_mfma (dx += dQ Wq)",
                             "gemm_bf16_mfma + split_reduce (dWq = dQ^T X)",
                             "gemm_bf16_mfma + split_reduce (dWo = bf16(dU)^T Q)"],
}

# Which training-step row a dispatch belongs to, from its kernel name and,
# for the products that several rows launch (gemm_lds), the dispatch before
# it: rows run in order a1, a2, a3/a4, a5 in every step, so a gemm_lds after
# the X rounding is the projection, and one after the backward (or after a
# W^T transpose that follows the backward) the backward-data product.
ROW_OF_KERNEL = [
    (r"round_bf16_kernel", "a1_round_x"),
    (r"gemm_bf16_mfma<.*>, float, false, ", "a1_projection"),
    (r"fwd_fast<|fwd_split<|fwd_generic<", "a2_forward"),
    (r"bwd_scan<|bwd_fast<|bwd_generic<|scan_clear|param_reduce", "a3_a4_backward"),
]
ROW_ONCE = {"a2_forward": r"fwd_fast<|fwd_split<|fwd_generic<"}   # one dispatch per step


def rows_of_dispatches(names):
    """Row of each dispatch (dict id -> row) given {id: kernel name}: a
    kernel named in ROW_OF_KERNEL fixes the row; gemm_lds takes the row of
    the dispatch before it; anything else (input generation, copies, the rows
    timed beyond the step) none.  Projection kernels count only when the
    forward recurrence comes next, since the same product kernels also serve
    rows beyond the step."""
    import re
    out, cur, pending, a5_transpose = {}, None, [], False
    for did in sorted(names):
        n = names[did]
        row = next((r for pat, r in ROW_OF_KERNEL if re.search(pat, n)), None)
        transpose = re.search(r"transpose16", n) is not None
        if row is None and transpose and cur == "a3_a4_backward":
            row = "a5_projection_bwd_data"               # W^T for the backward-data product
        elif row is None and re.search(r"gemm_lds<", n):
            if cur == "a1_round_x":
                row = "a1_projection"
            elif cur == "a3_a4_backward" or a5_transpose:
                row = "a5_projection_bwd_data"
        a5_transpose = transpose and row == "a5_projection_bwd_data"
        if row in ("a1_round_x", "a1_projection"):
            pending.append((did, row))
        else:
            if row == "a2_forward":
                out.update(dict(pending))
            pending = []
            if row is not None:
                out[did] = row
        cur = row
    return out


def _per_dispatch(run_dir, counter):
    """{(file, dispatch id): (kernel name, counter summed over its hardware
    instances)} from the rocpd database(s) a rocprofv3 --pmc run wrote under
    ``run_dir``."""
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


def write_traffic(workload, fetch_dir, write_dir, copy_bytes):
    """profiles/traffic.json, entry ``workload``: HBM bytes per call of each
    row at that workload (entries of other workloads are kept).  FETCH_SIZE and
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
        by_file = {}
        for (f, did), (n, v) in per.items():
            by_file.setdefault(f, {})[did] = (n, v)
        kib, calls = {}, {}
        for f, disp in by_file.items():
            owner = rows_of_dispatches({d: nv[0] for d, nv in disp.items()})
            for did, row in owner.items():
                n, v = disp[did]
                kib[row] = kib.get(row, 0.0) + v
                if re.search(ROW_ONCE["a2_forward"], n):
                    calls["steps"] = calls.get("steps", 0) + 1
        steps = calls.get("steps", 0)
        if not steps:
            raise SystemExit(f"{counter}: no forward dispatch under {run_dir}")
        for row, k in kib.items():
            r = rows.setdefault(row, {"calls": steps})
            r[counter.lower() + "_bytes"] = k * 1024.0 * factors[counter] / steps
    for r in rows.values():
        if "fetch_size_bytes" in r and "write_size_bytes" in r:
            r["bytes"] = r["fetch_size_bytes"] + r["write_size_bytes"]
    rec = {"source_digest": source_digest(), "copy_probe_bytes": copy_bytes,
           "calibration_factors": factors,
           "rows": {k: v["bytes"] for k, v in rows.items() if "bytes" in v},
           "detail": rows}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = {}
    if os.path.exists(path):
        with open(path) as f:
            allrec = json.load(f)
    allrec = {"workloads": dict(allrec.get("workloads", {}), **{workload: rec})}
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(rec, indent=1))


def traffic_for(workload, kernel_row, digest):
    """HBM bytes per call of a row from the committed counter summary, if it
    was taken at this workload on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get("workloads", {}).get(workload, {})
    if rec.get("source_digest") != digest:
        return None
    return rec.get("rows", {}).get(kernel_row)


def main():
    args = parse()
    if args.write_traffic:
        if not args.copy_probe_mib:
            raise SystemExit("--write-traffic needs the --copy-probe-mib the runs used")
        from parallelizable_recurrent_units_amd.workloads import WORKLOADS
        write_traffic(WORKLOADS[args.workload].name, *args.write_traffic,
                      copy_bytes=args.copy_probe_mib * (1 << 20))
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
    row_sets = row_sets_for(w, nsets, 100, args.x_copy)
    print("[bench] timing", file=sys.stderr, flush=True)
    ms, rows = time_rows(row_sets, args.steps, args.warmup, EXTRA_WARM_S)
    check_error_words(row_sets)
    beyond = {} if args.no_beyond else time_beyond(
        w, row_sets, args.steps, args.warmup, w.mode == "layer" and rounds_x_first(w, args.x_copy))
    del row_sets
    torch.cuda.empty_cache()
    x_copy = w.mode == "layer" and rounds_x_first(w, args.x_copy)
    work = row_work(w, x_copy)
    per_row = {n: dict(us=rows[n] * 1e6, **roofline_of(n, work[n], rows[n])) for n in rows}
    dominant = max(rows, key=lambda n: rows[n])
    digest = source_digest()
    roof = dict(roofline_of(dominant, work[dominant], rows[dominant]))
    roof["kernel"] = dominant
    roof["launches_per_call"] = ROW_LAUNCHES.get(dominant)
    roof["traffic"] = traffic_for(w.name, dominant, digest)
    gemm_roof = None
    if "a1_projection" in rows and dominant != "a1_projection":
        gemm_roof = dict(roofline_of("a1_projection", work["a1_projection"], rows["a1_projection"]))
        gemm_roof["kernel"] = "a1_projection"
        gemm_roof["launches_per_call"] = ROW_LAUNCHES.get("a1_projection")
        gemm_roof["traffic"] = traffic_for(w.name, "a1_projection", digest)
    step_bytes = sum(r["bytes"] for r in work.values())
    rec_rows = [n for n in per_row if n in RECURRENCE_ROWS]
    rec_bytes = sum(work[n]["bytes"] for n in rec_rows)
    rec_s = sum(rows[n] for n in rec_rows)
    line = {
        "metric": METRIC,
        "value": rec_bytes / rec_s / 1e9,
        "value_is": "the forward + backward recurrence rows' algorithmic bytes over their "
                    "event-timed time (" + " + ".join(rec_rows) + ")",
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_min_s": EXTRA_WARM_S,
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
                   "x": w.x_dtype, "W": w.w_dtype, "parallelism": "single GPU",
                   "projection_x": ("bf16 copy X~ = bf16(X) made in the row (sru_round_bf16)"
                                    if w.mode == "layer" and rounds_x_first(w, args.x_copy) else
                                    "as given (fp32 rounded to bf16 while staged)"
                                    if w.mode == "layer" else None)},
        "elem_steps_per_s": w.elem_steps / rec_s,
        "frac_of_hbm_peak": rec_bytes / rec_s / 1e9 / HBM_PEAK_GBS,
        "gemm_frac_of_mfma_peak": {n: per_row[n]["frac"] for n in GEMM_ROWS if n in per_row},
        "step_GB_per_s": step_bytes / (ms / 1e3) / 1e9,
        "step_elem_steps_per_s": w.elem_steps / (ms / 1e3),
        "step_algorithmic_bytes": step_bytes,
        "rows": per_row,
        "beyond_step": beyond,
        "roofline": roof,
        "roofline_projection_gemm": gemm_roof,
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
    if not args.no_extras:
        print("[bench] other workloads", file=sys.stderr, flush=True)
        line["other_workloads"] = extras(args.workload, max(10, args.steps // 2),
                                         0.0 if args.no_cpu_baseline else 3.0)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
