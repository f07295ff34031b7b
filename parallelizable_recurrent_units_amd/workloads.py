"""Seeded synthetic workloads for the SRU layer.

This module only draws random numbers and packs them; it holds none of the
layer's arithmetic.  It is the one piece the HIP path's tests/benchmark and the
CPU oracle share: both are handed the same arrays.

The pages measure on language-model and classification corpora (enwik8,
WikiText-103, Billion Word, IMDb, SQuAD); none is used.  Gaussian and uniform
draws of the same shapes stand in for them: hidden sizes follow the SRU++
paper's Figure 2 (d = 2048) and training unroll (1024).

Each workload uses ``numpy.random.default_rng(seed)`` (PCG64) with a fixed draw
order: x, W (or U), v, b, c0, dh, dc_last.  For a bidirectional layer the
direction-0 parameters are drawn before direction 1's inside each array.
bf16 tensors are drawn in fp32 and rounded once to bf16 (round to nearest even,
done by torch's CPU conversion); the fp32 view of those bf16 values is what the
oracle receives.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    L: int
    B: int
    d: int
    ndir: int
    alpha: float
    # "layer": X and W are given and U = X W^T is computed by the projection.
    # "given_u": U is supplied directly (e.g. produced by an attention block).
    mode: str
    x_dtype: str              # "f32" | "bf16"
    w_dtype: Optional[str]    # "f32" | "bf16" | None (given U)
    u_dtype: str              # dtype of U as stored ("f32" | "bf16")
    w_init: str = "xavier"    # "xavier" | "uniform_sqrt3"
    c0: str = "zero"          # "zero" | "normal0.1"
    backward: bool = False
    linear: bool = False      # v = 0 (linear recurrence), chunked scan
    chunk: int = 256
    uf_shift: float = 0.0     # mean of the f-gate pre-activation draw (given U)
    description: str = ""

    @property
    def elem_steps(self) -> int:
        return self.ndir * self.L * self.B * self.d


# The five workloads the hot path is specified on.
WORKLOADS = {
    1: Workload("sru-uni-fp32-L32-B4-d64", L=32, B=4, d=64, ndir=1, alpha=1.0,
                mode="layer", x_dtype="f32", w_dtype="f32", u_dtype="f32",
                w_init="uniform_sqrt3",
                description="single unidirectional layer, fp32 throughout, forward only"),
    2: Workload("sru-bi-L64-B128-d512", L=64, B=128, d=512, ndir=2, alpha=1.0,
                mode="layer", x_dtype="f32", w_dtype="bf16", u_dtype="f32",
                backward=True,
                description="bidirectional layer, classification shapes, forward + backward"),
    3: Workload("sru-given-u-bf16-L1024-B16-d2048", L=1024, B=16, d=2048, ndir=1,
                alpha=math.sqrt(3.0), mode="given_u", x_dtype="bf16", w_dtype=None,
                u_dtype="bf16",
                description="SRU++-style recurrence on a supplied bf16 U, forward only"),
    4: Workload("sru-train-L512-B32-d1024", L=512, B=32, d=1024, ndir=1, alpha=1.0,
                mode="layer", x_dtype="f32", w_dtype="bf16", u_dtype="f32",
                c0="normal0.1", backward=True,
                description="full layer training step: projection, forward, backward, dX"),
    5: Workload("sru-linear-L16384-B4-d4096", L=16384, B=4, d=4096, ndir=1, alpha=1.0,
                mode="given_u", x_dtype="f32", w_dtype=None, u_dtype="f32",
                backward=True, linear=True, chunk=256, uf_shift=2.0,
                description="linear recurrence (v = 0), chunked scan, forward + backward"),
}


def to_bf16(a: np.ndarray):
    """Round fp32 to bf16 (nearest even) with torch's CPU cast.

    Returns (bits as uint16, the same values widened to fp32)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16).copy()
    vals = t.to(torch.float32).numpy().copy()
    return bits, vals


def _std_normal(rng, shape, mean=0.0, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def make_inputs(w: Workload, seed: int, *, with_grads: Optional[bool] = None,
                dc_last: bool = False, v_scale: float = 0.1, b_scale: float = 0.0):
    """Draw one workload's inputs.

    Returns a dict of numpy arrays.  fp32 tensors are float32 arrays; a bf16
    tensor ``k`` appears twice: ``k`` (float32 values, exactly representable
    in bf16) and ``k + "_bits"`` (uint16 patterns for the device).

    ``b_scale`` > 0 draws b ~ U(-b_scale, b_scale) instead of the workloads'
    b = 0 (used by extra parity cases); ``dc_last`` draws a non-zero upstream
    gradient for the final state (the workloads themselves use 0).
    """
    rng = np.random.default_rng(seed)
    L, B, d, nd = w.L, w.B, w.d, w.ndir
    out = {}
    # x
    x = _std_normal(rng, (L, B, d))
    if w.x_dtype == "bf16":
        out["x_bits"], out["x"] = to_bf16(x)
    else:
        out["x"] = x
    # W or U
    if w.mode == "layer":
        if w.w_init == "uniform_sqrt3":
            bound = math.sqrt(3.0 / d)
        else:  # Xavier-uniform for a d -> 3d map
            bound = math.sqrt(6.0 / (d + 3 * d))
        W = rng.uniform(-bound, bound, size=(nd * 3 * d, d)).astype(np.float32)
        if w.w_dtype == "bf16":
            out["W_bits"], out["W"] = to_bf16(W)
        else:
            out["W"] = W
    else:
        U = _std_normal(rng, (L, B, nd, 3, d))
        if w.uf_shift:
            U[:, :, :, 0, :] += np.float32(w.uf_shift)
        if w.u_dtype == "bf16":
            out["U_bits"], out["U"] = to_bf16(U)
        else:
            out["U"] = U
    # v (zero in the linear mode), b
    if w.linear:
        out["v"] = np.zeros((nd, 2, d), np.float32)
    else:
        out["v"] = rng.uniform(-v_scale, v_scale, size=(nd, 2, d)).astype(np.float32)
    if b_scale > 0:
        out["b"] = rng.uniform(-b_scale, b_scale, size=(nd, 2, d)).astype(np.float32)
    else:
        out["b"] = np.zeros((nd, 2, d), np.float32)
    # c0
    if w.c0 == "normal0.1":
        out["c0"] = _std_normal(rng, (nd, B, d), std=0.1)
    else:
        out["c0"] = np.zeros((nd, B, d), np.float32)
    # upstream gradients
    if with_grads is None:
        with_grads = w.backward
    if with_grads:
        out["dh"] = _std_normal(rng, (L, B, nd, d))
        if dc_last:
            out["dc_last"] = _std_normal(rng, (nd, B, d))
        else:
            out["dc_last"] = np.zeros((nd, B, d), np.float32)
    return out


def custom(L, B, d, ndir=1, alpha=1.0, mode="given_u", x_dtype="f32", w_dtype=None,
           u_dtype="f32", c0="normal0.1", backward=True, linear=False, chunk=256,
           uf_shift=0.0, w_init="xavier", name="custom") -> Workload:
    """A workload of arbitrary shape for parity and edge-case tests."""
    if mode == "layer" and w_dtype is None:
        w_dtype = "bf16"
    return Workload(name, L=L, B=B, d=d, ndir=ndir, alpha=alpha, mode=mode,
                    x_dtype=x_dtype, w_dtype=w_dtype, u_dtype=u_dtype, w_init=w_init,
                    c0=c0, backward=backward, linear=linear, chunk=chunk,
                    uf_shift=uf_shift)


def factored_inputs(L, B, d, ndir, d_inner, seed, w_dtype="bf16"):
    """Inputs of the factorised projection (SRU++ paper, Fig. 2(b); the paper
    pairs d = 2048 with d' = 512, i.e. d' = d / 4).  Draw order: X, Wq, Wo,
    then stand-ins for the tensors the rest of the layer would supply: Q (an
    input of the U and weight products when tested on their own), dU and dQ.
    X, Q, dU, dQ ~ N(0, 1); Wq ~ Xavier-U for d -> d', Wo ~ Xavier-U for
    d' -> ndir*3d, rounded once to bf16 when ``w_dtype`` is "bf16".  Arrays
    are 2-D: [L*B, features] for activations, [out, in] for weights."""
    rng = np.random.default_rng(seed)
    M, n3 = L * B, ndir * 3 * d
    out = {"X": _std_normal(rng, (M, d))}
    for name, fan_in, fan_out in (("Wq", d, d_inner), ("Wo", d_inner, n3)):
        bound = math.sqrt(6.0 / (fan_in + fan_out))
        W = rng.uniform(-bound, bound, size=(fan_out, fan_in)).astype(np.float32)
        if w_dtype == "bf16":
            out[name + "_bits"], out[name] = to_bf16(W)
        else:
            out[name] = W
    out["Q"] = _std_normal(rng, (M, d_inner))
    out["dU"] = _std_normal(rng, (M, n3))
    out["dQ"] = _std_normal(rng, (M, d_inner))
    return out


def attention_inputs(L, B, d, ndir, d_inner, mem_len, seed):
    """Inputs of the SRU++ attention U-producer (SRU++ paper, section on
    SRU++; its models use d = 4 d').  Draw order: X ~ N(0, 1) [L*B, d]; Wq,
    Wk, Wv, Wo ~ Xavier-U for d -> d', d' -> d', d' -> d', d' -> ndir*3d, each
    rounded once to bf16 (Wk and Wv stacked as Wkv [2d', d']); the previous
    segment's keys and values ~ N(0, 1) [mem_len, B, d'] in bf16; gamma ~
    1 + U(-0.1, 0.1), beta ~ U(-0.1, 0.1) [d'] (fp32)."""
    rng = np.random.default_rng(seed)
    out = {"X": _std_normal(rng, (L * B, d))}
    ws = []
    for fan_in, fan_out in ((d, d_inner), (d_inner, d_inner), (d_inner, d_inner),
                            (d_inner, ndir * 3 * d)):
        bound = math.sqrt(6.0 / (fan_in + fan_out))
        ws.append(rng.uniform(-bound, bound, size=(fan_out, fan_in)).astype(np.float32))
    out["Wq_bits"], out["Wq"] = to_bf16(ws[0])
    out["Wkv_bits"], out["Wkv"] = to_bf16(np.concatenate([ws[1], ws[2]]))
    out["Wo_bits"], out["Wo"] = to_bf16(ws[3])
    out["Kmem_bits"], out["Kmem"] = to_bf16(_std_normal(rng, (mem_len, B, d_inner)))
    out["Vmem_bits"], out["Vmem"] = to_bf16(_std_normal(rng, (mem_len, B, d_inner)))
    out["gamma"] = (1.0 + rng.uniform(-0.1, 0.1, size=d_inner)).astype(np.float32)
    out["beta"] = rng.uniform(-0.1, 0.1, size=d_inner).astype(np.float32)
    return out
