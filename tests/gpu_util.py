"""Helpers for the GPU parity tests: device copies and error measures."""
import numpy as np


def dev_inputs(inp, device="cuda"):
    """numpy workload dict -> device tensors (bf16 tensors from their bit patterns)."""
    import torch
    out = {}
    for k, v in inp.items():
        if k.endswith("_bits"):
            continue
        if k + "_bits" in inp:
            bits = np.ascontiguousarray(inp[k + "_bits"]).view(np.int16)
            out[k] = torch.from_numpy(bits).to(device).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v)).to(device)
    return out


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def normwise(gpu, ref):
    """max |gpu - ref| / max |ref| (the tolerance measure of the parity bar)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    return float(err / scale) if scale > 0 else float(err)


def check(name, gpu, ref, tol, log=None):
    e = normwise(gpu, ref)
    if log is not None:
        log[name] = e
    print(f"  {name}: normwise rel err {e:.3e} (tol {tol:g})", flush=True)
    assert e <= tol, f"{name}: {e} > {tol}"
    return e
