"""GPU parity of the SRU++ attention U-producer (SRU++ paper, section on SRU++)
through the C ABI, against the CPU oracle on the same seeded inputs.

Tolerances (normwise, as in test_parity_gpu.py), against the oracle that
rounds the same operands to bf16 (round_ops):
  * Q: 1e-4 (one product; fp32 accumulation order only);
  * KV (stored in bf16): 8e-3, two bf16 ulps at the largest element.  The
    kernel rounds its fp32 sum and the oracle its double sum, so an element
    close to a rounding boundary can land one bf16 value apart (2^-8 of it);
  * R and U: 3e-3.  The same one-ulp flips enter through the rounded keys,
    attention weights and R~, each shifting a product by a fraction of 2^-8;
against the oracle without any rounding: 2e-2 (the bf16 bar) for all.
"""
import numpy as np
import pytest

import oracle
from parallelizable_recurrent_units_amd import SruAttnCfg, SruShape, layer, workloads
from tests.gpu_util import check, host

pytestmark = pytest.mark.gpu

GEMM_ACC = 1e-4
BF16_OUT = 8e-3
CHAIN = 3e-3
BF16_BAR = 2e-2


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


def run(L, B, d, nd, dp, Lm, causal, ln, alpha, inp, X=None, kv_mem=None, u_dtype=None):
    """GPU call; the KV buffer's first Lm rows hold the previous segment."""
    import torch
    shape = SruShape(L, B, d, nd == 2, 1.0)
    cfg = SruAttnCfg(dp, Lm, causal, ln, alpha, 1e-5)
    KV = torch.empty((Lm + L, B, 2 * dp), device="cuda", dtype=torch.bfloat16)
    if Lm:
        KV[:Lm] = kv_mem if kv_mem is not None else torch.cat(
            [dev(inp["Kmem"], inp["Kmem_bits"]), dev(inp["Vmem"], inp["Vmem_bits"])], dim=2)
    g = dict(gamma=dev(inp["gamma"]), beta=dev(inp["beta"])) if ln else {}
    if u_dtype is not None:
        g["u_dtype"] = u_dtype
    Q, KV, R, U = layer.attention_forward(
        shape, cfg, dev(inp["X"]) if X is None else X, dev(inp["Wq"], inp["Wq_bits"]),
        dev(inp["Wkv"], inp["Wkv_bits"]), dev(inp["Wo"], inp["Wo_bits"]), KV=KV, **g)
    return Q, KV, R, U


def reference(L, B, dp, Lm, causal, ln, alpha, inp, round_ops, X=None, Kmem=None, Vmem=None):
    Wkv = inp["Wkv"]
    return oracle.attention_project(
        inp["X"] if X is None else X, inp["Wq"], Wkv[:dp], Wkv[dp:], inp["Wo"], L, B, alpha,
        mem_len=Lm, Kmem=inp["Kmem"] if Kmem is None else Kmem,
        Vmem=inp["Vmem"] if Vmem is None else Vmem, causal=causal,
        ln=(inp["gamma"], inp["beta"], 1e-5) if ln else None, round_ops=round_ops)


def compare(L, B, dp, Lm, gpu, ref, round_ops):
    Q, KV, R, U = gpu
    M = L * B
    kv = host(KV)                                        # [Lm + L, B, 2dp]
    tol = (lambda t: t) if round_ops else (lambda t: BF16_BAR)
    check("Q", host(Q), ref["Q"], tol(GEMM_ACC))
    check("K (this segment)", kv[Lm:, :, :dp], ref["K"][Lm:], tol(BF16_OUT))
    check("V (this segment)", kv[Lm:, :, dp:], ref["V"][Lm:], tol(BF16_OUT))
    check("R", host(R), ref["R"], tol(CHAIN))
    check("U", host(U).reshape(M, -1), ref["U"], tol(CHAIN))


# (L, B, d, ndir, d', Lm, causal, layernorm, alpha): ragged sizes (bounds-
# checked product paths), context rows, both masks, layer norm, rows longer
# than the softmax register path (Lm + L > 2048)
CASES = [(8, 3, 64, 1, 16, 0, True, False, 0.5),
         (33, 5, 100, 2, 25, 7, True, True, 0.7),
         (64, 4, 128, 1, 32, 64, True, False, 1.0),
         (64, 2, 256, 1, 64, 0, False, True, 0.3),
         (130, 2, 128, 1, 32, 0, True, False, 1.0),
         (300, 1, 64, 2, 16, 44, False, False, 2.0),
         (1100, 1, 64, 1, 16, 1000, True, True, 1.0),
         # odd key counts (bf16 weight rows at odd element offsets): one query
         # that sees one key (weight exactly 1), one query over 5 context
         # steps, five queries over five keys without the mask
         (1, 3, 64, 1, 16, 0, True, False, 0.5),
         (1, 2, 64, 1, 16, 5, True, True, 1.0),
         (5, 2, 64, 1, 16, 0, False, False, 1.0)]

# d' in {64, 128, 256, 512} takes the fused kernel (scores, softmax, weights x
# values, residual and norm in one pass over key tiles of 32): query blocks
# of 64 with ragged ends, context rows not a multiple of 32, both masks,
# layer norm on and off, workgroup counts that are and are not multiples of
# 8 (the XCD grouping), one query over one key
FUSED_CASES = [(100, 3, 256, 1, 64, 37, True, True, 0.8),
               (130, 4, 512, 1, 128, 70, True, False, 1.0),
               (70, 8, 512, 2, 128, 0, False, True, 0.5),
               (200, 2, 1024, 1, 256, 100, True, True, 1.0),
               (129, 2, 2048, 1, 512, 64, True, True, 1.0),
               (64, 16, 1024, 1, 512, 31, False, True, 0.7),
               (1, 1, 256, 1, 64, 0, True, True, 1.0),
               (33, 2, 512, 1, 128, 5, True, False, 2.0),
               # two directions' U channels (n3 = 600) after the fused kernel
               (40, 2, 100, 2, 64, 10, True, True, 0.9)]


@pytest.mark.parametrize("L,B,d,nd,dp,Lm,causal,ln,alpha", CASES + FUSED_CASES)
def test_attention_forward(L, B, d, nd, dp, Lm, causal, ln, alpha):
    inp = workloads.attention_inputs(L, B, d, nd, dp, Lm, seed=1000 + L + dp)
    print(f"case L={L} B={B} d={d} nd={nd} d'={dp} Lm={Lm} causal={causal} ln={ln}", flush=True)
    gpu = run(L, B, d, nd, dp, Lm, causal, ln, alpha, inp)
    for round_ops in (True, False):
        print(f" vs {'rounded' if round_ops else 'exact'} oracle", flush=True)
        compare(L, B, dp, Lm, gpu, reference(L, B, dp, Lm, causal, ln, alpha, inp, round_ops),
                round_ops)


@pytest.mark.parametrize("L,B,d,nd,dp,Lm", [(96, 3, 128, 2, 32, 40), (70, 3, 128, 2, 64, 40)])
def test_attention_bf16_u(L, B, d, nd, dp, Lm):
    """U written in bf16 is the fp32 U of the same call rounded to nearest
    even, bit for bit (same product, same accumulation; only the epilogue
    rounds), and meets the oracle within the chain tolerance plus one
    rounding of the output (2^-9 relative per element).  d' = 64 takes the
    fused attention kernel before the product."""
    import torch
    inp = workloads.attention_inputs(L, B, d, nd, dp, Lm, seed=1250)
    shape = SruShape(L, B, d, nd == 2, 1.0)
    cfg = SruAttnCfg(dp, Lm, True, True, 0.7, 1e-5)
    mem = torch.cat([dev(inp["Kmem"], inp["Kmem_bits"]), dev(inp["Vmem"], inp["Vmem_bits"])], dim=2)
    args = (shape, cfg, dev(inp["X"]), dev(inp["Wq"], inp["Wq_bits"]),
            dev(inp["Wkv"], inp["Wkv_bits"]), dev(inp["Wo"], inp["Wo_bits"]))
    ln = dict(gamma=dev(inp["gamma"]), beta=dev(inp["beta"]))
    outs = []
    for u_dtype in (torch.float32, torch.bfloat16):
        KV = torch.empty((Lm + L, B, 2 * dp), device="cuda", dtype=torch.bfloat16)
        KV[:Lm] = mem
        outs.append(layer.attention_forward(*args, KV=KV, u_dtype=u_dtype, **ln))
    torch.cuda.synchronize()
    U32, Ub = outs[0][3], outs[1][3]
    assert Ub.dtype == torch.bfloat16
    assert torch.equal(Ub.view(torch.int16), U32.to(torch.bfloat16).view(torch.int16))
    ref = reference(L, B, dp, Lm, True, True, 0.7, inp, True)
    check("U (bf16)", host(Ub).reshape(L * B, -1), ref["U"], CHAIN + 2.0 ** -9)


def test_attention_alpha_zero_is_the_factorised_projection():
    """alpha = 0: U equals the factorised projection's U bit for bit (the
    attention term is multiplied by zero; both run Q and U on the same
    kernels with the same operands)."""
    L, B, d, dp = 64, 4, 128, 32
    inp = workloads.attention_inputs(L, B, d, 1, dp, 0, seed=1201)
    _, _, _, U = run(L, B, d, 1, dp, 0, True, False, 0.0, inp)
    _, Uf = layer.project_factored(SruShape(L, B, d, False, 1.0), dp, dev(inp["X"]),
                                   dev(inp["Wq"], inp["Wq_bits"]), dev(inp["Wo"], inp["Wo_bits"]))
    assert np.array_equal(host(U), host(Uf))


def test_attention_two_segments_carry_context():
    """Segment 2 attends to segment 1's keys and values, which segment 1's call
    wrote into its KV rows.  The oracle runs segment 1 on its own and hands its
    K, V to segment 2 as the context."""
    import torch
    L, B, d, dp = 48, 3, 128, 32
    inp = workloads.attention_inputs(L, B, d, 1, dp, 0, seed=1301)
    X2 = np.random.default_rng(1302).standard_normal((L * B, d)).astype(np.float32)
    _, KV1, _, _ = run(L, B, d, 1, dp, 0, True, True, 0.8, inp)
    gpu2 = run(L, B, d, 1, dp, L, True, True, 0.8, inp, X=dev(X2), kv_mem=KV1.clone())
    torch.cuda.synchronize()
    for round_ops in (True, False):
        r1 = reference(L, B, dp, 0, True, True, 0.8, inp, round_ops)
        r2 = reference(L, B, dp, L, True, True, 0.8, inp, round_ops, X=X2,
                       Kmem=oracle.round_bf16(r1["K"]), Vmem=oracle.round_bf16(r1["V"]))
        compare(L, B, dp, L, gpu2, r2, round_ops)


def test_attention_workload_sampled_sequences():
    """The shape whose U the given-U workload consumes: L=1024, B=16, d=2048,
    d' = d/4 = 512, causal, the previous 1024-step segment as context.  Two
    whole sequences (every row of Q, K, V, R, U) against the oracle; the bf16
    U that the given-U recurrence takes (the same product with a rounding
    epilogue) is the fp32 U rounded, bit for bit, over every row."""
    import torch
    L, B, d, dp, Lm = 1024, 16, 2048, 512, 1024
    inp = workloads.attention_inputs(L, B, d, 1, dp, Lm, seed=1401)
    print("workload attention L=1024 B=16 d=2048 d'=512 Lm=1024", flush=True)
    Q, KV, R, U = run(L, B, d, 1, dp, Lm, True, True, 1.0, inp)
    Ub = run(L, B, d, 1, dp, Lm, True, True, 1.0, inp, u_dtype=torch.bfloat16)[3]
    torch.cuda.synchronize()
    assert Ub.dtype == torch.bfloat16
    assert torch.equal(Ub.view(torch.int16), U.to(torch.bfloat16).view(torch.int16))
    del Ub
    X3 = inp["X"].reshape(L, B, d)
    for b in (0, B - 1):
        print(f" sequence {b}", flush=True)
        sub = dict(inp, X=np.ascontiguousarray(X3[:, b]),
                   Kmem=np.ascontiguousarray(inp["Kmem"][:, b:b + 1]),
                   Vmem=np.ascontiguousarray(inp["Vmem"][:, b:b + 1]))
        ref = reference(L, 1, dp, Lm, True, True, 1.0, sub, True)
        check("Q", host(Q.view(L, B, dp)[:, b]), ref["Q"], GEMM_ACC)
        kv = host(KV[Lm:, b])
        check("K", kv[:, :dp], ref["K"][Lm:, 0], BF16_OUT)
        check("V", kv[:, dp:], ref["V"][Lm:, 0], BF16_OUT)
        check("R", host(R.view(L, B, dp)[:, b]), ref["R"], CHAIN)
        check("U", host(U[:, b]).reshape(L, -1), ref["U"], CHAIN)
