"""Host logic of bench.py (no GPU): which training-step row each kernel
dispatch of a rocprofv3 trace is charged to."""
import bench

LDS = "void sru::gemm_lds<sru::LdsCfg<256, 256, 2, 4, 4, 1>, unsigned short, float, false>(MM)"
LDS_KN = "void sru::gemm_lds<sru::LdsCfg<256, 256, 2, 4, 4, 1>, unsigned short, float, true>(MM)"
MFMA_F32X = ("void sru::gemm_bf16_mfma<sru::TileCfg<256, 192, 64, 1, 1, 4, 2, false>, float, "
             "false, unsigned short, false, true, float>(MM)")
LDS_T = "void sru::gemm_lds_t<sru::LdsCfg<256, 256, 2, 4, 4, 1> >(MM)"


def _rows(seq):
    return bench.rows_of_dispatches({i: n for i, n in enumerate(seq)})


def test_step_with_rounded_x_and_untransposed_w():
    step = ["round_bf16_kernel(long, float const*, unsigned short*)", LDS, "fwd_split<false, 8, 4>",
            "scan_clear(unsigned int*, long)", "bwd_scan<float, float, 8, 8, 4>(BwdScanArgs)",
            "param_reduce(float const*, long, long, float*, float*)", LDS_KN]
    out = _rows(step + step)
    want = ["a1_round_x", "a1_projection", "a2_forward"] + ["a3_a4_backward"] * 3 + \
        ["a5_projection_bwd_data"]
    assert [out[i] for i in range(len(step) * 2)] == want + want


def test_step_with_fp32_x_and_transposed_w():
    step = [MFMA_F32X, "fwd_fast<false, 16, 8>", "bwd_fast<8, 4, true>",
            "param_reduce(float const*, long, long, float*, float*)",
            "transpose16<true>(long, long, unsigned short const*, unsigned short*)", LDS]
    out = _rows(step)
    assert [out[i] for i in range(len(step))] == [
        "a1_projection", "a2_forward", "a3_a4_backward", "a3_a4_backward",
        "a5_projection_bwd_data", "a5_projection_bwd_data"]


def test_products_outside_the_step_are_not_charged():
    # a projection-shaped kernel without the forward after it, the weight
    # gradient, and a second LDS product after the backward-data one
    seq = [MFMA_F32X, "split_reduce(float const*, long, long, float*, bool)",
           "bwd_fast<8, 4, true>", LDS_KN, LDS, LDS_T, LDS]
    out = _rows(seq)
    assert 0 not in out and 1 not in out
    assert out[2] == "a3_a4_backward" and out[3] == "a5_projection_bwd_data"
    assert 4 not in out and 5 not in out and 6 not in out


def test_transposes_outside_the_step_are_not_charged():
    # the attention backward's W_o^T and its product follow other kernels
    seq = ["fwd_split<true, 16, 8>", "attn_fwd_fused<512>(FusedArgs)",
           "transpose16<true>(long, long, unsigned short const*, unsigned short*)",
           "void sru::gemm_lds<sru::LdsCfg<256, 128, 3, 4, 2, 1>, unsigned short, float, false>(MM)"]
    out = _rows(seq)
    assert out == {0: "a2_forward"}
