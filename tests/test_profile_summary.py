"""Attribution of kernel names to C-ABI calls in the rocprofv3 summaries."""
from fine_grained_fp8_quant_amd.profile_summary import api_of, short


def test_short_names_spell_out_the_mode():
    assert short("void fgq::k_gemm_fp8_bs<fgq::TileCfg<192, 256, 2, 4, 2, false>, 0>(unsigned char const*)") \
        == "k_gemm_fp8_bs[192x256,exact]"
    assert short("void fgq::k_grouped_gemm_fp8_bs<fgq::TileCfg<64, 128, 1, 4, 2, true>, 3>(int)") \
        == "k_grouped_gemm_fp8_bs[64x128,incore]"


def test_quantisers_and_dispatch():
    assert api_of("k_quant_act_1x128<ScaleF32>", False) == ("quant_act_1x128", None)
    assert api_of("k_quant_w_128x128<ScaleE8M0, true>", True) == ("quant_w_128x128_e8m0", None)
    assert api_of("k_fused_rmsnorm_quant_regs<ScaleF32, 14, true>", False) == ("fused_rmsnorm_quant", None)
    assert api_of("k_dispatch_gather_scales<ScaleF32>", False) == ("quant_dispatch_1x128", None)


def test_gemm_kernels_and_their_reductions():
    assert api_of("k_gemm_fp8_bs[192x256,exact]", False) == ("gemm_fp8_blockscaled", "exact")
    assert api_of("k_gemm_fp8_bs_tail[256x256,fp8core]", False) == ("gemm_fp8_blockscaled", "fp8core")
    assert api_of("k_grouped_gemm_fp8_bs[128x128,exact]", False) == ("grouped_gemm_fp8_blockscaled", "exact")
    assert api_of("k_gemm_fused_a[128x256,exact,emit]", False) == ("gemm_bf16a_fp8_blockscaled", "exact")
    # the split-K reduction carries no mode: both modes' calls include it
    assert api_of("k_splitk_reduce", True) == ("gemm_fp8_e8m0", None)
    assert api_of("k_tail_reduce<TileCfg<192, 256, 2, 4, 2, false> >", False) == ("gemm_fp8_blockscaled", "exact")
    assert api_of("k_tail_reduce<TileCfg<256, 256, 2, 4, 2, false> >", False) == ("gemm_fp8_blockscaled", "fp8core")
    assert api_of("k_tail_reduce<TileCfg<256, 256, 2, 4, 2, false> >", True) == ("gemm_fp8_e8m0", "promote")
    assert api_of("k_tail_reduce<TileCfg<256, 256, 4, 4, 2, false> >", True) == ("gemm_fp8_e8m0", "incore")
    assert api_of("__amd_rocclr_copyBuffer", False) == (None, None)
