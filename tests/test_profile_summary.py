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


def _write_csv(path, header, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_timed_dispatches_are_those_between_the_markers(tmp_path):
    from fine_grained_fp8_quant_amd.profile_summary import read_trace_timed
    hdr = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [[1, "void fgq::k_quant_act_1x128<fgq::ScaleF32>(int)", 0, 5000],
            [2, "void fgq::k_debug_copy(int)", 6000, 7000],
            [4, "void fgq::k_quant_act_1x128<fgq::ScaleF32>(int)", 9000, 12000],
            [3, "void fgq::k_quant_w_128x128<fgq::ScaleF32, false>(int)", 8000, 8500],
            [5, "void fgq::k_debug_copy(int)", 13000, 14000],
            [6, "void fgq::k_quant_act_1x128<fgq::ScaleF32>(int)", 15000, 99000]]
    _write_csv(tmp_path / "t.csv", hdr, rows)
    got = read_trace_timed(tmp_path / "t.csv")
    assert got == [("k_quant_w_128x128<ScaleF32, false>", 0.5), ("k_quant_act_1x128<ScaleF32>", 3.0)]
    _write_csv(tmp_path / "u.csv", hdr, rows[:2])
    assert read_trace_timed(tmp_path / "u.csv") is None


def test_utilisation_ratios(tmp_path):
    from fine_grained_fp8_quant_amd.profile_summary import read_counters, util_metrics
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    k = "void fgq::k_gemm_fp8_bs<fgq::TileCfg<192, 256, 2, 4, 2, false>, 0>(int)"
    # 1 ms at 2 GHz on every XCD: 2e6 cycles each, 1.6e7 summed
    util = [[7, k, "GRBM_GUI_ACTIVE", 1.6e7, 0, 1_000_000], [7, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 1e6, 0, 1_000_000],
            [7, k, "SQ_VALU_MFMA_COEXEC_CYCLES", 256 * 1e6, 0, 1_000_000], [7, k, "SQ_INSTS_MFMA", 100, 0, 1_000_000],
            [7, k, "SQ_INSTS_VALU", 250, 0, 1_000_000], [7, k, "SQ_INSTS_LDS", 30, 0, 1_000_000]]
    l2 = [[7, k, "GRBM_GUI_ACTIVE", 1.6e7, 0, 1_000_000], [7, k, "TCC_HIT_sum", 3, 0, 1_000_000],
          [7, k, "TCC_MISS_sum", 1, 0, 1_000_000]]
    _write_csv(tmp_path / "util.csv", hdr, util)
    _write_csv(tmp_path / "l2.csv", hdr, l2)
    m = util_metrics({"util": read_counters(tmp_path / "util.csv"), "l2": read_counters(tmp_path / "l2.csv")})
    got = m["k_gemm_fp8_bs[192x256,exact]"]
    assert abs(got["clock GHz"] - 2.0) < 1e-12
    assert abs(got["MFMA busy"] - 0.5) < 1e-12
    assert abs(got["co-issue / MFMA busy"] - 0.25) < 1e-12
    assert abs(got["VALU inst / MFMA inst"] - 2.5) < 1e-12
    assert abs(got["L2 hit"] - 0.75) < 1e-12


def test_call_spans_group_consecutive_kernels_of_one_call():
    from fine_grained_fp8_quant_amd.profile_summary import call_spans
    timed = [("k_quant_act_1x128<ScaleF32>", 0.0, 3.0),
             ("k_gemm_fp8_bs_splitk[64x128,exact]", 4.0, 34.0), ("k_splitk_reduce", 38.0, 42.0),
             ("k_quant_act_1x128<ScaleF32>", 50.0, 53.0),
             ("k_gemm_fp8_bs_splitk[64x128,exact]", 54.0, 84.0), ("k_splitk_reduce", 86.0, 90.0)]
    sp = call_spans(timed, False, "exact")
    assert sp["gemm_fp8_blockscaled[exact]"] == 37.0  # (42 - 4 + 90 - 54) / 2
    assert sp["quant_act_1x128"] == 3.0


def test_call_gaps_split_edges_of_the_target_call_from_the_rest():
    from fine_grained_fp8_quant_amd.profile_summary import call_gaps
    timed = [("k_quant_act_1x128<ScaleF32>", 0.0, 3.0),
             ("k_gemm_fp8_bs_splitk[64x128,exact]", 8.0, 34.0), ("k_splitk_reduce", 34.0, 42.0),
             ("k_quant_act_1x128<ScaleF32>", 46.0, 49.0), ("k_quant_w_128x128<ScaleF32, false>", 50.0, 60.0),
             ("k_gemm_fp8_bs_splitk[64x128,exact]", 66.0, 84.0), ("k_splitk_reduce", 84.0, 90.0)]
    before, after, other = call_gaps(timed, False, "exact", "gemm_fp8_blockscaled[exact]")
    assert before == 5.5      # (8 - 3 + 66 - 60) / 2
    assert after == 4.0       # 46 - 42
    assert other == 1.0       # 50 - 49; the gaps inside the call are not counted
    assert call_gaps(timed[:1], False, "exact", "gemm_fp8_blockscaled[exact]") == (None, None, None)
