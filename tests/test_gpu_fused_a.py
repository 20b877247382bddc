"""GPU parity of the GEMM with the activation quantisation fused into its
A-load (fgq_gemm_bf16a_fp8_blockscaled).

  * bit-identical to fgq_quant_act_1x128 followed by fgq_gemm_fp8_blockscaled
    in the same mode (each output's arithmetic depends only on its row, its
    column and the chunk order, and both calls use the same split plan): the
    dense large-tile path, the small-tile path and split-K, ragged M, a padded
    row stride;
  * the emitted codes and scales are byte-identical to the oracle's 1x128
    quantisation, in row-major and K-block-major scale layouts, with guard
    bands; emitting does not change C;
  * the tolerance gate against the oracle on the tiny, decode and prefill
    workloads, and the full prefill size on sampled rows.
"""
import numpy as np
import pytest

import oracle
from synth import make_workload, normal_bf16, rng_for
from tests.gpu_util import Guarded, dev_bf16, dev_f32, dev_u8, host_bf16_f64, log
from tests.test_gpu_gemm import _check

pytestmark = pytest.mark.gpu

MODES = [0, 1]


def _bf16_padded(bits, ld):
    M, K = bits.shape
    if ld is None or ld == K:
        return dev_bf16(bits)
    pad = np.zeros((M, ld), np.uint16)
    pad[:, :K] = bits
    return dev_bf16(pad)[:, :K]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,K,lda", [(1, 128, 128, None), (129, 256, 384, None), (300, 384, 1024, 1040),
                                       (64, 18432, 7168, None), (513, 768, 512, None), (255, 640, 2048, None),
                                       (384, 18432, 7168, None)])
def test_fused_equals_quant_then_gemm(fgq_gpu, M, N, K, lda, mode):
    import torch
    log(f"fused A-load GEMM {M}x{N}x{K} lda={lda} mode={mode}")
    a = normal_bf16((M, K), 1.0, rng_for(30, M + K))
    w = normal_bf16((N, K), 0.02, rng_for(30, N))
    a_d = _bf16_padded(a, lda)
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(w))
    qa, sa = fgq_gpu.quant_act_1x128(a_d)
    c_sep = fgq_gpu.gemm_fp8_blockscaled(qa, sa, qw, sw, mode=mode)
    cg = Guarded(M, N, torch.bfloat16)
    fgq_gpu.gemm_bf16a_fp8_blockscaled(a_d, qw, sw, out=cg.view, mode=mode)
    torch.cuda.synchronize()
    cg.check_canaries()
    assert torch.equal(cg.view.view(torch.int16), c_sep.view(torch.int16))


@pytest.mark.parametrize("kmajor", [False, True])
@pytest.mark.parametrize("M,N,K", [(129, 256, 384), (64, 18432, 7168), (300, 512, 2048)])
def test_fused_emits_the_quantisation(fgq_gpu, M, N, K, kmajor):
    """Codes and scales written by the GEMM equal the oracle's 1x128
    quantisation byte for byte; C equals the non-emitting call's."""
    import torch
    a = normal_bf16((M, K), 1.0, rng_for(31, M))
    w = normal_bf16((N, K), 0.02, rng_for(31, N))
    a_d = dev_bf16(a)
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(w))
    qg = Guarded(M, K, torch.uint8)
    if kmajor:
        sg = Guarded(K // 128, M, torch.float32)
        s_view = sg.view.t()
    else:
        sg = Guarded(M, K // 128, torch.float32)
        s_view = sg.view
    c_emit = fgq_gpu.gemm_bf16a_fp8_blockscaled(a_d, qw, sw, qa_out=qg.view, sa_out=s_view)
    c_plain = fgq_gpu.gemm_bf16a_fp8_blockscaled(a_d, qw, sw)
    torch.cuda.synchronize()
    qg.check_canaries()
    sg.check_canaries()
    qo, so = oracle.quant_act_1x128(a)
    assert np.array_equal(qg.view.cpu().numpy(), qo)
    assert np.array_equal(s_view.cpu().numpy().view(np.uint32), so.view(np.uint32))
    assert torch.equal(c_emit.view(torch.int16), c_plain.view(torch.int16))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("name,rows", [("tiny", None), ("decode", None), ("prefill", 384)])
def test_fused_workloads_gate(fgq_gpu, name, rows, mode):
    import torch
    d = make_workload(name, rows=rows)
    qwo, swo = oracle.quant_w_128x128(d["W"])
    c = fgq_gpu.gemm_bf16a_fp8_blockscaled(dev_bf16(d["A"]), dev_u8(qwo), dev_f32(swo), mode=mode)
    torch.cuda.synchronize()
    qao, sao = oracle.quant_act_1x128(d["A"])
    _check(host_bf16_f64(c), oracle.gemm_ref(qao, sao, qwo, swo), f"fused {name}", mode, qao, sao, qwo, swo)


@pytest.mark.parametrize("mode", MODES)
def test_fused_prefill_full_size_sampled(fgq_gpu, mode):
    """8192 x 18432 x 7168 from BF16 activations in one call; 128 sampled rows
    against the oracle's quantisation and product."""
    import torch
    d = make_workload("prefill")
    A, W = d["A"], d["W"]
    qw, sw = fgq_gpu.quant_w_128x128(dev_bf16(W))
    c = fgq_gpu.gemm_bf16a_fp8_blockscaled(dev_bf16(A), qw, sw, mode=mode)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(6).choice(A.shape[0], 128, replace=False))
    rows[0], rows[-1] = 0, A.shape[0] - 1
    qao, sao = oracle.quant_act_1x128(A[rows])
    qwo, swo = oracle.quant_w_128x128(W)
    _check(host_bf16_f64(c[rows.tolist()]), oracle.gemm_ref(qao, sao, qwo, swo), "fused prefill full (sampled rows)",
           mode, qao, sao, qwo, swo)
