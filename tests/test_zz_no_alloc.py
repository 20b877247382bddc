"""The no-allocation GEMM entry point (fgq_gemm_fp8_blockscaled_noalloc)
against fgq_gemm_fp8_blockscaled: two calls in a row, the second on a smaller
input, each bit-identical to the entry point that takes a workspace (the two
run the same kernels on the same split plan)."""
import numpy as np
import pytest

from synth import normal_bf16, rng_for
from tests.gpu_util import dev_bf16, log

pytestmark = pytest.mark.gpu


def _operands(fgq, M, N, K, seed):
    a = normal_bf16((M, K), 1.0, rng_for(seed, 900))
    w = normal_bf16((N, K), 0.02, rng_for(seed, 901))
    qa, sa = fgq.quant_act_1x128(dev_bf16(a))
    qw, sw = fgq.quant_w_128x128(dev_bf16(w))
    return qa, sa, qw, sw


# (first, second) shapes: a split along K (scratch holds the partial sums),
# then a smaller split; a large product whose last round is split along K,
# then a smaller plain one
@pytest.mark.parametrize("shapes", [((64, 4096, 7168), (33, 2048, 2048)),
                                    ((2112, 6144, 2560), (1000, 2048, 1024))])
@pytest.mark.parametrize("mode", [0, 1])
def test_noalloc_matches_workspace_entry_point(fgq_gpu, shapes, mode):
    import torch
    for i, (M, N, K) in enumerate(shapes):
        log(f"noalloc call {i}: M={M} N={N} K={K} mode={mode}")
        qa, sa, qw, sw = _operands(fgq_gpu, M, N, K, seed=10 * i + mode)
        want = fgq_gpu.gemm_fp8_blockscaled(qa, sa, qw, sw, mode=mode)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = fgq_gpu.gemm_fp8_blockscaled_noalloc(qa, sa, qw, sw, out, mode=mode)
        torch.cuda.synchronize()
        assert got is out
        assert np.array_equal(got.view(torch.int16).cpu().numpy(), want.view(torch.int16).cpu().numpy()), (M, N, K)
