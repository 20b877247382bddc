"""The error bounds that the FP8-matrix-core GEMM tests widen their
elementwise check by: the all-outputs form must dominate the per-group form
it loosens, and both must cover a product whose groups are truncated as the
bound assumes.  CPU only."""
import numpy as np

import oracle
from tests.test_gpu_gemm import fp8_core_slack, fp8_core_slack_all


def _codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E     # no NaN codes
    return c


def test_all_outputs_bound_dominates_the_per_group_bound():
    rng = np.random.default_rng(11)
    M, N, K = 24, 256, 384
    qa, qw = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.uniform(0.5, 2, (M, K // 128))
    sw = rng.uniform(0.5, 2, (N // 128, K // 128))
    rows, cols = np.arange(M), np.arange(N)
    tight = fp8_core_slack(qa, sa, qw, sw, rows, cols)
    loose = fp8_core_slack_all(qa, sa, qw, sw)
    assert loose.shape == tight.shape
    assert np.all(loose >= tight * (1 - 1e-12))
    # equal when each group holds one nonzero code on both sides at the same
    # position (then max |a| * max |w| is the group's only product)
    qa1 = np.zeros((M, K), np.uint8)
    qw1 = np.zeros((N, K), np.uint8)
    qa1[:, ::8] = qa[:, ::8]
    qw1[:, ::8] = qw[:, ::8]
    assert np.allclose(fp8_core_slack_all(qa1, sa, qw1, sw), fp8_core_slack(qa1, sa, qw1, sw, rows, cols),
                       rtol=1e-12, atol=0)


def test_bounds_cover_a_group_truncated_to_its_window():
    # one output whose 8-product groups each lose everything below 12 bits of
    # the group's largest product: the loss stays within both bounds
    rng = np.random.default_rng(12)
    K = 256
    qa, qw = _codes(rng, (1, K)), _codes(rng, (1, K))
    a = oracle.e4m3_decode(qa).astype(np.float64)[0]
    w = oracle.e4m3_decode(qw).astype(np.float64)[0]
    p = (a * w).reshape(-1, 8)
    exact = p.sum()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(p).max(axis=1), 1e-300))) - 12)
    trunc = (np.trunc(p.sum(axis=1) / ulp) * ulp).sum()
    sa, sw = np.ones((1, K // 128)), np.ones((1, K // 128))
    assert abs(trunc - exact) <= fp8_core_slack(qa, sa, qw, sw, [0], [0])[0, 0]
    assert abs(trunc - exact) <= fp8_core_slack_all(qa, sa, qw, sw)[0, 0]
