"""Pins for the oracle's block-scaled GEMM, its grouped variant and the gate (CPU only).

  * brute force: a pure-Python triple loop with exactly rounded sums
    (math.fsum), decoding codes through torch's float8_e4m3fn (a library
    routine), on tiny shapes;
  * closed form: integer-valued codes and power-of-two scales make every
    product and sum an exact integer multiple of a power of two, checked
    against int64 arithmetic at K = 7168;
  * one-hot rows with distinct per-(row, group) and per-(block, group)
    scales pin the scale indexing (a transposed scale index fails);
  * the grouped variant against the brute force per expert, with empty
    experts, and against the dense GEMM when there is one expert;
  * the tolerance gate accepts a BF16-rounded reference and rejects
    planted errors.
"""
import math

import numpy as np
import pytest

from oracle import (bf16_round_f64, dequant_act, dequant_w, e4m3_decode, gemm_gate, gemm_ref,
                    grouped_gemm_ref, quant_act_1x128, quant_w_128x128)
from synth import normal_bf16, rng_for

torch = pytest.importorskip("torch")


def _torch_dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).float().double().numpy()


def _brute(qa, sa, qw, sw):
    av = _torch_dec(qa)
    wv = _torch_dec(qw)
    M, K = qa.shape
    N = qw.shape[0]
    out = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            terms = [float(av[m, k]) * float(sa[m, k // 128]) * float(wv[n, k]) * float(sw[n // 128, k // 128])
                     for k in range(K)]
            out[m, n] = math.fsum(terms)
    return out


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (3, 256, 256), (17, 128, 384)])
def test_gemm_matches_bruteforce(M, N, K):
    a = normal_bf16((M, K), 1.0, rng_for(1, 1000 + M))
    w = normal_bf16((N, K), 0.02, rng_for(1, 2000 + N))
    qa, sa = quant_act_1x128(a)
    qw, sw = quant_w_128x128(w)
    got = gemm_ref(qa, sa, qw, sw)
    want = _brute(qa, sa, qw, sw)
    # float64 BLAS vs exactly rounded sums: relative to the largest |term| sum
    assert np.all(np.abs(got - want) <= 1e-13 * np.abs(want).max())


def test_gemm_integer_codes_exact():
    """Codes of integers -8..8 and power-of-two scales: the exact result is an
    integer sum times powers of two, which int64 computes exactly."""
    rng = np.random.default_rng(3)
    M, N, K = 32, 256, 7168
    ints = np.arange(-8, 9)
    # E4M3 codes of the integers (from the format: 1.0 = 0x38, each doubling +8)
    code_of = {0: 0x00}
    for v in range(1, 9):
        e = int(math.floor(math.log2(v)))
        m = int((v / 2 ** e - 1) * 8)
        code_of[v] = ((e + 7) << 3) | m
        code_of[-v] = code_of[v] | 0x80
    ia = rng.choice(ints, size=(M, K))
    iw = rng.choice(ints, size=(N, K))
    qa = np.vectorize(code_of.get)(ia).astype(np.uint8)
    qw = np.vectorize(code_of.get)(iw).astype(np.uint8)
    assert np.array_equal(e4m3_decode(qa), ia.astype(np.float64))
    ea = rng.integers(-1, 2, size=(M, K // 128))
    ew = rng.integers(-1, 2, size=(N // 128, K // 128))
    sa = (2.0 ** ea).astype(np.float32)
    sw = (2.0 ** ew).astype(np.float32)
    # exact: scale every chunk product to a common 2**-2 grid with int64
    want = np.zeros((M, N), dtype=np.int64)
    for kb in range(K // 128):
        part = ia[:, 128 * kb:128 * kb + 128].astype(np.int64) @ iw[:, 128 * kb:128 * kb + 128].astype(np.int64).T
        sh = ea[:, kb][:, None] + np.repeat(ew[:, kb], 128)[None, :] + 2     # >= 0
        want += part << sh
    got = gemm_ref(qa, sa, qw, sw)
    assert np.array_equal(got, want.astype(np.float64) / 4.0)


def test_gemm_one_hot_pins_scale_indexing():
    M, N, K = 5, 256, 512
    qa = np.zeros((M, K), np.uint8)
    qw = np.zeros((N, K), np.uint8)
    rng = np.random.default_rng(4)
    ks = rng.integers(0, K, size=M)
    for m in range(M):
        qa[m, ks[m]] = 0x38           # 1.0
    qw[:, :] = 0x40                   # 2.0 everywhere
    sa = (np.arange(M * 4).reshape(M, 4) + 1).astype(np.float32)
    sw = (np.arange(8).reshape(2, 4) * 10 + 100).astype(np.float32)
    got = gemm_ref(qa, sa, qw, sw)
    for m in range(M):
        kb = ks[m] // 128
        for n in range(N):
            assert got[m, n] == 1.0 * sa[m, kb] * 2.0 * sw[n // 128, kb]
    # the transposed weight-scale index would give different values
    assert not np.allclose(sw, sw[:, ::-1])


def test_dequant_shapes_and_k128():
    a = normal_bf16((4, 128), 1.0, rng_for(2, 1))
    w = normal_bf16((128, 128), 0.02, rng_for(2, 2))
    qa, sa = quant_act_1x128(a)
    qw, sw = quant_w_128x128(w)
    assert dequant_act(qa, sa).shape == (4, 128) and dequant_w(qw, sw).shape == (128, 128)
    assert np.allclose(gemm_ref(qa, sa, qw, sw), _brute(qa, sa, qw, sw), rtol=1e-14, atol=1e-14)


def test_grouped_matches_bruteforce_with_empty_experts():
    E, N, K = 4, 128, 256
    counts = np.array([3, 0, 5, 0])
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    R = int(off[-1])
    a = normal_bf16((R, K), 1.0, rng_for(3, 1))
    w = normal_bf16((E, N, K), 0.02, rng_for(3, 2))
    qa, sa = quant_act_1x128(a)
    qw, sw = quant_w_128x128(w)
    got = grouped_gemm_ref(qa, sa, qw, sw, off)
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            want = _brute(qa[r0:r1], sa[r0:r1], qw[e], sw[e])
            assert np.allclose(got[r0:r1], want, rtol=1e-14, atol=1e-14 * np.abs(want).max())
    assert got.shape == (R, N)


def test_grouped_single_expert_is_dense():
    a = normal_bf16((37, 256), 1.0, rng_for(4, 1))
    w = normal_bf16((1, 256, 256), 0.02, rng_for(4, 2))
    qa, sa = quant_act_1x128(a)
    qw, sw = quant_w_128x128(w)
    g = grouped_gemm_ref(qa, sa, qw, sw, np.array([0, 37], np.int32))
    assert np.array_equal(g, gemm_ref(qa, sa, qw[0], sw[0]))


def test_grouped_all_rows_empty():
    qw = np.zeros((2, 128, 128), np.uint8)
    sw = np.ones((2, 1, 1), np.float32)
    g = grouped_gemm_ref(np.zeros((0, 128), np.uint8), np.zeros((0, 1), np.float32), qw, sw,
                         np.array([0, 0, 0], np.int32))
    assert g.shape == (0, 128)


def test_bf16_round_f64():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -3.0 - 2 ** -7 - 2 ** -9, 0.0, 2.0 ** -100])
    # 1+2^-8 ties to 1.0 (even mantissa); 1+3*2^-8 ties up to 1+2^-6 (even);
    # near 3 the BF16 spacing is 2^-6 and 2^-7 + 2^-9 is 0.625 of it: rounds away from 3.
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, -3.0 - 2 ** -6, 0.0, 2.0 ** -100])
    assert np.array_equal(bf16_round_f64(x), want)
    t = torch.from_numpy(np.random.default_rng(0).standard_normal(100000)).float()
    assert np.array_equal(bf16_round_f64(t.double().numpy()), t.bfloat16().double().numpy())


def test_gate_accepts_bf16_rounding_and_rejects_planted_errors():
    rng = np.random.default_rng(6)
    ref = rng.standard_normal((64, 512))
    c = bf16_round_f64(ref)
    g = gemm_gate(c, ref)
    assert g["ok"] and g["normwise"] < 2e-3
    bad = ref * (1 + 3e-3)
    assert not gemm_gate(bad, ref)["ok"]
    bad2 = c.copy()
    big = np.argmax(np.abs(ref))
    bad2.flat[big] *= 1.02
    assert not gemm_gate(bad2, ref)["ok"]
    bad3 = c.copy()
    bad3[3, 3] = np.nan
    assert not gemm_gate(bad3, ref)["ok"]
    # elements below 1e-2 * rms are not gated elementwise
    small = c.copy()
    tiny = np.argmin(np.abs(ref))
    small.flat[tiny] += 1e-3 * np.sqrt(np.mean(ref ** 2))
    assert gemm_gate(small, ref)["ok"]
