"""Pins for the oracle's power-of-two (E8M0) scale variant (CPU only).

Independent of the oracle's own arithmetic:
  * E8M0 decode against the OCP MX specification's points, and the scale
    exponent against hand-derived points (tests/golden/e8m0_points.txt);
  * the exponent against exact integer arithmetic for every positive finite
    BF16 value, and against a full enumeration of e = -127 .. 128 for
    random binary32 values;
  * a worked tile, with codes derived by hand;
  * codes against a brute-force nearest-value search over the E4M3 grid,
    ties to the even code (tiles with outliers, subnormal-only tiles, zeros);
  * agreement with the binary32-scale quantiser wherever the max-abs is
    448 * 2^k, where both rules give the same scale and the same codes;
  * planted per-block maxima pin the 128x128 block indexing;
  * the GEMM reference against an exact integer evaluation of the chunk
    sums times the power-of-two scales.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import (e4m3_decode, e8m0_decode, e8m0_exponent, fused_rmsnorm_quant_e8m0, gemm_e8m0_ref,
                    grouped_gemm_e8m0_ref, quant_act_1x128, quant_act_1x128_e8m0, quant_w_128x128_e8m0,
                    rmsnorm_r64)
from synth import bf16_bits_from_f32, normal_bf16, rng_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e8m0_points.txt")


def _golden(kind):
    out = []
    with open(GOLDEN) as f:
        for line in f:
            parts = line.split()
            if parts and parts[0] == kind:
                out.append(parts[1:3])
    return out


def test_decode_spec_points():
    pts = _golden("decode")
    assert len(pts) == 8
    for byte, value in pts:
        got = e8m0_decode(np.array([int(byte, 16)], np.uint8))[0]
        if value == "nan":
            assert np.isnan(got)
        else:
            assert got == float(value), (byte, got, value)


def test_exponent_hand_points():
    pts = _golden("exponent")
    assert len(pts) == 17
    for a, byte in pts:
        av = float(a)
        assert float(np.float32(av)) == av, f"{a} is not a binary32 value"
        got = int(e8m0_exponent(np.array([av]))[0]) + 127
        assert got == int(byte), (a, got, byte)


def _exponent_exact(a: float) -> int:
    """Smallest e in [-127, 128] with 448 * 2^e >= a, by exact integer
    comparisons (a = num / den) and bisection over the monotone predicate."""
    num, den = Fraction(a).as_integer_ratio()

    def ok(e):
        return 448 * den * 2 ** e >= num if e >= 0 else 448 * den >= num * 2 ** (-e)
    lo, hi = -127, 128
    if ok(lo):
        return lo
    while hi - lo > 1:        # ok(hi) holds, ok(lo) does not
        mid = (lo + hi) // 2
        if ok(mid):
            hi = mid
        else:
            lo = mid
    return hi


def test_exponent_every_bf16():
    bits = np.arange(1, 0x7F80, dtype=np.uint32)          # every positive finite BF16
    a = (bits << np.uint32(16)).view(np.float32)
    got = e8m0_exponent(a)
    want = np.array([_exponent_exact(float(v)) for v in a], dtype=np.int64)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(a[i]), int(got[i]), int(want[i])) for i in bad[:5]]


def test_exponent_random_binary32_enumeration():
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 0x7F800000, size=200_000, dtype=np.uint32)   # positive finite binary32
    a = bits.view(np.float32).astype(np.float64)
    es = np.arange(-127, 129)
    ok = np.ldexp(448.0, es)[:, None] >= a[None, :]        # [256, n]
    want = es[np.argmax(ok, axis=0)]
    assert np.array_equal(e8m0_exponent(a), want)


def test_worked_tile():
    # max-abs 3 -> e = -7 (448/128 = 3.5 >= 3 > 1.75), byte 120; the cast
    # multiplies by 2^7: 3 -> 384 = 1.5 * 2^8 (0x7C), -1 -> -128 = -2^7
    # (0xF0), 0.5 -> 64 = 2^6 (0x68), 2^-7 -> 1 (0x38), 2^-17 -> 2^-10, a tie
    # between 0 and the smallest subnormal 2^-9 -> 0 (0x00), -0 -> 0x80,
    # 0.01 (BF16 0.010009765625) -> 1.28125 = 1.25 + 1/32, between 1.25 and
    # 1.375 -> 1.25 (0x3A).  The binary32-scale rule would map 3 onto 448.
    vals = [3.0, -1.0, 0.5, 2.0 ** -7, 2.0 ** -17, -0.0, 0.010009765625] + [0.0] * 121
    x = bf16_bits_from_f32(np.array(vals, np.float32))[None, :]
    q, b = quant_act_1x128_e8m0(x)
    assert int(b[0, 0]) == 120
    assert q[0, :7].tolist() == [0x7C, 0xF0, 0x68, 0x38, 0x00, 0x80, 0x3A]
    qf, sf = quant_act_1x128(x)
    assert qf[0, 0] == 0x7E and sf[0, 0] == np.float32(3.0) / np.float32(448.0)


_GRID = e4m3_decode(np.arange(0x7F, dtype=np.uint8))      # codes 0x00 .. 0x7E, non-negative


def _nearest_codes(y: np.ndarray, neg: np.ndarray) -> np.ndarray:
    """Brute force: the non-negative E4M3 code nearest to |y| (ties to the even
    code), with the sign bit taken from ``neg``."""
    d = np.abs(_GRID[None, :] - np.abs(y)[:, None])
    dmin = d.min(axis=1, keepdims=True)
    tie = d == dmin
    # among tied codes prefer an even one (there are at most two, adjacent)
    codes = np.arange(0x7F)[None, :]
    pick = np.where(tie & (codes % 2 == 0), codes, 1000).min(axis=1)
    pick = np.where(pick == 1000, np.argmax(tie, axis=1), pick)
    return (pick | (neg.astype(np.int64) << 7)).astype(np.uint8)


def _check_tiles(x_f32: np.ndarray, q: np.ndarray, b: np.ndarray):
    """x_f32 [G, 128] groups, q [G, 128] codes, b [G] bytes."""
    a = np.max(np.abs(x_f32.astype(np.float64)), axis=1)
    e = b.astype(np.int64) - 127
    # the scale rule, stated as inequalities
    assert np.all(np.ldexp(448.0, e) >= a)
    assert np.all((e == -127) | (np.ldexp(448.0, e - 1) < a))
    y = x_f32.astype(np.float64) * np.ldexp(1.0, -e)[:, None]
    neg = np.signbit(x_f32)
    want = _nearest_codes(y.ravel(), neg.ravel()).reshape(q.shape)
    assert np.array_equal(q, want)


def test_codes_nearest_brute_force():
    rng = rng_for(5, 70)
    x = normal_bf16((24, 512), 1.0, rng)
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).copy()
    xf[0, 3] = 250.0                 # outlier
    xf[1, :128] = 0.0                # all-zero tile
    xf[2, :128] = np.ldexp(np.float32(1.0), -133) * rng.integers(-3, 4, size=128)   # subnormal-only tile
    xf[3, 128:256] *= np.float32(1e30)                                               # huge tile
    xf[4, :] = -xf[4, :]
    x = bf16_bits_from_f32(xf)
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    q, b = quant_act_1x128_e8m0(x)
    _check_tiles(xf.reshape(-1, 128), q.reshape(-1, 128), b.reshape(-1))
    assert b[1, 0] == 0 and np.all((q[1, :128] & 0x7F) == 0)


def test_matches_binary32_rule_on_power_of_two_maxima():
    """Where a = 448 * 2^k the binary32 scale a/448 = 2^k is exact, 448/a =
    2^-k is exact, and both rules give the same codes."""
    rng = rng_for(6, 70)
    x = normal_bf16((16, 1024), 1.0, rng)
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(16, 8, 128).copy()
    xf = np.clip(xf, -3.0, 3.0)
    for m in range(16):
        for kb in range(8):
            k = int(rng.integers(-20, 20))
            xf[m, kb] *= np.float32(2.0 ** (k + 7))       # now |values| <= 384 * 2^k < 448 * 2^k
            xf[m, kb, int(rng.integers(128))] = np.float32(448.0 * 2.0 ** k) * (1 if rng.random() < .5 else -1)
    x = bf16_bits_from_f32(xf.reshape(16, 1024))
    q8, b8 = quant_act_1x128_e8m0(x)
    qf, sf = quant_act_1x128(x)
    assert np.array_equal(q8, qf)
    assert np.array_equal(e8m0_decode(b8), sf.astype(np.float64))


def test_weight_block_indexing():
    B, N, K = 2, 256, 384
    w = np.zeros((B, N, K), np.float32)
    for b in range(B):
        for nb in range(N // 128):
            for kb in range(K // 128):
                w[b, nb * 128 + (b * 7 + kb * 5) % 128, kb * 128 + (nb * 11) % 128] = 448.0 * 2.0 ** (b + 2 * nb + 3 * kb)
    q, s = quant_w_128x128_e8m0(bf16_bits_from_f32(w))
    for b in range(B):
        for nb in range(N // 128):
            for kb in range(K // 128):
                assert int(s[b, nb, kb]) == 127 + b + 2 * nb + 3 * kb
    assert np.count_nonzero(q == 0x7E) == B * (N // 128) * (K // 128)
    # unbatched form
    q1, s1 = quant_w_128x128_e8m0(bf16_bits_from_f32(w[1]))
    assert np.array_equal(q1, q[1]) and np.array_equal(s1, s[1])


def test_fused_rmsnorm_e8m0_codes():
    rng = rng_for(7, 70)
    x = normal_bf16((6, 640), 2.0, rng)
    g = normal_bf16((640,), 1.0, rng)
    q, b = fused_rmsnorm_quant_e8m0(x, g, 1e-6)
    y = rmsnorm_r64(x, g, 1e-6)          # pinned in test_oracle_quant
    _check_tiles(y.reshape(-1, 128), q.reshape(-1, 128), b.reshape(-1))


def test_gemm_ref_exact_integer_sums():
    """Every E4M3 value is an integer times 2^-9, every scale a power of two:
    the chunk sums are exact integers and the result is exact up to float64
    rounding of the final sum."""
    rng = np.random.default_rng(9)
    M, N, K = 3, 128, 384
    qa = rng.integers(0, 256, size=(M, K)).astype(np.uint8)
    qw = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x3C
    qw[(qw & 0x7F) == 0x7F] = 0xB5
    ba = rng.integers(110, 140, size=(M, K // 128)).astype(np.uint8)
    bw = rng.integers(110, 140, size=(N // 128, K // 128)).astype(np.uint8)
    ia = np.rint(e4m3_decode(qa) * 512).astype(np.int64)      # exact integers
    iw = np.rint(e4m3_decode(qw) * 512).astype(np.int64)
    ref = gemm_e8m0_ref(qa, ba, qw, bw)
    for m in range(M):
        for n in range(N):
            tot, mag = Fraction(0), Fraction(0)
            for kb in range(K // 128):
                sl = slice(kb * 128, (kb + 1) * 128)
                sc = Fraction(2) ** (int(ba[m, kb]) + int(bw[n // 128, kb]) - 254 - 18)
                tot += int(np.dot(ia[m, sl], iw[n, sl])) * sc
                mag += int(np.dot(np.abs(ia[m, sl]), np.abs(iw[n, sl]))) * sc
            # float64 evaluation of a 384-term sum: error <= 384 * 2^-53 * sum |terms|
            assert abs(Fraction(ref[m, n]) - tot) <= mag * Fraction(1, 2 ** 43)


def test_grouped_ref_uses_each_experts_scales():
    rng = np.random.default_rng(10)
    E, N, K = 3, 128, 256
    offsets = np.array([0, 2, 2, 5])
    qa = rng.integers(0, 0x70, size=(5, K)).astype(np.uint8)
    qw = rng.integers(0, 0x70, size=(E, N, K)).astype(np.uint8)
    ba = rng.integers(120, 135, size=(5, K // 128)).astype(np.uint8)
    bw = np.stack([np.full((1, K // 128), 127 + 3 * e, np.uint8) for e in range(E)])
    out = grouped_gemm_e8m0_ref(qa, ba, qw, bw, offsets)
    for e in range(E):
        r0, r1 = offsets[e], offsets[e + 1]
        if r1 > r0:
            unit = gemm_e8m0_ref(qa[r0:r1], ba[r0:r1], qw[e], np.full((1, K // 128), 127, np.uint8))
            np.testing.assert_array_equal(out[r0:r1], unit * 2.0 ** (3 * e))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -1.0])
def test_exponent_rejects_outside_contract(bad):
    with pytest.raises(ValueError):
        e8m0_exponent(np.array([bad]))
