"""Pins for the oracle's 1x128 / 128x128 quantisation and fused RMSNorm (CPU only).

Independent of the oracle's own arithmetic:
  * scales against exact rational arithmetic (fractions.Fraction) rounded
    to binary32 by an exact nearest-value choice;
  * exact round trip of tiles already representable in E4M3 (times 2**k);
  * the max-abs element of every non-zero group encodes to +-448;
  * all-zero groups: scale 0, codes +-0, no NaN;
  * the E4M3 error bound on random data with outliers;
  * planted per-block maxima pin the 128x128 block indexing;
  * the fused RMSNorm: closed form on constant rows, and agreement with a
    float64 RMSNorm within its binary32 forward-error bound on random rows (including a ragged lane tail);
  * its summation order: crafted rows whose hand-derived binary32 sums of
    squares differ from a sequential sum, contiguous per-partial vectors, a
    reversed butterfly, a fused multiply-add accumulation and a reversed
    vector order within a partial.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import (e4m3_decode, fused_rmsnorm_quant, f32_from_bf16, quant_act_1x128,
                    quant_w_128x128, rmsnorm_r64, sum_squares_r64)
from synth import bf16_bits_from_f32, normal_bf16, rng_for


def round_f32(fr: Fraction) -> np.float32:
    """Nearest binary32 to an exact rational, ties to even (normal range)."""
    if fr == 0:
        return np.float32(0.0)
    neg = fr < 0
    fr = abs(fr)
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]

    def key(v):
        return (abs(Fraction(float(v)) - fr), int(np.float32(v).view(np.uint32)) & 1)
    best = min(cands, key=key)
    return np.float32(-best if neg else best)


def sqrt_f32(v: np.float32) -> np.float32:
    """Correctly rounded binary32 square root, by exact comparison of squares."""
    fr = Fraction(float(v))
    c = np.float32(math.sqrt(float(v)))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
    return min(cands, key=lambda x: (abs(Fraction(float(x)) ** 2 - fr),
                                     int(np.float32(x).view(np.uint32)) & 1))


def _bf16(x):
    return bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def _random_act(M, K, seed, outliers=4, mult=50.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    cols = rng.choice(K, size=outliers, replace=False)
    x[:, cols] *= mult
    x *= np.exp(rng.standard_normal((M, 1))).astype(np.float32)
    return _bf16(x)


# ---------------------------------------------------------------- 1x128 act

def test_act_scale_is_amax_over_448_exactly():
    xb = _random_act(24, 512, 1)
    q, s = quant_act_1x128(xb)
    x = f32_from_bf16(xb).astype(np.float64)
    for m in range(xb.shape[0]):
        for kb in range(4):
            a = max(abs(float(v)) for v in x[m, 128 * kb:128 * kb + 128])
            assert s[m, kb] == round_f32(Fraction(a) / 448), (m, kb)
            assert s[m, kb].dtype == np.float32


def test_act_exact_roundtrip_of_representable_tiles():
    rng = np.random.default_rng(2)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    for k in range(-20, 21):
        codes = rng.choice(finite, size=(3, 256))
        codes[:, 5] = 0x7E
        codes[:, 200] = 0xFE
        codes[1, 7] = 0x01          # a subnormal code
        vals = e4m3_decode(codes) * 2.0 ** k
        xb = _bf16(vals)
        assert np.array_equal(f32_from_bf16(xb).astype(np.float64), vals)  # exact in BF16
        q, s = quant_act_1x128(xb)
        assert np.all(s == np.float32(2.0 ** k)), k
        back = e4m3_decode(q) * np.repeat(s.astype(np.float64), 128, axis=1)
        assert np.array_equal(back, vals), k
        # the codes themselves come back (zero keeps its sign)
        assert np.array_equal(q, codes), k


def test_act_max_element_gets_max_code():
    xb = _random_act(32, 1024, 3)
    q, s = quant_act_1x128(xb)
    x = f32_from_bf16(xb).reshape(32, 8, 128)
    qq = q.reshape(32, 8, 128)
    idx = np.argmax(np.abs(x), axis=2)
    top = np.take_along_axis(qq, idx[..., None], axis=2)[..., 0]
    assert np.all((top == 0x7E) | (top == 0xFE))
    assert np.all(qq & 0x7F <= 0x7E)   # never NaN


def test_act_zero_tiles():
    xb = _bf16(np.zeros((2, 256), np.float32))
    xb[1] = _bf16(-np.zeros(256, np.float32))
    xb[0, 128:] = _bf16(np.full(128, 3.0, np.float32))
    q, s = quant_act_1x128(xb)
    assert s[0, 0] == 0 and s[1, 0] == 0 and s[1, 1] == 0
    assert np.all(q[0, :128] == 0x00) and np.all(q[1] == 0x80)
    assert np.all(q[0, 128:] == 0x7E)
    assert not np.any(np.isnan(s))


def test_act_tiny_amax_saturates_reciprocal():
    # amax far below 448 / FLT_MAX: the reciprocal saturates at FLT_MAX and codes stay finite
    vals = np.zeros((1, 128), np.float32)
    vals[0, :4] = [1e-39, -2e-39, 5e-40, 0.0]   # BF16 subnormals
    xb = _bf16(vals)
    q, s = quant_act_1x128(xb)
    assert np.all(np.isfinite(s)) and s[0, 0] > 0
    assert np.all(q & 0x7F <= 0x7E)


def test_act_error_bound():
    xb = _random_act(64, 2048, 4)
    q, s = quant_act_1x128(xb)
    x = f32_from_bf16(xb).astype(np.float64)
    sb = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(e4m3_decode(q) * sb - x)
    normal = np.abs(x) / sb >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -21) * np.abs(x[normal]))
    assert np.all(err[~normal] <= (2.0 ** -10 + 2.0 ** -21) * sb[~normal])


def test_act_empty_and_shape_checks():
    q, s = quant_act_1x128(np.zeros((0, 256), np.uint16))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    with pytest.raises(ValueError):
        quant_act_1x128(np.zeros((2, 100), np.uint16))


def test_act_outliers_only_affect_their_tile():
    """Fine-grained scaling: an outlier channel only changes its own tile's scale."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    q0, s0 = quant_act_1x128(_bf16(x))
    x[:, 300] *= 1000.0
    q1, s1 = quant_act_1x128(_bf16(x))
    assert np.array_equal(s0[:, [0, 1, 3]], s1[:, [0, 1, 3]])
    assert np.all(s1[:, 2] > s0[:, 2])
    assert np.array_equal(q0[:, :256], q1[:, :256])


# ---------------------------------------------------------------- 128x128 weights

def test_w_planted_block_maxima_pin_indexing():
    rng = np.random.default_rng(5)
    NB, KB = 3, 4
    w = rng.uniform(-1, 1, (NB * 128, KB * 128)).astype(np.float32)
    want = np.zeros((NB, KB), np.float32)
    for i in range(NB):
        for j in range(KB):
            e = i - 2 * j
            blk = w[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            blk *= np.float32(2.0 ** e * 100)          # all |.| < 448 * 2**e
            r, c = rng.integers(0, 128, 2)
            blk[r, c] = np.float32(448.0 * 2.0 ** e) * (1 if (i + j) % 2 else -1)
            want[i, j] = 2.0 ** e
    q, s = quant_w_128x128(_bf16(w))
    assert np.array_equal(s, want)
    x = f32_from_bf16(_bf16(w))
    for i in range(NB):
        for j in range(KB):
            blk = x[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            qb = q[128 * i:128 * i + 128, 128 * j:128 * j + 128]
            r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[r, c] == (0x7E if blk[r, c] > 0 else 0xFE)


def test_w_scale_closed_form_and_bound():
    wb = normal_bf16((256, 384), 0.02, rng_for(0, 99))
    q, s = quant_w_128x128(wb)
    x = f32_from_bf16(wb).astype(np.float64)
    for i in range(2):
        for j in range(3):
            a = float(np.max(np.abs(x[128 * i:128 * i + 128, 128 * j:128 * j + 128])))
            assert s[i, j] == round_f32(Fraction(a) / 448)
    sb = np.kron(s.astype(np.float64), np.ones((128, 128)))
    err = np.abs(e4m3_decode(q) * sb - x)
    normal = np.abs(x) / sb >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -21) * np.abs(x[normal]))
    assert np.all(err[~normal] <= (2.0 ** -10 + 2.0 ** -21) * sb[~normal])


def test_w_batched_equals_per_expert():
    wb = normal_bf16((3, 128, 256), 0.02, rng_for(0, 98))
    q, s = quant_w_128x128(wb)
    assert q.shape == (3, 128, 256) and s.shape == (3, 1, 2)
    for e in range(3):
        qe, se = quant_w_128x128(wb[e])
        assert np.array_equal(q[e], qe) and np.array_equal(s[e], se)


def test_w_zero_block():
    wb = _bf16(np.zeros((128, 256), np.float32))
    wb[:, 128:] = _bf16(np.ones((128, 128), np.float32))
    q, s = quant_w_128x128(wb)
    assert s[0, 0] == 0 and np.all(q[:, :128] == 0) and np.all(q[:, 128:] == 0x7E)


# ---------------------------------------------------------------- fused RMSNorm

def _rmsnorm_f64(xb, gb, eps):
    x = f32_from_bf16(xb).astype(np.float64)
    g = f32_from_bf16(gb).astype(np.float64)
    return x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps) * g[None, :]


@pytest.mark.parametrize("c", [1.0, -3.0, 0.015625, 2.5])
def test_rmsnorm_constant_rows_closed_form(c):
    K = 7168
    xb = _bf16(np.full((2, K), c, np.float32))
    gb = _bf16(np.ones(K, np.float32))
    y = rmsnorm_r64(xb, gb, 1e-6)
    # exact: every partial sum is a small multiple of c*c
    ss = np.float32(K * c * c)
    mean = round_f32(Fraction(float(ss)) / K)
    v = round_f32(Fraction(float(mean)) + Fraction(float(np.float32(1e-6))))
    rstd = round_f32(1 / Fraction(float(sqrt_f32(v))))
    want = round_f32(Fraction(c) * Fraction(float(rstd)))
    assert np.all(y == want)
    q, s = fused_rmsnorm_quant(xb, gb, 1e-6)
    assert np.all(q == (0x7E if c > 0 else 0xFE))
    assert np.all(s == round_f32(Fraction(abs(float(want))) / 448))


@pytest.mark.parametrize("K", [128, 640, 7168, 8320])
def test_rmsnorm_faithful_to_float64(K):
    rng = np.random.default_rng(K)
    x = (rng.standard_normal((16, K)) * 2).astype(np.float32)
    x[3] *= 1e-3
    x[5, :7] *= 40
    xb = _bf16(x)
    gb = _bf16(rng.uniform(0.5, 1.5, K).astype(np.float32))
    y = rmsnorm_r64(xb, gb, 1e-6).astype(np.float64)
    ref = _rmsnorm_f64(xb, gb, 1e-6)
    # Forward error of the binary32 evaluation: each partial adds L positive
    # terms in turn (relative error <= (L-1)u), the butterfly adds 6 levels,
    # the square root halves it, and mean, eps, sqrt, 1/., x*rstd and *gamma
    # add one rounding each.  u = 2**-24.
    L = -(-(K // 8) // 64) * 8
    bound = ((L - 1 + 6) / 2 + 6) * 2.0 ** -24 * 1.01
    rel = np.abs(y - ref) / np.abs(ref)
    assert np.all(rel[ref != 0] <= bound), (rel.max(), bound)


def test_rmsnorm_eps_matters_for_small_rows():
    K = 256
    xb = _bf16(np.full((1, K), 1e-4, np.float32))
    gb = _bf16(np.ones(K, np.float32))
    y = rmsnorm_r64(xb, gb, 1e-6).astype(np.float64)
    ref = _rmsnorm_f64(xb, gb, 1e-6)
    assert np.allclose(y, ref, rtol=1e-6) and abs(y[0, 0] - 1.0) > 1e-3


def test_fused_equals_quant_of_rmsnorm_output_invariants():
    rng = np.random.default_rng(12)
    K = 1024
    xb = _bf16((rng.standard_normal((8, K)) * 2).astype(np.float32))
    gb = _bf16(rng.uniform(0.5, 1.5, K).astype(np.float32))
    q, s = fused_rmsnorm_quant(xb, gb, 1e-6)
    y = rmsnorm_r64(xb, gb, 1e-6).astype(np.float64)
    for m in range(8):
        for kb in range(K // 128):
            a = np.max(np.abs(y[m, 128 * kb:128 * kb + 128]))
            assert s[m, kb] == round_f32(Fraction(float(a)) / 448)
    sb = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(e4m3_decode(q) * sb - y)
    normal = np.abs(y) / sb >= 2.0 ** -6
    assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -21) * np.abs(y[normal]))
    # y is not rounded to BF16 before the cast: differs from quantising bf16(y)
    qb, sb2 = quant_act_1x128(_bf16(y.astype(np.float32)))
    assert not (np.array_equal(q, qb) and np.array_equal(s, sb2))


# ------------------------------------------- the R64 summation order, pinned
#
# Crafted rows (K = 1024, so 128 vectors of 8 values; in the R64 order partial
# l takes vectors l and l + 64) whose binary32 sum of squares is derived by
# hand below.  Each row is built so that one or more plausible alternative
# orders round differently; the alternatives are evaluated by the small loops
# in this test, written independently of the oracle.

def _rne_f32(fr: Fraction) -> Fraction:
    """Nearest binary32 value (subnormals included), ties to even, as a Fraction."""
    if fr == 0:
        return Fraction(0)
    mag = abs(fr)
    e = mag.numerator.bit_length() - mag.denominator.bit_length()
    if Fraction(2) ** e > mag:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 23)      # spacing of the binade (subnormal: 2**-149)
    n, r = divmod(mag, q)
    n = int(n)
    if r > q / 2 or (r == q / 2 and n % 2 == 1):
        n += 1
    return (n * q) if fr > 0 else -(n * q)


def _f32(v) -> np.float32:
    return np.float32(v)


def _ss_loop(x, assign, ds, fused=False):
    """Sum of squares of one float32 row: 64 partials, partial l adding the
    squares of the vectors assign(l) one value at a time, then a butterfly over
    the distances ds.  fused: each step rounds acc + x*x once (a fused
    multiply-add) instead of rounding the square first."""
    acc = [_f32(0.0)] * 64
    for lane in range(64):
        a = _f32(0.0)
        for v in assign(lane):
            for j in range(8):
                xv = x[8 * v + j]
                if fused:
                    a = _f32(float(_rne_f32(Fraction(float(a)) + Fraction(float(xv)) ** 2)))
                else:
                    a = _f32(a + _f32(xv * xv))
        acc[lane] = a
    for d in ds:
        acc = [_f32(acc[lane] + acc[lane ^ d]) for lane in range(64)]
    return acc[0]


def _ss_sequential(x):
    a = _f32(0.0)
    for xv in x:
        a = _f32(a + _f32(xv * xv))
    return a


_V = 128  # vectors in a K = 1024 row
_ALT = {
    "sequential": _ss_sequential,
    "contiguous partials": lambda x: _ss_loop(x, lambda l: range(2 * l, 2 * l + 2), (32, 16, 8, 4, 2, 1)),
    "reversed butterfly": lambda x: _ss_loop(x, lambda l: (l, l + 64), (1, 2, 4, 8, 16, 32)),
    "fused multiply-add": lambda x: _ss_loop(x, lambda l: (l, l + 64), (32, 16, 8, 4, 2, 1), fused=True),
    "later vector first": lambda x: _ss_loop(x, lambda l: (l + 64, l), (32, 16, 8, 4, 2, 1)),
}


def _row_big_then_lane_eights():
    # x_0 = 2**12 (square 2**24); in vectors 1..63 (first vectors of partials
    # 1..63) every value is 1.
    x = np.zeros(1024, np.float32)
    x[0] = 4096.0
    x[8:512] = 1.0
    return x


def _row_big_and_upper_half_ones():
    # x_0 = 2**12; the first value of vectors 32..63 is 1 (partials 32..63
    # hold 1 each).
    x = np.zeros(1024, np.float32)
    x[0] = 4096.0
    x[8 * np.arange(32, 64)] = 1.0
    return x


def _row_ones_then_big():
    # vector 0 all ones, then x_512 = 2**12 (first value of vector 64, the
    # second vector of partial 0).
    x = np.zeros(1024, np.float32)
    x[0:8] = 1.0
    x[512] = 4096.0
    return x


def _row_subnormal_tie():
    # x_0 = 3 * 2**-76 (square 9 * 2**-152 = 1.125 * 2**-149), x_1 = 2**-75
    # (square exactly 2**-150, half the smallest subnormal).
    x = np.zeros(1024, np.float32)
    x[0] = 3.0 * 2.0 ** -76
    x[1] = 2.0 ** -75
    return x


# (row, hand-derived R64 sum, {alternative: its hand-derived sum}).  Every
# listed alternative differs from the R64 sum.
#
# Row 1.  R64: partial 0 holds 2**24; partials 1..63 hold 8 (eight squares of
# 1, exact).  Every butterfly sum is an even integer below 2**25, so exact:
# 2**24 + 63 * 8 = 16777720.  Sequential: each later +1 meets 2**24, a tie
# between 2**24 and 2**24 + 2, which rounds to even (2**24): 16777216.
# Contiguous partials: partial 0 takes vectors 0 and 1, so the eight ones of
# vector 1 are dropped one by one against 2**24; the other 62 vectors of ones
# (31 partials of 16) arrive exactly: 2**24 + 496 = 16777712.
#
# Row 2.  R64: after d = 32, partial 0 is 2**24 + 1 -> 2**24 (tie, even),
# partials 1..31 hold 1.  d = 16: 2**24 + 1 -> 2**24 again; partials 1..15
# hold 2.  d = 8: 2**24 + 2 (exact); partials 1..7 hold 4.  d = 4: + 4 ->
# 2**24 + 6; d = 2: + 8 -> 2**24 + 14; d = 1: + 16 -> 2**24 + 30 = 16777246.
# Reversed butterfly: the 32 ones meet each other first (partials 32..63 reach
# 32 by d = 16), partial 0 stays 2**24 until d = 32 adds 32: 16777248.
# Sequential: every one is dropped: 16777216.  Contiguous partials: vectors
# 32..63 land in partials 16..31 (2 each); d = 32 adds zeros, then d = 16
# adds 2, d = 8 adds 2, d = 4 adds 4, d = 2 adds 8, d = 1 adds 16: 16777248.
#
# Row 3.  R64: partial 0 adds the eight ones (8), then 2**24: 2**24 + 8 =
# 16777224 (exact).  Taking the later vector first gives 2**24, then eight
# dropped ones: 16777216.
#
# Row 4.  R64: fl32(x_0**2) = 2**-149 (1.125 units of 2**-149 round to 1);
# fl32(x_1**2) = 0 (half a unit, a tie, rounds to even 0); the sum is 2**-149.
# Fused multiply-add: the first step gives 2**-149, the second rounds
# 2**-149 + 2**-150 = 1.5 units, a tie, to even: 2 units = 2**-148.
_R64_CASES = [
    (_row_big_then_lane_eights, 16777720.0,
     {"sequential": 16777216.0, "contiguous partials": 16777712.0}),
    (_row_big_and_upper_half_ones, 16777246.0,
     {"reversed butterfly": 16777248.0, "sequential": 16777216.0, "contiguous partials": 16777248.0}),
    (_row_ones_then_big, 16777224.0, {"later vector first": 16777216.0}),
    (_row_subnormal_tie, 2.0 ** -149, {"fused multiply-add": 2.0 ** -148}),
]


@pytest.mark.parametrize("case", range(len(_R64_CASES)))
def test_r64_order_pinned_by_crafted_rows(case):
    make, want, alternatives = _R64_CASES[case]
    x = make()
    xb = _bf16(x)
    assert np.array_equal(f32_from_bf16(xb), x), "crafted values must be exact in BF16"
    ss = sum_squares_r64(xb[None, :])[0]
    assert ss.dtype == np.float32
    assert float(ss) == want, (float(ss), want)
    for name, alt_want in alternatives.items():
        got = float(_ALT[name](x))
        assert got == alt_want, (name, got, alt_want)   # the alternative loop agrees with its derivation
        assert got != want, name                       # ... and R64 tells it apart


def test_r64_alternatives_all_rejected():
    # every alternative order is told apart from R64 by at least one crafted row
    rejected = set()
    for _, _, alternatives in _R64_CASES:
        rejected |= set(alternatives)
    assert rejected == set(_ALT)


def test_rmsnorm_uses_the_r64_sum():
    # row 1 through the whole norm: with gamma = 1 the output at a value of 1
    # is rstd itself, which the R64 sum (not the sequential one) determines
    x = _row_big_then_lane_eights()
    xb = _bf16(x)[None, :]
    gb = _bf16(np.ones(1024, np.float32))
    y = rmsnorm_r64(xb, gb, 1e-6)

    def rstd_of(ss):
        mean = round_f32(Fraction(ss) / 1024)
        v = round_f32(Fraction(float(mean)) + Fraction(float(np.float32(1e-6))))
        return round_f32(1 / Fraction(float(sqrt_f32(v))))

    assert y[0, 8] == rstd_of(16777720.0)
    assert rstd_of(16777720.0) != rstd_of(16777216.0)
    assert np.array_equal(y[0], (x * y[0, 8]).astype(np.float32))
