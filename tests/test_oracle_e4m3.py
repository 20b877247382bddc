"""Pins for the oracle's E4M3 codec (CPU only).

Each check is independent of the oracle's own arithmetic:
  * hand-written OCP E4M3 code points (tests/golden/e4m3_ocp_points.txt);
  * round trip over all 254 finite codes and monotonicity;
  * brute-force nearest-value search over all 127 positive finite codes;
  * an exhaustive sweep over every float32 in [2**-11, 448] against a
    bisection-based nearest-value search and against torch's float8_e4m3fn
    cast (a library routine);
  * everything below 2**-11 encodes to (signed) zero.
"""
import os

import numpy as np
import pytest

from oracle import E4M3_MAX, e4m3_decode, e4m3_decode_table, e4m3_encode

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_points.txt")


def _positive_codes():
    """The 127 positive finite codes 0x00..0x7E with their values, by the
    spec's field layout (written independently of the oracle's table)."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals, dtype=np.float64)


def _nearest_bruteforce(y):
    """Nearest positive code to |y| by scanning all 127 codes; ties to even code."""
    vals = _positive_codes()
    a = np.abs(np.asarray(y, dtype=np.float64))
    d = np.abs(a[:, None] - vals[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    # at most two candidates on a tie; pick the even code (even mantissa)
    idx = np.where(cand.sum(axis=1) == 1, cand.argmax(axis=1), -1)
    tie_rows = np.nonzero(idx < 0)[0]
    for i in tie_rows:
        cs = np.nonzero(cand[i])[0]
        even = [c for c in cs if c % 2 == 0]
        assert len(cs) == 2 and len(even) == 1
        idx[i] = even[0]
    return idx.astype(np.uint8)


def _nearest_bisect(a):
    """Nearest positive code to a (>= 0, float64) via bisection; ties to even."""
    vals = _positive_codes()
    hi = np.searchsorted(vals, a, side="left")       # vals[hi-1] < a <= vals[hi]
    hi = np.clip(hi, 1, len(vals) - 1)
    lo = hi - 1
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    out = np.where(a == 0, 0, out)
    return out.astype(np.uint8)


def test_golden_ocp_points():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                v, c = line.split()[:2]
                rows.append((float(v), int(c, 16)))
    y = np.array([r[0] for r in rows], dtype=np.float32)
    want = np.array([r[1] for r in rows], dtype=np.uint8)
    got = e4m3_encode(y)
    assert np.array_equal(got, want), list(zip(y, got, want))
    # decoding the code gives the value back wherever the value is a code point
    for v, c in rows:
        if float(np.float32(v)) == v and e4m3_encode(np.float32([v]))[0] == c:
            d = e4m3_decode(np.uint8([c]))[0]
            if d == v:
                assert np.signbit(d) == np.signbit(v)


def test_decode_table_special_values():
    t = e4m3_decode_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.sum(np.isnan(t)) == 2
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    assert np.signbit(t[0x80]) and t[0x80] == 0.0
    assert np.array_equal(t[:0x7F], _positive_codes())


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3_encode(vals), codes)


def test_monotone_positive():
    y = np.sort(np.random.default_rng(5).uniform(0, 448, 200000).astype(np.float32))
    q = e4m3_encode(y)
    assert np.all(np.diff(q.astype(np.int32)) >= 0)


def test_bruteforce_nearest_random_and_midpoints():
    rng = np.random.default_rng(7)
    vals = _positive_codes()
    mids = (vals[1:] + vals[:-1]) / 2
    pts = [vals, mids]
    for k in (1, 2, 3):
        pts.append(np.nextafter(mids.astype(np.float32), np.float32(0), dtype=np.float32).astype(np.float64))
        pts.append(np.nextafter(mids.astype(np.float32), np.float32(1e9), dtype=np.float32).astype(np.float64))
    logu = rng.uniform(np.log(2.0 ** -12), np.log(448.0), 300000)
    pts.append(np.exp(logu))
    y = np.concatenate(pts).astype(np.float32)
    y = y[(y <= 448) & (y >= 0)]
    assert np.array_equal(e4m3_encode(y), _nearest_bruteforce(y))
    # negative values: same magnitude code with the sign bit set
    assert np.array_equal(e4m3_encode(-y), _nearest_bruteforce(y) | np.uint8(0x80))


def test_exhaustive_float32_sweep():
    """Every float32 in [2**-11, 448]: oracle vs bisection vs torch's cast."""
    torch = pytest.importorskip("torch")
    lo = np.float32(2.0 ** -11).view(np.uint32)
    hi = np.float32(448.0).view(np.uint32)
    step = 1 << 23
    for start in range(int(lo), int(hi) + 1, step):
        stop = min(int(hi) + 1, start + step)
        y = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        q = e4m3_encode(y)
        assert np.array_equal(q, _nearest_bisect(y.astype(np.float64))), hex(start)
        t = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q, t), hex(start)


def test_below_half_smallest_subnormal_is_zero():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, int(np.float32(2.0 ** -11).view(np.uint32)), 2_000_000, dtype=np.uint32)
    y = bits.view(np.float32)
    assert np.all(e4m3_encode(y) == 0)
    assert np.all(e4m3_encode(-y) == 0x80)


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        e4m3_encode(np.float32([E4M3_MAX * 1.01]))
    with pytest.raises(ValueError):
        e4m3_encode(np.float32([np.nan]))
