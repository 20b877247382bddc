"""E4M3 (OCP "E4M3FN") encode and decode, oracle side.

The pages say only "FP8" (P1 paragraph 1, P2 paragraph 3); the workload
definition names E4M3 with largest value 448, which is the OCP 8-bit
floating point E4M3 format: 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits, no infinities, NaN = 0x7F / 0xFF, largest finite 448
(0x7E), smallest normal 2**-6 (0x08), smallest subnormal 2**-9 (0x01).

Readings (the pages are silent):
  * rounding is to nearest, ties to the even mantissa (IEEE default);
  * subnormals are kept (gradual underflow), the sign of zero is kept;
  * the encoder is only defined on ``|y| <= 448``; callers clamp first, so
    no NaN code is ever produced.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
FLT_MAX = np.float32(3.4028234663852886e38)


def e4m3_decode_table() -> np.ndarray:
    """All 256 codes as float64 (exact); 0x7F and 0xFF are NaN."""
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = sign * m * 2.0 ** -9
        else:
            t[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


_DEC = e4m3_decode_table()


def e4m3_decode(q: np.ndarray) -> np.ndarray:
    """Codes (uint8) to exact float64 values."""
    return _DEC[np.asarray(q, dtype=np.uint8)]


def e4m3_encode(y: np.ndarray) -> np.ndarray:
    """float32 values with ``|y| <= 448`` to E4M3 codes (uint8).

    Works in float64, where every step below is exact for a float32 input:
      * normal range ``|y| >= 2**-6``: write ``|y| = f * 2**e`` with
        ``f in [1, 2)``; the 3-bit mantissa is ``t = rne(8 * (f - 1))``;
        ``t == 8`` carries into the exponent;
      * below it: a subnormal count ``t = rne(|y| * 2**9)`` of units 2**-9
        (``t == 8`` lands exactly on the smallest normal code 0x08).
    """
    y = np.ascontiguousarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("e4m3_encode takes finite |y| <= 448 (clamp first)")
    sign = ((y.view(np.uint32) >> np.uint32(31)).astype(np.uint8)) << np.uint8(7)
    a = np.abs(y.astype(np.float64))
    frac, ex = np.frexp(a)            # a = frac * 2**ex, frac in [0.5, 1)
    f = 2.0 * frac                    # a = f * 2**(ex-1), f in [1, 2)
    e = ex.astype(np.int64) - 1
    t = np.rint(8.0 * (f - 1.0)).astype(np.int64)   # np.rint: ties to even
    carry = t == 8
    e = e + carry
    t = np.where(carry, 0, t)
    normal_code = ((e + 7) << 3) | t
    sub_code = np.rint(a * 2.0 ** 9).astype(np.int64)
    code = np.where(a >= 2.0 ** -6, normal_code, sub_code)
    return code.astype(np.uint8) | sign
