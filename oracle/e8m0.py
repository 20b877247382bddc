"""Power-of-two (E8M0) block scales, oracle side.

What the pages fix: the 1x128 / 128x128 group scaling is in line with
microscaling formats, and newer matrix units support such formats natively
[P1 paragraph 4, P4 paragraph 3].  They give no scale encoding.

External definition (OCP Microscaling Formats (MX) specification v1.0): a
microscaling block scale is E8M0, an unsigned 8-bit biased exponent with no
mantissa: byte b means 2**(b - 127) for b = 0 .. 254; b = 255 is NaN; there
is no zero.

Readings (the pages do not fix them; one bit-exact answer needs them):
  * the scale of a group with max-abs ``a`` is the method's ``a / 448``
    rounded UP to a power of two: the smallest integer ``e`` with
    ``448 * 2**e >= a``.  Rounding up keeps every scaled value inside +-448,
    so no clamp is ever needed.  (The MX specification's own rule,
    ``floor(log2 a) - 8``, can push values past 448, which must then
    saturate.)
  * ``e`` is clamped below to -127 (byte 0).  That covers ``a = 0`` and
    ``a < 448 * 2**-127``, whose true ``e`` the format cannot hold; the
    scaled values then still satisfy ``|x * 2**-e| <= 448``.
  * the cast is ``q = E4M3_rne(x * 2**-e)``.  The product is exact: a float32
    ``x`` times a power of two, computed in float64.
  * the dequantised value is ``dec(q) * 2**(b - 127)``.  The GEMM is the same
    float64 definition as ``oracle.gemm``, with these scales.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, e4m3_encode
from .gemm import gemm_ref, grouped_gemm_ref
from .quant import f32_from_bf16, rmsnorm_r64

E8M0_BIAS = 127
E8M0_MIN_EXP = -127


def e8m0_decode(b: np.ndarray) -> np.ndarray:
    """E8M0 bytes to float64 scales ``2**(b - 127)``; byte 255 is NaN."""
    b = np.asarray(b, dtype=np.uint8)
    v = np.ldexp(1.0, b.astype(np.int64) - E8M0_BIAS)
    return np.where(b == 255, np.nan, v)


def e8m0_exponent(a: np.ndarray) -> np.ndarray:
    """Smallest integer ``e >= -127`` with ``448 * 2**e >= a`` (``a >= 0``
    finite, any float dtype), as int64.

    Search from a start below the answer: with ``a = f * 2**p``
    (``0.5 <= f < 1``), ``a / 448`` lies in ``[2**(p - 10), 2**(p - 8))``,
    so the answer is ``p - 9`` or ``p - 8``.  Starting at ``p - 10`` and
    stepping up while ``448 * 2**e < a`` reaches it.  Every comparison is
    exact in float64.  ``a = 0`` satisfies every ``e``, so its answer is the
    lower limit -127.
    """
    a = np.asarray(a, dtype=np.float64)
    if np.any(~np.isfinite(a)) or np.any(a < 0):
        raise ValueError("e8m0_exponent takes finite a >= 0")
    _, p = np.frexp(a)
    e = p.astype(np.int64) - 10
    for _ in range(3):
        e = np.where(np.ldexp(E4M3_MAX, e) < a, e + 1, e)
    e = np.where(a == 0, E8M0_MIN_EXP, np.maximum(e, E8M0_MIN_EXP))
    assert np.all(np.ldexp(E4M3_MAX, e) >= a)
    return e


def _e8m0_cast(x: np.ndarray, a: np.ndarray, group_axes) -> tuple[np.ndarray, np.ndarray]:
    """float32 values ``x`` and their group max-abs ``a`` -> (codes, E8M0 bytes)."""
    e = e8m0_exponent(a)
    y = x.astype(np.float64) * np.expand_dims(np.ldexp(1.0, -e), group_axes)   # exact
    assert np.all(np.abs(y) <= E4M3_MAX)
    # y is exact in float32 unless |y| < 2**-126, where any rounding still
    # encodes to a signed zero (the smallest E4M3 magnitude is 2**-9)
    q = e4m3_encode(y.astype(np.float32))
    return q, (e + E8M0_BIAS).astype(np.uint8)


def quant_act_1x128_e8m0(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 ``[M, K]`` -> E4M3 codes ``[M, K]`` and E8M0 bytes ``[M, K/128]``."""
    M, K = x_bits.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    x = f32_from_bf16(x_bits).reshape(M, K // 128, 128)
    a = np.max(np.abs(x), axis=2) if M else np.zeros((0, K // 128), np.float32)
    q, b = _e8m0_cast(x, a, (2,))
    return q.reshape(M, K), b


def quant_w_128x128_e8m0(w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 ``[N, K]`` or ``[B, N, K]`` -> codes and E8M0 bytes ``[(B,) N/128, K/128]``."""
    batched = w_bits.ndim == 3
    w = w_bits if batched else w_bits[None]
    B, N, K = w.shape
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    x = f32_from_bf16(w).reshape(B, N // 128, 128, K // 128, 128)
    a = np.max(np.abs(x), axis=(2, 4))
    q, b = _e8m0_cast(x, a, (2, 4))
    q = q.reshape(B, N, K)
    return (q, b) if batched else (q[0], b[0])


def fused_rmsnorm_quant_e8m0(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float
                             ) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm (``oracle.quant.rmsnorm_r64``, float32, not rounded to BF16)
    followed by the E8M0 1x128 quantisation of its output."""
    M, K = x_bits.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    y = rmsnorm_r64(x_bits, gamma_bits, eps).reshape(M, K // 128, 128)
    a = np.max(np.abs(y), axis=2) if M else np.zeros((0, K // 128), np.float32)
    q, b = _e8m0_cast(y, a, (2,))
    return q.reshape(M, K), b


def gemm_e8m0_ref(qa, ba, qw, bw) -> np.ndarray:
    """Dense GEMM with E8M0 scale bytes, float64 ``[M, N]``."""
    return gemm_ref(qa, e8m0_decode(ba), qw, e8m0_decode(bw))


def grouped_gemm_e8m0_ref(qa, ba, qw, bw, offsets) -> np.ndarray:
    """Grouped GEMM with E8M0 scale bytes, float64 ``[R, N]``."""
    return grouped_gemm_ref(qa, e8m0_decode(ba), qw, e8m0_decode(bw), offsets)
