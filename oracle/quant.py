"""Online max-abs FP8 quantisation: 1x128 activation tiles, 128x128 weight
blocks, and RMSNorm fused with the activation quantisation (oracle side).

What the pages fix:
  * activations are grouped and scaled per token per 128 channels (1x128
    tiles), weights per 128 input x 128 output channels (128x128 blocks)
    [P1 paragraph 1];
  * the scale maps the group's max-abs value onto the largest FP8 value
    [P2 paragraph 3] and is derived online from it before the cast
    [P2 paragraph 4, P4 paragraph 1];
  * quantised activations are stored as 1x128 FP8 tiles [P3 paragraph 3];
  * a layer normalisation can be fused with the FP8 cast [P3 paragraph 3],
    the normalisation itself kept in higher precision [P2 paragraph 1].

The workload definition adds E4M3 and ``scale = amax / 448``.

Readings where the pages are silent (one bit-exact answer needs them):
  * the stored scale is the dequantisation multiplier ``s = fl32(a / 448)``;
  * the cast multiplies by ``r = min(fl32(448 / a), FLT_MAX)`` (one
    correctly rounded division per group), so an all-zero group gives
    ``s = 0``, codes +-0 and no NaN;
  * ``y = fl32(x * r)`` is clamped to +-448 (sign of zero kept), then
    encoded with round-to-nearest-even (``oracle.e4m3``);
  * ``fl32`` is IEEE binary32 round-to-nearest-even; subnormals are kept.
  * NaN / Inf inputs are outside the contract.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import E4M3_MAX, FLT_MAX, e4m3_encode

_F448 = np.float32(E4M3_MAX)


def f32_from_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) to float32; exact (the bits move up 16)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_and_cast(x: np.ndarray, a: np.ndarray, group_axes) -> tuple[np.ndarray, np.ndarray]:
    """Given float32 values ``x`` and their group max-abs ``a`` (float32), return
    (codes, scales).  ``group_axes`` are the axes of ``x`` that ``a`` lacks."""
    s = (a / _F448).astype(np.float32)                 # fl32(a / 448)
    with np.errstate(divide="ignore", over="ignore"):
        r = (_F448 / a).astype(np.float32)             # fl32(448 / a); a = 0 -> +inf
    r = np.minimum(r, FLT_MAX)
    r_b = np.expand_dims(r, group_axes)
    y = (x * r_b).astype(np.float32)                   # fl32(x * r)
    y = np.minimum(np.maximum(y, -_F448), _F448)       # keeps -0.0
    return e4m3_encode(y), s


def quant_act_1x128(x_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 ``[M, K]`` -> E4M3 codes ``[M, K]`` (uint8), scales ``[M, K/128]`` (float32).

    One scale per (token, 128-channel group): the 1x128 tile.
    """
    M, K = x_bits.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    x = f32_from_bf16(x_bits).reshape(M, K // 128, 128)
    a = np.max(np.abs(x), axis=2) if M else np.zeros((0, K // 128), np.float32)
    q, s = _scale_and_cast(x, a, (2,))
    return q.reshape(M, K), s


def quant_w_128x128(w_bits: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """BF16 ``[N, K]`` or ``[B, N, K]`` -> codes of the same shape and scales
    ``[N/128, K/128]`` (or ``[B, N/128, K/128]``): one scale per 128x128 block."""
    batched = w_bits.ndim == 3
    w = w_bits if batched else w_bits[None]
    B, N, K = w.shape
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    x = f32_from_bf16(w).reshape(B, N // 128, 128, K // 128, 128)
    a = np.max(np.abs(x), axis=(2, 4))
    q, s = _scale_and_cast(x, a, (2, 4))
    q = q.reshape(B, N, K)
    return (q, s) if batched else (q[0], s[0])


def sum_squares_r64(x_bits: np.ndarray) -> np.ndarray:
    """Sum of squares of each row of BF16 ``x [M, K]`` in the fixed order
    "R64"; returns float32 ``[M]``.

    Reading: the pages say only that the normalisation stays in higher
    precision and may be fused with the cast; a bit-exact answer needs one
    summation order, and this one is fixed here.  The row is cut into
    vectors of 8 consecutive values.  64 partial sums each take every 64th
    vector in turn (partial ``l`` takes vectors ``l, l+64, ...``) and add the
    squares of its 8 values one by one, ``acc = fl32(acc + fl32(x*x))`` (a
    multiply, then an add: no fused multiply-add).  The 64 partials are then
    combined by a butterfly: for ``d = 32, 16, 8, 4, 2, 1`` every partial
    ``l`` becomes ``fl32(acc_l + acc_(l xor d))``; the result is partial 0.
    """
    M, K = x_bits.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    x = f32_from_bf16(x_bits)
    V = K // 8
    acc = np.zeros((M, 64), dtype=np.float32)
    xv = x.reshape(M, V, 8)
    for base in range(0, V, 64):
        lanes = min(64, V - base)
        for j in range(8):
            v = xv[:, base:base + lanes, j]
            sq = (v * v).astype(np.float32)
            acc[:, :lanes] = (acc[:, :lanes] + sq).astype(np.float32)
    for d in (32, 16, 8, 4, 2, 1):
        partner = np.arange(64) ^ d
        acc = (acc + acc[:, partner]).astype(np.float32)
    return acc[:, 0].copy()


def rmsnorm_r64(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm ``y = x * rsqrt(mean(x**2) + eps) * gamma`` in binary32;
    returns float32 ``[M, K]`` (not rounded to BF16).

    The workload names RMSNorm with ``eps = 1e-6`` and BF16 gamma.  The sum
    of squares is ``sum_squares_r64`` (one fixed order); then ``mean =
    fl32(ss / K)``, ``v = fl32(mean + fl32(eps))``, ``rstd = fl32(1 /
    fl32(sqrt(v)))``, ``y = fl32(fl32(x * rstd) * gamma)``.
    """
    M, K = x_bits.shape
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    x = f32_from_bf16(x_bits)
    g = f32_from_bf16(gamma_bits)
    ss = sum_squares_r64(x_bits)
    mean = (ss / np.float32(K)).astype(np.float32)
    v = (mean + np.float32(eps)).astype(np.float32)
    rstd = (np.float32(1.0) / np.sqrt(v).astype(np.float32)).astype(np.float32)
    y = (x * rstd[:, None]).astype(np.float32)
    y = (y * g[None, :]).astype(np.float32)
    return y


def fused_rmsnorm_quant(x_bits: np.ndarray, gamma_bits: np.ndarray, eps: float
                        ) -> tuple[np.ndarray, np.ndarray]:
    """RMSNorm (``rmsnorm_r64``) followed by 1x128 quantisation of its float32
    output: codes ``[M, K]`` and scales ``[M, K/128]``."""
    M, K = x_bits.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    y = rmsnorm_r64(x_bits, gamma_bits, eps).reshape(M, K // 128, 128)
    a = np.max(np.abs(y), axis=2) if M else np.zeros((0, K // 128), np.float32)
    q, s = _scale_and_cast(y, a, (2,))
    return q.reshape(M, K), s
