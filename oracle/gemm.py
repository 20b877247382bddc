"""Block-scaled FP8 GEMM and its ragged grouped (MoE) variant, oracle side.

What the pages fix: the GEMM consumes FP8 operands with per-group scaling
factors along the inner dimension K, which are multiplied in as the
dequantisation step [P2 paragraph 3]; partial sums are accumulated in FP32
rather than the limited width of the MMA unit [P1 paragraph 4,
P4 paragraph 4]; MoE up-projections run their forward GEMM in FP8
[P2 paragraph 4], one GEMM per expert [P3 paragraph 4].

The oracle is the definition in float64:
  ``C*[m, n] = sum_k (dec(qa[m,k]) * sa[m, k//128]) * (dec(qw[n,k]) * sw[n//128, k//128])``
evaluated by dequantising both operands exactly (an E4M3 value times a
float32 scale has at most 4 + 24 significant bits, exact in float64) and
one float64 matrix product.  This equals the chunk-wise
``sum_kb sa*sw * sum_{k in kb} dec*dec`` up to float64 rounding.

Layouts (a reading; the pages give none): A ``[M, K]``, W ``[N, K]``, both
K-contiguous; activation scales ``[M, K/128]``, weight scales
``[N/128, K/128]``; grouped: rows of A concatenated by expert, expert ``e``
owning rows ``offsets[e] .. offsets[e+1]``, weights ``[E, N, K]`` and scales
``[E, N/128, K/128]``.

The tolerance gate is the workload definition's: normwise relative error
``||C - C*||_F / ||C*||_F <= 2e-3`` and ``|C - C*| <= 1e-2 |C*|`` wherever
``|C*| > 1e-2 * rms(C*)``.
"""
from __future__ import annotations

import numpy as np

from .e4m3 import e4m3_decode


def dequant_act(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes ``[M, K]`` and 1x128 scales ``[M, K/128]`` to float64 ``[M, K]``."""
    M, K = q.shape
    v = e4m3_decode(q).reshape(M, K // 128, 128)
    return (v * s.astype(np.float64)[:, :, None]).reshape(M, K)


def dequant_w(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes ``[N, K]`` and 128x128 scales ``[N/128, K/128]`` to float64 ``[N, K]``."""
    N, K = q.shape
    v = e4m3_decode(q).reshape(N // 128, 128, K // 128, 128)
    return (v * s.astype(np.float64)[:, None, :, None]).reshape(N, K)


def gemm_ref(qa, sa, qw, sw) -> np.ndarray:
    """Dense block-scaled GEMM ``C* = A_hat @ W_hat.T`` in float64, ``[M, N]``."""
    return dequant_act(qa, sa) @ dequant_w(qw, sw).T


def grouped_gemm_ref(qa, sa, qw, sw, offsets) -> np.ndarray:
    """Grouped GEMM: rows ``offsets[e]..offsets[e+1]`` of A times expert ``e``'s
    weight; ``[R, N]`` float64.  Experts with no rows contribute nothing."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    R = int(offsets[-1])
    N = qw.shape[1]
    out = np.zeros((R, N), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 > r0:
            out[r0:r1] = gemm_ref(qa[r0:r1], sa[r0:r1], qw[e], sw[e])
    return out


def bf16_round_f64(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest BF16 value (ties to even), returned as float64.

    Used for the "rounding floor" report: the error the BF16 output format
    alone costs.  Rounds float64 to BF16 directly (no float32 step)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # |m| in [0.5, 1)
    # BF16 keeps 8 significant bits: scale the significand to [128, 256).
    r = np.rint(m * 256.0)
    return np.ldexp(r, e - 8)


def gemm_gate(c: np.ndarray, ref: np.ndarray, normwise: float = 2e-3, elementwise: float = 1e-2,
              rel_mask: float = 1e-2) -> dict:
    """Apply the tolerance gate to a GPU result ``c`` against ``ref`` (both
    float64-convertible, same shape).  Returns a dict with the measured
    figures and ``ok``."""
    c = np.asarray(c, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if c.shape != ref.shape:
        raise ValueError(f"shape mismatch {c.shape} vs {ref.shape}")
    if ref.size == 0:
        return {"ok": True, "normwise": 0.0, "max_elem_rel": 0.0, "finite": True}
    finite = bool(np.all(np.isfinite(c)))
    diff = c - ref
    nref = float(np.linalg.norm(ref.ravel()))
    nerr = float(np.linalg.norm(diff.ravel()))
    normrel = nerr / nref if nref > 0 else (0.0 if nerr == 0 else np.inf)
    rms = float(np.sqrt(np.mean(ref * ref)))
    mask = np.abs(ref) > rel_mask * rms
    if np.any(mask):
        elem = float(np.max(np.abs(diff[mask]) / np.abs(ref[mask])))
    else:
        elem = 0.0
    ok = finite and normrel <= normwise and elem <= elementwise
    return {"ok": bool(ok), "normwise": normrel, "max_elem_rel": elem, "finite": finite}
