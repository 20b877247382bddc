"""Quantise-then-dispatch: FP8 activation rows grouped by expert.

Source: P2 (Q&A board page) paragraph 4 -- the activations entering the MoE
up-projection are quantised to FP8 first and dispatched to the experts in
that form; P3 paragraph 4 -- each token is routed to 8 experts.

The pages fix neither the row order inside an expert nor what happens to
unusable expert ids.  Readings:

  * Every (token, slot) pair ``i = t * topk + j`` with an expert id in
    ``[0, E)`` becomes one output row; other ids are not routed.
  * Rows are ordered by expert and, inside an expert, by increasing ``i``
    (a stable sort by expert id), so the layout is unique.
  * A routed row holds the 1x128 quantisation of its token's row, which is
    exactly ``quant_act_1x128`` of that row (per-tile scales do not depend
    on which rows are quantised together).

Outputs besides the codes and scales: ``offsets[E + 1]`` (rows of expert e
are ``offsets[e] .. offsets[e + 1] - 1``), ``row_src[r]`` = the pair ``i``
that filled row ``r`` and ``dest[i]`` = the row of pair ``i`` (-1 if not
routed), the two index maps a combine step needs.
"""
from __future__ import annotations

import numpy as np

from .quant import quant_act_1x128


def dispatch_ref(ids: np.ndarray, n_experts: int):
    """Stable routing of the (token, slot) pairs of ``ids [T, topk]``.

    Returns ``(offsets int32 [E+1], row_src int32 [R], dest int32 [T*topk])``.
    A library stable sort is the step that orders the pairs by expert.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    valid = (flat >= 0) & (flat < n_experts)
    idx = np.nonzero(valid)[0]
    row_src = idx[np.argsort(flat[idx], kind="stable")]
    counts = np.bincount(flat[idx], minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    dest = np.full(flat.shape[0], -1, dtype=np.int64)
    dest[row_src] = np.arange(row_src.shape[0])
    return offsets.astype(np.int32), row_src.astype(np.int32), dest.astype(np.int32)


def quant_dispatch_ref(x_bits: np.ndarray, ids: np.ndarray, n_experts: int):
    """``x_bits`` BF16 bits ``[T, K]``, ``ids [T, topk]`` -> ``(q [R, K], s [R, K/128], offsets, row_src, dest)``."""
    ids = np.asarray(ids)
    topk = ids.shape[1] if ids.ndim == 2 else 1
    offsets, row_src, dest = dispatch_ref(ids, n_experts)
    tokens = row_src.astype(np.int64) // topk
    q, s = quant_act_1x128(np.asarray(x_bits)[tokens])
    return q, s, offsets, row_src, dest


def quant_dispatch_e8m0_ref(x_bits: np.ndarray, ids: np.ndarray, n_experts: int):
    """As ``quant_dispatch_ref`` with power-of-two scales (``oracle.e8m0``):
    ``(q [R, K], E8M0 bytes [R, K/128], offsets, row_src, dest)``."""
    from .e8m0 import quant_act_1x128_e8m0
    ids = np.asarray(ids)
    topk = ids.shape[1] if ids.ndim == 2 else 1
    offsets, row_src, dest = dispatch_ref(ids, n_experts)
    tokens = row_src.astype(np.int64) // topk
    q, b = quant_act_1x128_e8m0(np.asarray(x_bits)[tokens])
    return q, b, offsets, row_src, dest
