"""Per-tensor scaling against fine-grained (1x128 / 128x128) scaling: the
accuracy ablation behind the pages' outlier claim.  Oracle side, CPU only,
reported and never gated.

    python -m oracle.ablation [tiny decode]

What the pages claim: a single scale for a whole tensor, taken from its
max-abs value, is very sensitive to activation outliers [P2 paragraph 3];
smaller groups along K with their own scales accommodate outliers better
[P4 paragraph 3].  The pages print no figure for it.

The ablation quantises A and W of a workload two ways with the same cast
rule (``oracle.quant``: ``s = fl32(amax/448)``, ``r = min(fl32(448/amax),
FLT_MAX)``, ``fl32(x*r)`` clamped to +-448 and encoded to E4M3 with round to
nearest even), once with the fine-grained groups and once with one group per
tensor, dequantises exactly, multiplies in float64, and compares each
product with the float64 product of the unquantised BF16 operands.

Reading for "per-tensor": the group is the whole tensor (one scale for A,
one for W); nothing else changes.
"""
from __future__ import annotations

import sys

import numpy as np

from .e4m3 import e4m3_decode
from .gemm import dequant_act, dequant_w
from .quant import _scale_and_cast, f32_from_bf16, quant_act_1x128, quant_w_128x128


def quant_per_tensor(x_bits: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """BF16 tensor (any shape) -> E4M3 codes of the same shape and one float32
    scale: the 1x128 rule with the whole tensor as its single group."""
    x = f32_from_bf16(x_bits.reshape(-1)).reshape(x_bits.shape)
    a = np.max(np.abs(x)) if x.size else np.float32(0.0)
    q, s = _scale_and_cast(x[None], np.asarray(a, dtype=np.float32).reshape(1),
                           tuple(range(1, x.ndim + 1)))
    return q[0], np.float32(s[0])


def dequant_per_tensor(q: np.ndarray, s: np.float32) -> np.ndarray:
    """Codes and one scale to float64 values (exact)."""
    return e4m3_decode(q).astype(np.float64) * np.float64(s)


def product_errors(c: np.ndarray, ref: np.ndarray) -> dict:
    """Normwise relative error, and the elementwise relative error over the
    entries with ``|ref| > 1e-2 * rms(ref)`` (the workload gate's set): its
    maximum, 99th percentile and the share of entries above 1e-2."""
    ref = np.asarray(ref, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    normwise = float(np.linalg.norm(c - ref) / np.linalg.norm(ref))
    rms = float(np.sqrt(np.mean(ref * ref)))
    sel = np.abs(ref) > 1e-2 * rms
    rel = np.abs(c[sel] - ref[sel]) / np.abs(ref[sel])
    return {"normwise": normwise, "elementwise_max": float(rel.max()),
            "elementwise_p99": float(np.percentile(rel, 99)), "share_above_1e-2": float(np.mean(rel > 1e-2))}


def zero_share(q: np.ndarray, x_bits: np.ndarray) -> float:
    """Share of the nonzero inputs whose code is a zero (magnitude lost)."""
    nz = f32_from_bf16(x_bits.reshape(-1)) != 0
    return float(np.mean((q.reshape(-1)[nz] & 0x7F) == 0)) if nz.any() else 0.0


def regular_channel_error(a_hat: np.ndarray, a_bits: np.ndarray, outlier_cols) -> float:
    """Normwise relative error of the dequantised activations over the
    channels that are not outliers: what the outliers' scale costs the rest."""
    a = f32_from_bf16(a_bits).astype(np.float64)
    keep = np.ones(a.shape[1], dtype=bool)
    keep[np.asarray(outlier_cols, dtype=np.int64)] = False
    return float(np.linalg.norm(a_hat[:, keep] - a[:, keep]) / np.linalg.norm(a[:, keep]))


def ablate(a_bits: np.ndarray, w_bits: np.ndarray, outlier_cols=()) -> dict:
    """Both schemes on one dense GEMM ``A [M, K] @ W [N, K].T``; ``outlier_cols``
    names A's outlier channels for the regular-channel error."""
    ref = f32_from_bf16(a_bits).astype(np.float64) @ f32_from_bf16(w_bits).astype(np.float64).T
    qa, sa = quant_act_1x128(a_bits)
    qw, sw = quant_w_128x128(w_bits)
    a_hat = dequant_act(qa, sa)
    fine = a_hat @ dequant_w(qw, sw).T
    out = {"fine_grained": product_errors(fine, ref)}
    out["fine_grained"].update(a_zero_share=zero_share(qa, a_bits), w_zero_share=zero_share(qw, w_bits),
                               a_regular_error=regular_channel_error(a_hat, a_bits, outlier_cols))
    del fine
    ta, tsa = quant_per_tensor(a_bits)
    tw, tsw = quant_per_tensor(w_bits)
    a_hat = dequant_per_tensor(ta, tsa)
    tens = a_hat @ dequant_per_tensor(tw, tsw).T
    out["per_tensor"] = product_errors(tens, ref)
    out["per_tensor"].update(a_zero_share=zero_share(ta, a_bits), w_zero_share=zero_share(tw, w_bits),
                             a_regular_error=regular_channel_error(a_hat, a_bits, outlier_cols))
    return out


def run(name: str, seed: int = 0) -> dict:
    """The ablation on a named dense workload (``tiny`` or ``decode``)."""
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from synth import make_workload
    d = make_workload(name, seed=seed)
    return ablate(d["A"], d["W"], d["outlier_channels"])


def run_tiny_outliers(factor: float, seed: int = 0) -> dict:
    """The tiny workload with its 4 outlier channels scaled by ``factor``
    instead of 50 (the same draws, rescaled in float32, then rounded to
    BF16): how the gap grows with the outliers' size."""
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from synth import make_workload
    from synth.workloads import bf16_bits_from_f32
    d = make_workload("tiny", seed=seed)
    a = f32_from_bf16(d["A"]).copy()
    a[:, d["outlier_channels"]] *= np.float32(factor / 50.0)
    return ablate(bf16_bits_from_f32(a), d["W"], d["outlier_channels"])


def main(argv):
    names = argv or ["tiny", "decode"]
    cols = ["normwise", "elementwise_max", "elementwise_p99", "share_above_1e-2", "a_zero_share", "w_zero_share",
            "a_regular_error"]
    print("| workload | scaling | " + " | ".join(cols) + " |")
    print("|---|---" + "|---" * len(cols) + "|")
    runs = [(n, lambda n=n: run(n)) for n in names]
    if "tiny" in names:
        runs += [(f"tiny, outliers x{f:g}", lambda f=f: run_tiny_outliers(f)) for f in (1e3, 1e4)]
    for label, fn in runs:
        r = fn()
        for scheme in ("fine_grained", "per_tensor"):
            print(f"| {label} | {scheme} | " + " | ".join(f"{r[scheme][c]:.3e}" for c in cols) + " |", flush=True)


if __name__ == "__main__":
    main(sys.argv[1:])
