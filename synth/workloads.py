"""The MoE-transformer-shaped synthetic workloads, seeded.

Every tensor is drawn from ``numpy.random.default_rng([seed, key])`` with a
fixed key per tensor role, so that the decode and prefill workloads share
one weight matrix and a tensor never depends on the order in which others
were drawn.  Values are drawn in float32, scaled in float32 and rounded to
BF16 (round to nearest, ties to even).  BF16 tensors are returned as their
raw ``uint16`` bit patterns.

Layouts: activations ``[rows, K]`` and weights ``[N, K]`` (per expert
``[E, N, K]``), both K-contiguous.  A weight written "K x N" in a workload
description is generated directly in its transposed ``[N, K]`` storage; the
entries are i.i.d., so the distribution is the same.

Readings of the workload descriptions (the descriptions give no more):
  * ``N(0, s)`` names the standard deviation ``s``.
  * "1% of channels as x30 outliers" means ``round(0.01 * K)`` channels,
    chosen without replacement, multiplied by 30 before BF16 rounding.
  * "per-token log-normal row scale (sigma 1)" multiplies row ``m`` by
    ``exp(g_m)``, ``g_m ~ N(0, 1)``.
  * Zipf(s=1.1) expert counts: see ``zipf_counts``.
  * The grouped down-projection continues the 16384-row RMSNorm batch: it
    routes 16384 rows, with its own ``N(0, 1)`` activations ``[16384, 2048]``.
  * The dispatch workload routes 4096 tokens to 8 of 32 experts each (the
    pages activate 8 routed experts per token), so it produces the 32768
    routed rows of the grouped up-projection; expert popularity follows the
    same Zipf(1.1) profile (see ``route_ids``).
  * The decode-shaped MoE workload is the same routing for a 256-token decode
    batch, so every expert gets at most 256 rows (the pages' decode regime).
"""
from __future__ import annotations

import numpy as np

# One key per tensor role.  Keys never change: stored results depend on them.
_KEYS = {
    "A_tiny": 1, "W_tiny": 2, "outlier_tiny": 3,
    "A_decode": 10, "outlier_decode": 11, "W_dense": 12,
    "A_prefill": 20, "rowscale_prefill": 21,
    "counts_up": 30, "A_up": 31, "W_up": 32,
    "X_norm": 40, "gamma_norm": 41, "counts_down": 42, "A_down": 43, "W_down": 44,
    "X_dispatch": 50, "ids_dispatch": 51,
}


def rng_for(seed: int, key: str | int) -> np.random.Generator:
    """Independent generator for one tensor role."""
    k = _KEYS[key] if isinstance(key, str) else int(key)
    return np.random.default_rng([int(seed), k])


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to BF16, ties to even; return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def normal_bf16(shape, std: float, rng: np.random.Generator, chunk_rows: int = 4096) -> np.ndarray:
    """``N(0, std)`` in float32, rounded to BF16, generated in row chunks."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    flat = out.reshape(-1, shape[-1]) if len(shape) > 1 else out.reshape(1, -1)
    for r0 in range(0, flat.shape[0], chunk_rows):
        r1 = min(flat.shape[0], r0 + chunk_rows)
        z = rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32)
        if std != 1.0:
            z *= np.float32(std)
        flat[r0:r1] = bf16_bits_from_f32(z)
    return out


def _normal_bf16_with(shape, rng, col_scale=None, row_scale=None, chunk_rows=4096):
    """``N(0,1)`` times optional per-column / per-row float32 factors, to BF16."""
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        z = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        if col_scale is not None:
            z *= col_scale[None, :]
        if row_scale is not None:
            z *= row_scale[r0:r1, None]
        out[r0:r1] = bf16_bits_from_f32(z)
    return out


def zipf_counts(total_rows: int, n_experts: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Ragged per-expert row counts with a Zipf(s) profile and some empty experts.

    1. rank probabilities ``p_i ~ i**-s`` for ranks ``i = 1..E``, normalised;
    2. counts by rank from one multinomial draw of ``total_rows``;
    3. the two lightest ranks give their rows to rank 1, so they hold zero rows
       (a plain multinomial over 32 ranks leaves no expert empty, yet the
       workloads ask for some);
    4. ranks are assigned to expert ids by a random permutation.
    Returns int64 counts by expert id; they sum to ``total_rows``.
    """
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-float(s))
    p /= p.sum()
    c = rng.multinomial(int(total_rows), p).astype(np.int64)
    if n_experts >= 3:
        c[0] += c[-1] + c[-2]
        c[-1] = 0
        c[-2] = 0
    perm = rng.permutation(n_experts)
    counts = np.zeros(n_experts, dtype=np.int64)
    counts[perm] = c
    return counts


def route_ids(n_tokens: int, topk: int, n_experts: int, s: float, rng: np.random.Generator,
              drop: float = 0.0) -> np.ndarray:
    """Routing decisions: ``int32 [n_tokens, topk]`` expert ids.

    Each token picks ``topk`` distinct experts, drawn without replacement
    with probabilities ``~ rank**-s`` (ranks assigned to expert ids by a
    random permutation), by the Gumbel-top-k construction: the ``topk``
    largest of ``log p_e + G_e`` with i.i.d. standard Gumbel ``G_e``.  The
    slot order within a token is the draw order.  A fraction ``drop`` of the
    (token, slot) entries is then set to -1 (not routed).
    """
    ranks = np.arange(1, n_experts + 1, dtype=np.float64)
    p = ranks ** (-float(s))
    p /= p.sum()
    perm = rng.permutation(n_experts)
    logp = np.empty(n_experts)
    logp[perm] = np.log(p)
    g = rng.gumbel(size=(int(n_tokens), n_experts))
    keys = logp[None, :] + g
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :topk].astype(np.int32)
    if drop > 0.0:
        ids[rng.random(ids.shape) < drop] = -1
    return ids


def offsets_from_counts(counts: np.ndarray) -> np.ndarray:
    """``[0, cumsum(counts)]`` as int32 (row offsets of each expert)."""
    off = np.zeros(len(counts) + 1, dtype=np.int64)
    off[1:] = np.cumsum(counts)
    return off.astype(np.int32)


# name -> description; the sizes are the ones each workload is quoted at.
WORKLOADS = {
    "tiny": "A 128x512 N(0,1), 4 outlier channels x50; W [256,512] N(0,0.02); GEMM 128x256",
    "decode": "A 64x7168 N(0,1), 72 outlier channels x30; W [18432,7168] N(0,0.02); GEMM 64x18432",
    "prefill": "A 8192x7168 N(0,1) x exp(N(0,1)) per row; W [18432,7168] N(0,0.02); GEMM 8192x18432",
    "grouped_up": "32 experts, 32768 Zipf(1.1) rows; A [32768,7168] N(0,1); W [32,4096,7168] N(0,0.02)",
    "fused_down": "RMSNorm(eps 1e-6, gamma U(0.5,1.5)) + quant of X [16384,7168] N(0,2); "
                  "grouped down: 32 experts, 16384 Zipf(1.1) rows, A [16384,2048] N(0,1), W [32,7168,2048] N(0,0.02)",
    "dispatch": "quantise-then-dispatch: X [4096,7168] N(0,1) tokens, top-8 of 32 experts per token "
                "(Zipf(1.1) expert popularity) -> 32768 expert-ordered FP8 rows; W [32,4096,7168] as grouped_up",
    "moe_decode": "decode-shaped MoE up-projection: 256 tokens, top-8 of 32 experts (at most 256 rows per expert), "
                  "dispatched, grouped GEMM against W [32,4096,7168] as grouped_up",
}


def make_workload(name: str, seed: int = 0, rows: int | None = None, parts=None) -> dict:
    """Build the named workload's BF16 inputs (uint16 bits) and metadata.

    ``rows`` optionally truncates the activation rows (tests use it to keep
    oracle work small; the weights and, for grouped workloads, the
    per-expert profile are unchanged).  ``parts`` optionally restricts which
    tensors are generated (a set of keys of the returned dict).
    """
    want = (lambda k: True) if parts is None else (lambda k: k in parts)
    d: dict = {"name": name, "seed": seed}
    if name == "tiny":
        M, K, N = 128, 512, 256
        M = M if rows is None else rows
        cols = rng_for(seed, "outlier_tiny").choice(K, size=4, replace=False)
        cs = np.ones(K, dtype=np.float32)
        cs[cols] = 50.0
        d.update(M=M, K=K, N=N, outlier_channels=np.sort(cols))
        if want("A"):
            d["A"] = _normal_bf16_with((M, K), rng_for(seed, "A_tiny"), col_scale=cs)
        if want("W"):
            d["W"] = normal_bf16((N, K), 0.02, rng_for(seed, "W_tiny"))
    elif name in ("decode", "prefill"):
        K, N = 7168, 18432
        if want("W"):
            d["W"] = normal_bf16((N, K), 0.02, rng_for(seed, "W_dense"))
        if name == "decode":
            M = 64 if rows is None else rows
            n_out = int(round(0.01 * K))
            cols = rng_for(seed, "outlier_decode").choice(K, size=n_out, replace=False)
            cs = np.ones(K, dtype=np.float32)
            cs[cols] = 30.0
            d["outlier_channels"] = np.sort(cols)
            if want("A"):
                d["A"] = _normal_bf16_with((M, K), rng_for(seed, "A_decode"), col_scale=cs)
        else:
            M = 8192 if rows is None else rows
            g = rng_for(seed, "rowscale_prefill").standard_normal(8192).astype(np.float32)
            rs = np.exp(g).astype(np.float32)[:M]
            d["row_scale"] = rs
            if want("A"):
                d["A"] = _normal_bf16_with((M, K), rng_for(seed, "A_prefill"), row_scale=rs)
        d.update(M=M, K=K, N=N)
    elif name == "grouped_up":
        E, R, K, N = 32, 32768, 7168, 4096
        counts = zipf_counts(R, E, 1.1, rng_for(seed, "counts_up"))
        if rows is not None:
            counts = _shrink_counts(counts, rows)
            R = int(counts.sum())
        d.update(E=E, R=R, K=K, N=N, counts=counts, offsets=offsets_from_counts(counts))
        if want("A"):
            d["A"] = normal_bf16((R, K), 1.0, rng_for(seed, "A_up"))
        if want("W"):
            d["W"] = normal_bf16((E, N, K), 0.02, rng_for(seed, "W_up"))
    elif name == "fused_down":
        Mx, Kx = 16384, 7168
        E, R, K, N = 32, 16384, 2048, 7168
        Mx = Mx if rows is None else rows
        counts = zipf_counts(R, E, 1.1, rng_for(seed, "counts_down"))
        if rows is not None:
            counts = _shrink_counts(counts, rows)
            R = int(counts.sum())
        d.update(Mx=Mx, Kx=Kx, eps=1e-6, E=E, R=R, K=K, N=N, counts=counts,
                 offsets=offsets_from_counts(counts))
        if want("X"):
            d["X"] = normal_bf16((Mx, Kx), 2.0, rng_for(seed, "X_norm"))
        if want("gamma"):
            gam = rng_for(seed, "gamma_norm").uniform(0.5, 1.5, size=Kx).astype(np.float32)
            d["gamma"] = bf16_bits_from_f32(gam)
        if want("A"):
            d["A"] = normal_bf16((R, K), 1.0, rng_for(seed, "A_down"))
        if want("W"):
            d["W"] = normal_bf16((E, N, K), 0.02, rng_for(seed, "W_down"))
    elif name in ("dispatch", "moe_decode"):
        T, topk, E, K = (4096 if name == "dispatch" else 256), 8, 32, 7168
        T = T if rows is None else rows
        d.update(T=T, topk=topk, E=E, K=K, N=4096)
        if want("ids"):
            d["ids"] = route_ids(T, topk, E, 1.1, rng_for(seed, "ids_dispatch"))
        if want("X"):
            d["X"] = normal_bf16((T, K), 1.0, rng_for(seed, "X_dispatch"))
        if want("W"):  # the up-projection weights of the grouped_up workload (same key)
            d["W"] = normal_bf16((E, 4096, K), 0.02, rng_for(seed, "W_up"))
    else:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")
    return d


def _shrink_counts(counts: np.ndarray, rows: int) -> np.ndarray:
    """Scale a count profile down to about ``rows`` rows, keeping empty experts empty
    and every non-empty expert at least one row (so the ragged shape survives)."""
    total = counts.sum()
    c = np.floor(counts * (rows / total)).astype(np.int64)
    c[(counts > 0) & (c == 0)] = 1
    return c
