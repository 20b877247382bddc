"""Benchmark of the fine-grained FP8 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole path over one batch of the workload, with
the BF16 inputs already resident in HBM:
  * prefill (default): quant_act_1x128(A 8192x7168) + quant_w_128x128(W
    18432x7168) + gemm_fp8_blockscaled -> C 8192x18432 BF16;
  * decode: the same three calls at A 64x7168;
  * grouped_up: quant A 32768x7168, quant W 32x4096x7168, grouped GEMM;
  * fused_down: fused_rmsnorm_quant(X 16384x7168) + quant A_down
    16384x2048 + quant W 32x7168x2048 + grouped down-projection GEMM;
  * dispatch: quant_dispatch_1x128 of 4096 tokens routed to 8 of 32 experts
    each (32768 expert-ordered FP8 rows) + quant W 32x4096x7168 + grouped
    up-projection GEMM on the dispatched rows;
  * moe_decode: the same for a 256-token decode batch (at most 256 rows per
    expert): the grouped GEMM is bound by reading the expert weights.
With --scales e8m0 every step uses the power-of-two scale variant (E8M0
scale bytes, applied by the FP8 matrix core); --mode then picks how the GEMM
accumulates (promote: per-chunk FP32 promotion; incore: in the matrix core).
Inputs rotate over several buffer sets so the 256 MB last-level cache
cannot serve one step from the previous one.  `value` is whole-step GEMM
throughput: GEMM FLOPs per step / step time.  The GEMM's per-call time comes
from fence-free HIP events around the GEMM call, on its launch stream, in
every timed step; each other call is timed after the timed steps in groups
of back-to-back calls, one event pair per group.  The one process prints one
JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOP/s (% FP8 MFMA peak); quant GB/s (% HBM peak)"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_FP16_TFLOPS = 2500.0     # MI355X dense FP16 MFMA (the exact-product GEMM mode runs on these)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SOURCE = os.path.join(ROOT, "fine_grained_fp8_quant_amd", "csrc", "gemm.hip")
QUANT_SOURCE = os.path.join(ROOT, "fine_grained_fp8_quant_amd", "csrc", "quant.hip")
DISPATCH_SOURCE = os.path.join(ROOT, "fine_grained_fp8_quant_amd", "csrc", "dispatch.hip")

WORKLOAD_TITLES = {
    "prefill": "dense prefill GEMM 8192x7168x18432 (A 1x128 + W 128x128 E4M3 quant + GEMM)",
    "decode": "decode GEMM 64x7168x18432 (A 1x128 + W 128x128 E4M3 quant + GEMM)",
    "grouped_up": "grouped MoE up-proj 32 experts, 32768 Zipf rows, K 7168, N 4096",
    "fused_down": "fused RMSNorm+quant 16384x7168, grouped MoE down-proj 32 experts, 16384 rows, K 2048, N 7168",
    "dispatch": "quantise-then-dispatch 4096 tokens x top-8 of 32 experts (K 7168) + grouped MoE up-proj, N 4096",
    "moe_decode": "decode-shaped MoE: 256 tokens x top-8 of 32 experts (<= 256 rows each), dispatch + grouped "
                  "up-proj K 7168, N 4096",
}


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="prefill", choices=sorted(WORKLOAD_TITLES))
    p.add_argument("--sets", type=int, default=0, help="rotating input sets (0 = enough to exceed 768 MB)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--scales", default="f32", choices=["f32", "e8m0"],
                   help="scale format: binary32 (a/448) or power-of-two E8M0 bytes")
    p.add_argument("--fused-a", action="store_true",
                   help="prefill/decode: quantise A inside the GEMM's A-load (gemm_bf16a_fp8_blockscaled) "
                        "instead of a separate quant_act_1x128 launch")
    p.add_argument("--mode", default=None, choices=["exact", "fp8core", "promote", "incore"],
                   help="GEMM accumulation. f32 scales: exact products (FP16 matrix cores, default) or FP8 "
                        "matrix cores; e8m0 scales: promote (default) or incore")
    args = p.parse_args()
    modes = {"f32": ("exact", "fp8core"), "e8m0": ("promote", "incore")}[args.scales]
    if args.mode is None:
        args.mode = modes[0]
    if args.mode not in modes:
        p.error(f"--mode {args.mode} does not apply to --scales {args.scales} (use {' or '.join(modes)})")
    if args.fused_a and (args.scales != "f32" or args.workload not in ("prefill", "decode")):
        p.error("--fused-a applies to the prefill and decode workloads with binary32 scales")
    return args


def sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


class TimingEvent:
    """A HIP event for timing only, recorded on torch's current stream.

    Created with hipEventDisableSystemFence: recording it performs no
    system-scope fence, so it neither writes back and invalidates the caches
    between the launches it brackets nor adds that work to the timeline (the
    decode GEMM, a 40 us call, read 2 us longer between fenced events).
    Elapsed times are read after a device synchronisation, so nothing relies
    on the fence.  The calls go to the HIP runtime torch has loaded (the one
    libfgq resolves to as well)."""

    FLAGS = 0x20000000          # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as maps:
                for line in maps:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("no HIP runtime is loaded in this process")
            lib = ctypes.CDLL(path)
            lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = lib
        return cls._hip

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def __init__(self):
        import ctypes
        self.ev = ctypes.c_void_p()
        self._check(self._lib().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS), "hipEventCreateWithFlags")

    def record(self):
        import torch
        self._check(self._lib().hipEventRecord(self.ev, torch.cuda.current_stream().cuda_stream), "hipEventRecord")

    def elapsed_time(self, end):
        """Milliseconds from this event to ``end`` (both complete)."""
        import ctypes
        ms = ctypes.c_float()
        self._check(self._lib().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "ev", None):
            self._hip.hipEventDestroy(self.ev)


class NoTimer:
    """Runs the launches and records nothing (device warm-up)."""

    def run(self, name, fn):
        return fn()


class Collect:
    """Runs the launches and keeps each one, per name, for replay."""

    def __init__(self):
        self.fns = {}

    def run(self, name, fn):
        self.fns.setdefault(name, []).append(fn)
        return fn()


def time_back_to_back(fns, n, groups=5):
    """Per-call milliseconds of the calls in ``fns`` (one per input set, used in
    turn): ``groups`` groups of ``n`` back-to-back calls, one HIP event pair
    per group, so the events' own device time is spread over n calls.
    Returns (mean, p10, median, p90) over the groups."""
    import torch
    pairs = []
    for _ in range(groups):
        s, e = TimingEvent(), TimingEvent()
        s.record()
        for j in range(n):
            fns[j % len(fns)]()
        e.record()
        pairs.append((s, e))
    torch.cuda.synchronize()
    t = np.array([s.elapsed_time(e) / n for s, e in pairs])
    return float(t.mean()), float(np.percentile(t, 10)), float(np.median(t)), float(np.percentile(t, 90))


class Timer:
    """HIP events around launches on the current stream, summed per name
    (with ``only``: around the launches whose name contains it, the others
    run untimed)."""

    def __init__(self, only=None):
        self.pairs = {}
        self.only = only

    def run(self, name, fn):
        if self.only is not None and self.only not in name:
            return fn()
        s, e = TimingEvent(), TimingEvent()
        s.record()
        out = fn()
        e.record()
        self.pairs.setdefault(name, []).append((s, e))
        return out

    def avg_ms(self):
        return {k: float(np.mean([s.elapsed_time(e) for s, e in v])) for k, v in self.pairs.items()}

    def spread_ms(self):
        """p10, median and p90 of each name's per-call durations."""
        out = {}
        for k, v in self.pairs.items():
            t = np.array([s.elapsed_time(e) for s, e in v])
            out[k] = {"p10": float(np.percentile(t, 10)), "median": float(np.median(t)),
                      "p90": float(np.percentile(t, 90))}
        return out


def build_sets(args):
    """Device inputs and outputs for the chosen workload, several copies."""
    import torch
    from synth import make_workload
    d = make_workload(args.workload, seed=args.seed)
    sets = []
    sb = 1 if args.scales == "e8m0" else 4      # bytes per stored scale
    if args.workload in ("prefill", "decode"):
        A, W = dev_bf16(d["A"]), dev_bf16(d["W"])
        M, K, N = d["M"], d["K"], d["N"]
        per_set = (A.numel() * 3 + W.numel() * 3 + M * N * 2)
        flops = 2.0 * M * N * K
        quant_bytes = {"quant_act_1x128": 3 * M * K + sb * M * K // 128,
                       "quant_w_128x128": 3 * N * K + sb * N * K // 16384}
        shape = {"M": M, "N": N, "K": K}
    elif args.workload == "grouped_up":
        A, W = dev_bf16(d["A"]), dev_bf16(d["W"])
        R, K, N, E = d["R"], d["K"], d["N"], d["E"]
        off = torch.from_numpy(d["offsets"]).cuda()
        per_set = A.numel() * 3 + W.numel() * 3 + R * N * 2
        flops = 2.0 * R * N * K
        quant_bytes = {"quant_act_1x128": 3 * R * K + sb * R * K // 128,
                       "quant_w_128x128": 3 * E * N * K + sb * E * N * K // 16384}
        shape = {"E": E, "rows": R, "N": N, "K": K, "counts": d["counts"].tolist()}
    elif args.workload in ("dispatch", "moe_decode"):
        X, W = dev_bf16(d["X"]), dev_bf16(d["W"])
        T, topk, E, K, N = d["T"], d["topk"], d["E"], d["K"], d["N"]
        ids = torch.from_numpy(d["ids"]).cuda()
        R = T * topk
        per_set = X.numel() * 2 + R * K + W.numel() * 3 + R * N * 2
        flops = 2.0 * R * N * K
        quant_bytes = {"quant_dispatch_1x128": 2 * T * K + R * K + sb * R * K // 128 + 4 * R + 4 * (E + 1) + 8 * R,
                       "quant_w_128x128": 3 * E * N * K + sb * E * N * K // 16384}
        shape = {"tokens": T, "topk": topk, "E": E, "rows": R, "N": N, "K": K}
    else:
        X, G = dev_bf16(d["X"]), dev_bf16(d["gamma"])
        A, W = dev_bf16(d["A"]), dev_bf16(d["W"])
        R, K, N, E = d["R"], d["K"], d["N"], d["E"]
        Mx, Kx = d["Mx"], d["Kx"]
        off = torch.from_numpy(d["offsets"]).cuda()
        per_set = X.numel() * 3 + A.numel() * 3 + W.numel() * 3 + R * N * 2
        flops = 2.0 * R * N * K
        quant_bytes = {"fused_rmsnorm_quant": 3 * Mx * Kx + sb * Mx * Kx // 128 + 2 * Kx,
                       "quant_act_1x128": 3 * R * K + sb * R * K // 128,
                       "quant_w_128x128": 3 * E * N * K + sb * E * N * K // 16384}
        shape = {"Mx": Mx, "Kx": Kx, "E": E, "rows": R, "N": N, "K": K, "counts": d["counts"].tolist()}
    if args.scales == "e8m0":
        quant_bytes = {k + "_e8m0": v for k, v in quant_bytes.items()}
    n_sets = args.sets or max(2, int(np.ceil(768e6 / per_set)))
    for i in range(n_sets):
        s = {}
        if args.workload in ("prefill", "decode", "grouped_up"):
            s["A"] = A if i == 0 else A.clone()
            s["W"] = W if i == 0 else W.clone()
        elif args.workload in ("dispatch", "moe_decode"):
            s["X"] = X if i == 0 else X.clone()
            s["W"] = W if i == 0 else W.clone()
            s["ids"] = ids
        else:
            s["X"] = X if i == 0 else X.clone()
            s["G"] = G
            s["A"] = A if i == 0 else A.clone()
            s["W"] = W if i == 0 else W.clone()
        if args.workload in ("grouped_up", "fused_down"):
            s["off"] = off
        sets.append(s)
    return d, sets, flops, quant_bytes, shape


def gemm_mode(fgq, name):
    return {"exact": fgq.GEMM_EXACT, "fp8core": fgq.GEMM_FP8_CORE, "promote": fgq.E8M0_PROMOTE,
            "incore": fgq.E8M0_IN_CORE}[name]


class Api:
    """The calls of one scale format under the names the step times them by."""

    def __init__(self, fgq, scales):
        import torch
        e8 = scales == "e8m0"
        sfx = "_e8m0" if e8 else ""
        self.sdtype = torch.uint8 if e8 else torch.float32
        self.names = {n: n + sfx for n in ("quant_act_1x128", "quant_w_128x128", "fused_rmsnorm_quant",
                                           "quant_dispatch_1x128")}
        self.names["gemm"] = "gemm_fp8_e8m0" if e8 else "gemm_fp8_blockscaled"
        self.names["grouped"] = "grouped_gemm_fp8_e8m0" if e8 else "grouped_gemm_fp8_blockscaled"
        self.quant_act = getattr(fgq, self.names["quant_act_1x128"])
        self.quant_w = getattr(fgq, self.names["quant_w_128x128"])
        self.fused = getattr(fgq, self.names["fused_rmsnorm_quant"])
        self.dispatch = getattr(fgq, self.names["quant_dispatch_1x128"])
        gemm, grouped = getattr(fgq, self.names["gemm"]), getattr(fgq, self.names["grouped"])
        kw = "accumulate" if e8 else "mode"
        self.gemm = lambda *a, mode, **k: gemm(*a, **{kw: mode}, **k)
        self.grouped = lambda *a, mode, **k: grouped(*a, **{kw: mode}, **k)


def make_step(args, fgq, d, n_sets, mode):
    """Allocates every output buffer up front; returns step(i, set, timer)
    running the whole path once on input set i."""
    import torch
    api = Api(fgq, args.scales)
    nm = api.names
    sdt = api.sdtype
    eps = d.get("eps", 0.0)
    outs = []
    for _ in range(n_sets):
        o = {}
        if args.workload in ("prefill", "decode"):
            M, K, N = d["M"], d["K"], d["N"]
            o["qa"] = torch.empty((M, K), dtype=torch.uint8, device="cuda")
            o["sa"] = fgq.act_scales(M, K, "cuda", sdt)
            o["qw"] = torch.empty((N, K), dtype=torch.uint8, device="cuda")
            o["sw"] = torch.empty((N // 128, K // 128), dtype=sdt, device="cuda")
            o["c"] = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            ws = fgq.gemm_workspace_bytes(M, N, K)
            o["ws"] = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda") if ws else None
        elif args.workload in ("dispatch", "moe_decode"):
            T, topk, K, N, E = d["T"], d["topk"], d["K"], d["N"], d["E"]
            R = T * topk
            o["qa"] = torch.empty((R, K), dtype=torch.uint8, device="cuda")
            o["sa"] = fgq.act_scales(R, K, "cuda", sdt)
            o["off"] = torch.empty(E + 1, dtype=torch.int32, device="cuda")
            o["src"] = torch.empty(R, dtype=torch.int32, device="cuda")
            o["dest"] = torch.empty(R, dtype=torch.int32, device="cuda")
            o["dws"] = torch.empty(max(fgq.quant_dispatch_workspace_bytes(T, topk, E, K), 1), dtype=torch.uint8,
                                   device="cuda")
            o["qw"] = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
            o["sw"] = torch.empty((E, N // 128, K // 128), dtype=sdt, device="cuda")
            o["c"] = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        else:
            R, K, N, E = d["R"], d["K"], d["N"], d["E"]
            if args.workload == "fused_down":
                o["qx"] = torch.empty((d["Mx"], d["Kx"]), dtype=torch.uint8, device="cuda")
                o["sx"] = fgq.act_scales(d["Mx"], d["Kx"], "cuda", sdt)
            o["qa"] = torch.empty((R, K), dtype=torch.uint8, device="cuda")
            o["sa"] = fgq.act_scales(R, K, "cuda", sdt)
            o["qw"] = torch.empty((E, N, K), dtype=torch.uint8, device="cuda")
            o["sw"] = torch.empty((E, N // 128, K // 128), dtype=sdt, device="cuda")
            o["c"] = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        outs.append(o)

    def step(i, s, t):
        o = outs[i]
        if args.workload in ("dispatch", "moe_decode"):
            t.run(nm["quant_dispatch_1x128"],
                  lambda: api.dispatch(s["X"], s["ids"], d["E"], q=o["qa"], s=o["sa"], offsets=o["off"],
                                       row_src=o["src"], dest=o["dest"], workspace=o["dws"]))
            t.run(nm["quant_w_128x128"], lambda: api.quant_w(s["W"], q=o["qw"], s=o["sw"]))
            t.run(nm["grouped"], lambda: api.grouped(o["qa"], o["sa"], o["qw"], o["sw"], o["off"], out=o["c"],
                                                     mode=mode))
            return
        if args.workload == "fused_down":
            t.run(nm["fused_rmsnorm_quant"], lambda: api.fused(s["X"], s["G"], eps, q=o["qx"], s=o["sx"]))
        if args.fused_a:
            t.run(nm["quant_w_128x128"], lambda: api.quant_w(s["W"], q=o["qw"], s=o["sw"]))
            t.run("gemm_bf16a_fp8_blockscaled",
                  lambda: fgq.gemm_bf16a_fp8_blockscaled(s["A"], o["qw"], o["sw"], out=o["c"], workspace=o["ws"],
                                                         mode=mode))
            return
        t.run(nm["quant_act_1x128"], lambda: api.quant_act(s["A"], q=o["qa"], s=o["sa"]))
        t.run(nm["quant_w_128x128"], lambda: api.quant_w(s["W"], q=o["qw"], s=o["sw"]))
        if args.workload in ("prefill", "decode"):
            t.run(nm["gemm"], lambda: api.gemm(o["qa"], o["sa"], o["qw"], o["sw"], out=o["c"], workspace=o["ws"],
                                               mode=mode))
        else:
            t.run(nm["grouped"], lambda: api.grouped(o["qa"], o["sa"], o["qw"], o["sw"], s["off"], out=o["c"],
                                                     mode=mode))
    step.outputs = outs
    return step


def measured_ceilings(fgq):
    """The matrix cores' sustained rate on register-only loops over every
    SIMD (two waves each), and the shader clock the waves measured meanwhile:
    the ceiling this box reaches, beside the nominal peaks."""
    import torch
    out = {}
    fgq.debug_mfma_loop(0, 200)                    # wake the clocks
    for kind, key in ((0, "mfma_fp8_tflops"), (1, "mfma_fp16_tflops"), (2, "mfma_fp16_32x32_tflops")):
        r = fgq.debug_mfma_loop(kind, 4000 if kind == 0 else 8000, waves=2048)
        out[key] = r["tflops"]
        out[key.replace("tflops", "sclk_ghz")] = r["sclk_ghz"]
    torch.cuda.synchronize()
    out["note"] = ("register-only MFMA loops, 2048 waves (two per SIMD), 8 independent operations per round; "
                   "clock = s_memtime / s_memrealtime (100 MHz) over the loop")
    return out


def bf16_product_error(args, d, s0, c):
    """Normwise error of the step's BF16 output against the float64 product of
    the unquantised BF16 operands, on sampled rows (reported, not gated)."""
    import torch
    rng = np.random.default_rng(1)
    if args.workload in ("prefill", "decode"):
        A, W = s0["A"], s0["W"]
        rows = np.sort(rng.choice(A.shape[0], min(64, A.shape[0]), replace=False))
        ref = A[rows].double() @ W.double().t()
        got = c[rows].double()
    elif args.workload in ("grouped_up", "fused_down"):
        A, W, off = s0["A"], s0["W"], d["offsets"]
        rows = np.sort(rng.choice(A.shape[0], 64, replace=False))
        expert = np.searchsorted(off, rows, side="right") - 1
        ref = torch.stack([A[int(r)].double() @ W[int(e)].double().t() for r, e in zip(rows, expert)])
        got = c[rows].double()
    else:
        return None   # dispatch workloads: rows are expert-ordered copies of token rows
    err = float(torch.linalg.norm(got - ref) / torch.linalg.norm(ref))
    return {"normwise_vs_unquantised_bf16_product": err, "rows_sampled": len(rows),
            "note": "float64 product of the BF16 operands; reported, not gated"}


PREWARM_S = 0.5      # untimed device warm-up before the counted warm-up steps
CPU_TARGET_S = 10.0   # the oracle's sample grows in whole units until it has run this long


def cpu_baseline(args, d):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole units of it (1024-row blocks of the dense GEMM, whole experts
    largest first), added until about CPU_TARGET_S seconds have run."""
    import oracle
    e8 = args.scales == "e8m0"
    q_act = oracle.quant_act_1x128_e8m0 if e8 else oracle.quant_act_1x128
    q_w = oracle.quant_w_128x128_e8m0 if e8 else oracle.quant_w_128x128
    gemm_ref = oracle.gemm_e8m0_ref if e8 else oracle.gemm_ref
    q_disp = oracle.quant_dispatch_e8m0_ref if e8 else oracle.quant_dispatch_ref
    fused = oracle.fused_rmsnorm_quant_e8m0 if e8 else oracle.fused_rmsnorm_quant
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        blas_threads = max([p.get("num_threads", 1) for p in blas] or [1])
        blas_name = ",".join(sorted({p.get("internal_api", "?") for p in blas})) or "?"
    except Exception:
        blas_threads, blas_name = 1, "?"
    cpu_model = "?"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    t0 = time.perf_counter()
    flops = 0.0
    if args.workload in ("prefill", "decode"):
        K, N, M = d["K"], d["N"], d["M"]
        qw, sw = q_w(d["W"])
        rows = 0
        while rows < M and (rows == 0 or time.perf_counter() - t0 < CPU_TARGET_S):
            r1 = min(M, rows + 1024)
            qa, sa = q_act(d["A"][rows:r1])
            gemm_ref(qa, sa, qw, sw)
            flops += 2.0 * (r1 - rows) * N * K
            rows = r1
        sample = f"quant W (all {N} rows), then A rows 0..{rows - 1} of {M}: quant A, float64 GEMM against all of W"
    else:
        K, N = d["K"], d["N"]
        if args.workload in ("dispatch", "moe_decode"):
            offsets, row_src, _ = oracle.dispatch_ref(d["ids"], d["E"])
            counts = np.diff(offsets)
        else:
            offsets, counts = d["offsets"], d["counts"]
        if args.workload == "fused_down":
            fused(d["X"][:1024], d["gamma"], d["eps"])
        done = []
        for e in np.argsort(-counts, kind="stable"):
            if done and time.perf_counter() - t0 >= CPU_TARGET_S:
                break
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 == r0:
                continue
            if args.workload in ("dispatch", "moe_decode"):
                toks = row_src[r0:r1].astype(np.int64) // d["topk"]
                qa, sa, _, _, _ = q_disp(d["X"][toks], np.full((r1 - r0, 1), e, np.int32), d["E"])
            else:
                qa, sa = q_act(d["A"][r0:r1])
            qw, sw = q_w(d["W"][e])
            gemm_ref(qa, sa, qw, sw)
            flops += 2.0 * (r1 - r0) * N * K
            done.append((int(e), r1 - r0))
        sample = (("routing of all tokens, then " if args.workload in ("dispatch", "moe_decode") else "")
                  + ("fused RMSNorm of 1024 rows, then " if args.workload == "fused_down" else "")
                  + f"{len(done)} experts, largest first ({sum(r for _, r in done)} rows: "
                  + ", ".join(f"e{e}:{r}" for e, r in done) + f") x {N} weight rows, full K={K}: "
                  + ("dispatch quant" if args.workload in ("dispatch", "moe_decode") else "quant A")
                  + ", quant W_e, float64 GEMM")
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(blas_threads, 1)), "kind": "oracle",
            "sample": sample + f"; {dt:.1f} s; quantisation single-threaded NumPy, GEMM float64 BLAS ({blas_name}, "
                      f"{blas_threads} threads)" + ("; E8M0 scales" if e8 else ""),
            "seconds": dt, "host_cores_available": cores, "cpu_model": cpu_model, "blas": blas_name,
            "blas_threads": int(blas_threads), "quant_threads": 1}


def traffic_for(kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (key "<workload>/<kernel>[<mode>]"), only if the kernel source is
    unchanged since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except Exception:
        return None
    entry = t.get(kernel)
    if not entry:
        return None
    src = GEMM_SOURCE if "gemm" in kernel else (DISPATCH_SOURCE if "dispatch" in kernel else QUANT_SOURCE)
    if entry.get("source_sha") != sha(src):
        return None
    return entry.get("bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fine_grained_fp8_quant_amd as fgq
    fgq.load_library()
    torch.cuda.set_device(0)
    print(f"[bench] building {args.workload} inputs", file=sys.stderr, flush=True)
    d, sets, flops, quant_bytes, shape = build_sets(args)
    step = make_step(args, fgq, d, len(sets), gemm_mode(fgq, args.mode))
    # Device warm-up, untimed: the chip takes tens of milliseconds of
    # sustained load to settle its clocks (after an idle gap of 25 ms a 1.75 ms
    # prefill GEMM ran 2.1-2.37 ms and needed about fifteen calls to settle),
    # so the step is repeated for PREWARM_S of wall time before the counted
    # warm-up steps, and the timed steps follow the warm-up steps with no host
    # work in between beyond one synchronisation.
    #
    # Each event marker still adds its processing to the device timeline (in
    # a kernel trace the GPU idles about 4.5 us at a marker, under 1 us
    # between unmarked kernels of a step).  The timed steps therefore carry
    # events around the GEMM call only (the roofline's kernel); the other
    # calls are timed right after, in groups of back-to-back calls with one
    # event pair per group (time_back_to_back).
    timer = Timer(only="gemm")
    # A 256-byte device copy before the timed steps, between them and the
    # per-call pass, and after it: in a kernel trace of this run, the
    # dispatches between the first two copies are exactly the timed steps.
    mark = torch.zeros(512, dtype=torch.uint8, device="cuda")
    start, end = TimingEvent(), TimingEvent()
    n_pre, t_pre = 0, time.perf_counter()
    while time.perf_counter() - t_pre < PREWARM_S:
        for _ in range(4):
            step(n_pre % len(sets), sets[n_pre % len(sets)], NoTimer())
            n_pre += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i % len(sets), sets[i % len(sets)], NoTimer())
    fgq.debug_copy(mark[:256], mark[256:])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(args.steps):
        step(i % len(sets), sets[i % len(sets)], timer)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fgq.debug_copy(mark[:256], mark[256:])
    # the other calls: back-to-back groups over the input sets (each group's
    # calls read different sets in turn, as the steps do)
    col = Collect()
    for i in range(len(sets)):
        step(i, sets[i], col)
    calls = {name: time_back_to_back(fns, max(4, args.steps // 4)) for name, fns in col.fns.items()
             if "gemm" not in name}
    fgq.debug_copy(mark[:256], mark[256:])
    torch.cuda.synchronize()
    print(f"[bench] {n_pre} device warm-up steps, {args.warmup} counted warm-up steps, {len(sets)} input sets",
          file=sys.stderr, flush=True)
    ms_step = start.elapsed_time(end) / args.steps
    kern = {name: v[0] for name, v in calls.items()}
    spread = {name: {"p10": v[1], "median": v[2], "p90": v[3]} for name, v in calls.items()}
    last_c = step.outputs[0]["c"]
    # the roofline's kernel: its time in the timed steps themselves
    gemm_name = [k for k in timer.avg_ms() if "gemm" in k][0]
    kern[gemm_name] = timer.avg_ms()[gemm_name]
    spread[gemm_name] = timer.spread_ms()[gemm_name]
    gemm_ms = kern[gemm_name]
    achieved = flops / (gemm_ms * 1e-3) / 1e12
    # the contraction's own matrix-core dtype: exact products run on the FP16
    # cores, the other modes on the FP8 cores
    dtype_peak = PEAK_FP16_TFLOPS if args.mode == "exact" else PEAK_FP8_TFLOPS
    kernels = {}
    for k, ms in kern.items():
        if "gemm" in k:
            kernels[k] = {"ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
                          "frac_fp8_peak": flops / (ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
        else:
            gbs = quant_bytes[k] / (ms * 1e-3) / 1e9
            kernels[k] = {"ms": ms, "GB/s": gbs, "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                          "algorithmic_bytes": quant_bytes[k]}
        kernels[k]["ms_p10_median_p90"] = [spread[k]["p10"], spread[k]["median"], spread[k]["p90"]]
    traffic = traffic_for(f"{args.workload}/{gemm_name}[{args.mode}]")
    if args.workload in ("decode", "moe_decode"):
        # memory-bound: algorithmic bytes = W codes + weight scales + A codes + act scales + C
        if args.workload == "decode":
            M, N, K, nw = d["M"], d["N"], d["K"], 1
        else:
            M, N, K, nw = d["T"] * d["topk"], d["N"], d["K"], d["E"]
        sb = 1 if args.scales == "e8m0" else 4
        gbytes = nw * (N * K + sb * (N // 128) * (K // 128)) + M * K + sb * M * (K // 128) + 2 * M * N
        gbs = gbytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": gemm_name, "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": gbytes, "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "kernel": gemm_name, "achieved": achieved, "peak": PEAK_FP8_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / PEAK_FP8_TFLOPS,
                    "peak_note": "dense FP8 MFMA peak (the metric's); the exact mode's products run on the "
                                 "FP16 matrix cores" if args.mode == "exact" else "dense FP8 MFMA peak",
                    "algorithmic_flops": flops,
                    "frac_contraction_dtype_peak": achieved / dtype_peak,
                    "contraction_dtype": "fp16" if args.mode == "exact" else "fp8",
                    "traffic": traffic}
    print(f"[bench] timed {args.steps} steps: {ms_step:.3f} ms/step", file=sys.stderr, flush=True)
    accuracy = bf16_product_error(args, d, sets[0], last_c)
    # the other GEMM accumulation mode, timed alone (not part of the step)
    other = {"exact": "fp8core", "fp8core": "exact", "promote": "incore", "incore": "promote"}[args.mode]
    alt_step = make_step(args, fgq, d, len(sets), gemm_mode(fgq, other))
    # the same treatment as the timed steps: a device warm-up in this mode,
    # then the steps with events around the GEMM call only
    n_alt, t_alt = 0, time.perf_counter()
    while time.perf_counter() - t_alt < PREWARM_S / 2:
        for _ in range(4):
            alt_step(n_alt % len(sets), sets[n_alt % len(sets)], NoTimer())
            n_alt += 1
        torch.cuda.synchronize()
    alt_t = Timer(only="gemm")
    for i in range(args.steps):
        alt_step(i % len(sets), sets[i % len(sets)], alt_t)
    torch.cuda.synchronize()
    alt_ms = alt_t.avg_ms()[gemm_name]
    alt = {"mode": other, "ms": alt_ms, "TFLOP/s": flops / (alt_ms * 1e-3) / 1e12,
           "frac_fp8_peak": flops / (alt_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS}
    ceilings = measured_ceilings(fgq)
    if roofline["bound"] == "mfma":
        ceiling = ceilings["mfma_fp16_tflops" if args.mode == "exact" else "mfma_fp8_tflops"]
        roofline["frac_measured_ceiling"] = achieved / ceiling
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(args, d)
    line = {
        "metric": METRIC,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 codes; " + ("products on fp16 matrix cores (exact)" if args.mode == "exact"
                                   else "fp8 matrix cores") + "; "
                 + {"exact": "fp32 scales, fp32 accumulate", "fp8core": "fp32 scales, fp32 accumulate",
                    "promote": "e8m0 scales applied by the unit, fp32 accumulate",
                    "incore": "e8m0 scales applied by the unit, accumulate in the matrix core"}[args.mode],
        "data": "synthetic (seeded, shapes and distributions of the named workload)",
        "config": {"workload": WORKLOAD_TITLES[args.workload], **{k: v for k, v in shape.items() if k != "counts"},
                   "scales": args.scales, "fused_a": bool(args.fused_a), "input_sets": len(sets)},
        "roofline": roofline,
        "kernels": kernels,
        "gemm_mode": args.mode,
        "gemm_other_mode": alt,
        "cpu_baseline": cpu,
        "accuracy": accuracy,
        "ceilings": ceilings,
        "timing": "value and ms_per_step: the timed steps, fence-free HIP events around the GEMM call only "
                  "(each marker still adds its processing to the timeline); kernels: the GEMM's per-call time "
                  "from those steps, "
                  "each other call's from five groups of back-to-back calls over the input sets, one event pair "
                  "per group (mean; p10 / median / p90 over the groups)",
        "wall_s_timed": wall,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
