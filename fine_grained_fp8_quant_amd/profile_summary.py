"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m fine_grained_fp8_quant_amd.profile_summary <out_dir> <workload>[:e8m0] [...]

<out_dir> holds, per workload, the output of the two commands printed in
each summary (a kernel trace of bench.py, and FETCH_SIZE / WRITE_SIZE
counter passes of profile_workload.py).  Writes profiles/<workload>_kernels.md
(<workload>_e8m0_kernels.md for the power-of-two scale variant) and updates
profiles/traffic.json with HBM bytes per launch.

Traffic calibration: the counter passes also run a 1 GiB device copy
(fgq_debug_copy).  Its FETCH_SIZE and WRITE_SIZE against the known 1 GiB
read and 1 GiB written give the factors applied to every kernel.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
SOURCES = {"gemm": "fine_grained_fp8_quant_amd/csrc/gemm.hip", "quant": "fine_grained_fp8_quant_amd/csrc/quant.hip",
           "dispatch": "fine_grained_fp8_quant_amd/csrc/dispatch.hip"}

TRACE_CMD = ("rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace/{tag} -o trace -- "
             "python -u bench.py --workload {w} --scales {sc} --steps 5 --warmup 2 --no-cpu-baseline")
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc/{tag}/{c} -o pmc -- "
           "python -u -m fine_grained_fp8_quant_amd.profile_workload --workload {w} --scales {sc}")
MODE_NAMES = {"0": "exact", "1": "fp8core", "2": "promote", "3": "incore"}


def sha(rel):
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def short(name: str) -> str:
    """Kernel display name without the argument list, with the GEMM mode spelled out."""
    base = name.split("(")[0].replace("void ", "").replace("fgq::", "")
    # k_name<TileCfg<BM, BN, waves_m, waves_n[, stages][, skip]>, mode[, emit]>
    m = re.match(r"(k_\w+)<TileCfg<(\d+), (\d+), \d+, \d+(?:, \d+)?(?:, (?:true|false))?>, (\d)(, true|, false)?>",
                 base)
    if m:
        emit = ",emit" if m.group(5) == ", true" else ""
        return f"{m.group(1)}[{m.group(2)}x{m.group(3)},{MODE_NAMES[m.group(4)]}{emit}]"
    return base


def api_of(kname: str, e8: bool):
    """(C-ABI call name, mode) a kernel belongs to; ``e8`` says the run used
    power-of-two scales (the routing kernels and the split-K reduction carry
    no scale type of their own)."""
    sfx = "_e8m0" if e8 else ""
    if kname.startswith("k_quant_act"):
        return "quant_act_1x128" + sfx, None
    if kname.startswith("k_quant_w"):
        return "quant_w_128x128" + sfx, None
    if kname.startswith("k_fused"):
        return "fused_rmsnorm_quant" + sfx, None
    if kname.startswith("k_dispatch"):
        return "quant_dispatch_1x128" + sfx, None
    mode = next((m for m in MODE_NAMES.values() if "," + m + "]" in kname or "," + m + "," in kname), None)
    if kname.startswith("k_gemm_fused_a"):
        return "gemm_bf16a_fp8_blockscaled", mode
    if kname.startswith("k_grouped"):
        return ("grouped_gemm_fp8_e8m0" if e8 else "grouped_gemm_fp8_blockscaled"), mode
    if kname.startswith("k_tail_reduce"):
        # the last-round reduction of the dense GEMM, named by its tile
        # configuration: 192-row tiles are the exact mode's, sixteen waves
        # (4 x 4) the in-core mode's
        api = "gemm_fp8_e8m0" if e8 else "gemm_fp8_blockscaled"
        if "<192," in kname:
            return api, "exact"
        if e8:
            return api, ("incore" if re.search(r"<256, 256, 4, 4\b", kname) else "promote")
        return api, "fp8core"
    if kname.startswith("k_gemm") or kname.startswith("k_splitk"):
        return ("gemm_fp8_e8m0" if e8 else "gemm_fp8_blockscaled"), mode
    return None, None


def read_stats(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((short(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def read_pmc(path):
    """dispatch-ordered list of (kernel, value in KiB)."""
    out = []
    with open(path) as f:
        for r in csv.DictReader(f):
            out.append((int(r["Dispatch_Id"]), short(r["Kernel_Name"]), float(r["Counter_Value"])))
    out.sort()
    return [(k, v) for _, k, v in out]


def summarise(out_dir, spec, traffic):
    w, _, sc = spec.partition(":")
    sc = sc or "f32"
    e8 = sc == "e8m0"
    tag = w + ("_e8m0" if e8 else "")
    stats = read_stats(os.path.join(out_dir, "trace", tag, "trace_kernel_stats.csv"))
    fetch = read_pmc(os.path.join(out_dir, "pmc", tag, "FETCH_SIZE", "pmc_counter_collection.csv"))
    write = read_pmc(os.path.join(out_dir, "pmc", tag, "WRITE_SIZE", "pmc_counter_collection.csv"))
    gib_kib = 1024 * 1024
    f_copy = [v for k, v in fetch if k.startswith("k_debug_copy")][0]
    w_copy = [v for k, v in write if k.startswith("k_debug_copy")][0]
    f_factor, w_factor = gib_kib / f_copy, gib_kib / w_copy
    per_kernel = defaultdict(lambda: [[], []])
    for k, v in fetch:
        per_kernel[k][0].append(v * f_factor * 1024)
    for k, v in write:
        per_kernel[k][1].append(v * w_factor * 1024)
    title = w + (" with power-of-two (E8M0) scales" if e8 else "")
    lines = [f"# {title}: kernel durations and HBM traffic (one MI355X)", "",
             "Commands (from the repository root; `<out>` is any scratch directory):", "",
             "    " + TRACE_CMD.format(w=w, sc=sc, tag=tag), "    " + PMC_CMD.format(w=w, sc=sc, tag=tag, c="FETCH_SIZE"),
             "    " + PMC_CMD.format(w=w, sc=sc, tag=tag, c="WRITE_SIZE"),
             "    python -m fine_grained_fp8_quant_amd.profile_summary <out> " + spec, "",
             "## Kernel trace (`--kernel-trace --stats`; includes warm-up calls)", "",
             "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in stats:
        lines.append(f"| {name} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f} |")
    # one call of the C ABI can launch several kernels (split-K and its
    # reduction; the dense last-round split and its reduction): their
    # average durations add up to the call
    per_call = defaultdict(float)
    for name, calls, avg, mn, mx, pct in stats:
        api, mode = api_of(name, e8)
        if not api:
            continue
        modes = [mode] if mode or "gemm" not in api else (["promote", "incore"] if e8 else ["exact", "fp8core"])
        for md in modes:
            per_call[api + (f"[{md}]" if md else "")] += avg
    lines += ["", "Per call (sum of the average durations of the call's kernels):", "",
              "| call | avg us |", "|---|---|"]
    for key in sorted(per_call):
        lines.append(f"| {key} | {per_call[key]:.1f} |")
    lines += ["", "## HBM traffic per launch (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`)", "",
              f"Calibration from the 1 GiB copy in the same runs: FETCH_SIZE x{f_factor:.3f}, "
              f"WRITE_SIZE x{w_factor:.3f}.", "",
              "| kernel | launches | read MB | written MB |", "|---|---|---|---|"]
    sums = defaultdict(lambda: [0.0, 0.0, 0])
    for k, (fs, ws) in per_kernel.items():
        if k.startswith("k_debug_copy"):
            continue
        rd = sum(fs) / len(fs)
        wr = sum(ws) / len(ws) if ws else 0.0
        lines.append(f"| {k} | {len(fs)} | {rd / 1e6:.1f} | {wr / 1e6:.1f} |")
        api, mode = api_of(k, e8)
        if api:
            # the split-K reduction runs once per dense GEMM call in either mode
            modes = [mode] if mode or "gemm" not in api else (["promote", "incore"] if e8 else ["exact", "fp8core"])
            for md in modes:
                key = f"{w}/{api}" + (f"[{md}]" if md else "")
                sums[key][0] += rd
                sums[key][1] += wr
                sums[key][2] = sha(SOURCES["gemm" if "gemm" in api else ("dispatch" if "dispatch" in api else "quant")])
    for key, (rd, wr, src) in sums.items():
        traffic[key] = {"bytes_per_launch": rd + wr, "read_bytes": rd, "write_bytes": wr, "source_sha": src}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, f"{tag}_kernels.md"), "w") as f:
        f.write("\n".join(lines) + "\n")


def main():
    out_dir = sys.argv[1]
    tpath = os.path.join(PROFILES, "traffic.json")
    traffic = json.load(open(tpath)) if os.path.exists(tpath) else {}
    for w in sys.argv[2:]:
        summarise(out_dir, w, traffic)
    with open(tpath, "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
        f.write("\n")


if __name__ == "__main__":
    main()
