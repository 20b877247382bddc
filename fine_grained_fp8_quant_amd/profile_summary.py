"""Turn rocprofv3 CSV output into the short text summaries kept in profiles/.

    python -m fine_grained_fp8_quant_amd.profile_summary <out_dir> <workload>[:e8m0] [...]

<out_dir> holds, per workload, the output of the commands printed in each
summary: a kernel trace of bench.py (with bench.py's own JSON line saved
beside it), FETCH_SIZE / WRITE_SIZE counter passes of profile_workload.py
and, for the GEMM-bound workloads, three passes of utilisation counters.
Writes profiles/<workload>_kernels.md (<workload>_e8m0_kernels.md for the
power-of-two scale variant) and updates profiles/traffic.json with HBM bytes
per launch.

Timed steps: bench.py launches a 256-byte device copy (fgq_debug_copy) just
before and just after its timed region.  The per-call table averages only the
dispatches between those two copies, so it covers the same calls as the
HIP-event times of the bench line saved with the trace.

Traffic calibration: the counter passes also run a 1 GiB device copy
(fgq_debug_copy).  Its FETCH_SIZE and WRITE_SIZE against the known 1 GiB
read and 1 GiB written give the factors applied to every kernel.

Utilisation counters (per dispatch, then averaged per kernel):
  clock        GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration (launches of 200 us
               or more only)
  MFMA busy    SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8)
  co-issue     SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES
  waiting      SQ_WAIT_ANY / SQ_WAVE_CYCLES (wave-cycles waiting on anything)
  LDS conflict SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
  L2 hit       TCC_HIT / (TCC_HIT + TCC_MISS)
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
             "python -u bench.py --workload {w} --scales {sc} --steps 20 --warmup 5 --no-cpu-baseline "
             "> <out>/trace/{tag}/bench.json")
PMC_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc/{tag}/{c} -o pmc -- "
           "python -u -m fine_grained_fp8_quant_amd.profile_workload --workload {w} --scales {sc}")
UTIL_CMD = ("rocprofv3 --pmc {c} --output-format csv -d <out>/pmc/{tag}/{p} -o pmc -- "
            "python -u -m fine_grained_fp8_quant_amd.profile_workload --workload {w} --scales {sc}")
MODE_NAMES = {"0": "exact", "1": "fp8core", "2": "promote", "3": "incore"}
# utilisation counter passes: each fits one rocprofv3 run (at most 8 SQ,
# 4 TCC and 2 GRBM counters)
UTIL_PASSES = {
    "util": "GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
            "SQ_INSTS_LDS",
    "stall": "GRBM_GUI_ACTIVE SQ_WAVE_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE",
    "l2": "GRBM_GUI_ACTIVE TCC_HIT_sum TCC_MISS_sum",
}
N_XCD, N_SIMD = 8, 1024


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


def read_trace_timed(path, spans=False):
    """(kernel, duration us) of every dispatch between the first two marker
    copies (k_debug_copy) of a kernel trace, in dispatch order (with
    ``spans``: (kernel, start us, end us)); None when the trace holds fewer
    than two markers."""
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Dispatch_Id"]), short(r["Kernel_Name"]), int(r["Start_Timestamp"]) / 1e3,
                         int(r["End_Timestamp"]) / 1e3))
    rows.sort()
    marks = [i for i, row in enumerate(rows) if row[1].startswith("k_debug_copy")]
    if len(marks) < 2:
        return None
    timed = rows[marks[0] + 1:marks[1]]
    if spans:
        return [(k, t0, t1) for _, k, t0, t1 in timed]
    return [(k, t1 - t0) for _, k, t0, t1 in timed]


def call_key(kname, e8, mode):
    """The C-ABI call a kernel belongs to (GEMMs with their mode), or None;
    kernels that carry no mode belong to ``mode``."""
    api, md = api_of(kname, e8)
    return None if api is None else api + (f"[{md or mode}]" if "gemm" in api and (md or mode) else "")


def call_spans(timed, e8, mode):
    """Average span (first kernel's start to last kernel's end, us) of each
    C-ABI call in the timed dispatches, consecutive kernels of one call
    grouped; kernels that carry no mode belong to ``mode``."""
    spans = defaultdict(list)
    cur, t_start, t_end = None, 0.0, 0.0
    for k, t0, t1 in timed:
        key = call_key(k, e8, mode)
        if key != cur:
            if cur is not None:
                spans[cur].append(t_end - t_start)
            cur, t_start = key, t0
        t_end = t1
    if cur is not None:
        spans[cur].append(t_end - t_start)
    return {k: sum(v) / len(v) for k, v in spans.items() if k is not None}


def call_gaps(timed, e8, mode, target):
    """Average idle time (us) of the GPU in the timed dispatches: right before
    the first kernel of each ``target`` call, right after its last, and
    between consecutive kernels that are not at its edges.  None where no
    such gap occurs."""
    before, after, other = [], [], []
    prev_key, prev_end = None, None
    for k, t0, t1 in timed:
        key = call_key(k, e8, mode)
        if prev_end is not None:
            gap = t0 - prev_end
            if key == target and prev_key != target:
                before.append(gap)
            elif prev_key == target and key != target:
                after.append(gap)
            elif key != target and prev_key != target:
                other.append(gap)
        prev_key, prev_end = key, t1
    return tuple(sum(v) / len(v) if v else None for v in (before, after, other))


def read_counters(path):
    """{dispatch id: (kernel, duration ns, {counter: value})} of one --pmc pass."""
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            if d not in out:
                out[d] = (short(r["Kernel_Name"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]), {})
            out[d][2][r["Counter_Name"]] = float(r["Counter_Value"])
    return out


def util_metrics(passes):
    """Per-kernel averages of the utilisation ratios over the dispatches of
    the counter passes ({pass name: read_counters output})."""
    per = defaultdict(lambda: defaultdict(list))
    for name, disp in passes.items():
        for k, dur, c in disp.values():
            if k.startswith("k_debug_copy") or dur <= 0 or not c.get("GRBM_GUI_ACTIVE"):
                continue
            cyc = c["GRBM_GUI_ACTIVE"] / N_XCD
            m = per[k]
            if dur >= 200_000:
                # the counter also runs through the launch's set-up and
                # drain, which only long launches make negligible
                m["clock GHz"].append(cyc / dur)
            if name == "util":
                busy = c["SQ_VALU_MFMA_BUSY_CYCLES"]
                m["MFMA busy"].append(busy / (N_SIMD * cyc))
                if busy:
                    m["co-issue / MFMA busy"].append(c["SQ_VALU_MFMA_COEXEC_CYCLES"] / busy)
                if c["SQ_INSTS_MFMA"]:
                    m["VALU inst / MFMA inst"].append(c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"])
                    m["LDS inst / MFMA inst"].append(c["SQ_INSTS_LDS"] / c["SQ_INSTS_MFMA"])
            elif name == "stall":
                if c["SQ_WAVE_CYCLES"]:
                    m["waiting"].append(c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"])
                    m["waiting to issue"].append(c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"])
                if c["SQ_LDS_IDX_ACTIVE"]:
                    m["LDS conflict"].append(c["SQ_LDS_BANK_CONFLICT"] / c["SQ_LDS_IDX_ACTIVE"])
            elif name == "l2":
                tot = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
                if tot:
                    m["L2 hit"].append(c["TCC_HIT_sum"] / tot)
    return {k: {n: sum(v) / len(v) for n, v in m.items()} for k, m in per.items()}


def summarise(out_dir, spec, traffic):
    w, _, sc = spec.partition(":")
    sc = sc or "f32"
    e8 = sc == "e8m0"
    tag = w + ("_e8m0" if e8 else "")
    tdir = os.path.join(out_dir, "trace", tag)
    stats = read_stats(os.path.join(tdir, "trace_kernel_stats.csv"))
    timed = read_trace_timed(os.path.join(tdir, "trace_kernel_trace.csv"))
    bench = None
    if os.path.exists(os.path.join(tdir, "bench.json")):
        with open(os.path.join(tdir, "bench.json")) as f:
            lines = [ln for ln in f if ln.startswith("{")]
        bench = json.loads(lines[-1]) if lines else None
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
    util_passes = {p: os.path.join(out_dir, "pmc", tag, p, "pmc_counter_collection.csv") for p in UTIL_PASSES}
    util_passes = {p: path for p, path in util_passes.items() if os.path.exists(path)}
    cmds = ["    " + TRACE_CMD.format(w=w, sc=sc, tag=tag),
            "    " + PMC_CMD.format(w=w, sc=sc, tag=tag, c="FETCH_SIZE"),
            "    " + PMC_CMD.format(w=w, sc=sc, tag=tag, c="WRITE_SIZE")]
    cmds += ["    " + UTIL_CMD.format(w=w, sc=sc, tag=tag, p=p, c=UTIL_PASSES[p]) for p in util_passes]
    lines = [f"# {title}: kernel durations and HBM traffic (one MI355X)", "",
             "Commands (from the repository root; `<out>` is any scratch directory):", "", *cmds,
             "    python -m fine_grained_fp8_quant_amd.profile_summary <out> " + spec, ""]
    # one call of the C ABI can launch several kernels (split-K and its
    # reduction; the dense last-round split and its reduction): their
    # average durations add up to the call
    def per_call_table(rows):
        per_call = defaultdict(float)
        for name, avg in rows:
            api, mode = api_of(name, e8)
            if not api:
                continue
            modes = [mode] if mode or "gemm" not in api else (["promote", "incore"] if e8 else ["exact", "fp8core"])
            for md in modes:
                per_call[api + (f"[{md}]" if md else "")] += avg
        return per_call

    if timed is not None:
        mode = bench.get("gemm_mode") if bench else None
        tk = defaultdict(list)
        for k, us in timed:
            tk[k].append(us)
        lines += ["## Timed steps only (the dispatches between the two marker copies)", "",
                  "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for k, v in sorted(tk.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {k} | {len(v)} | {sum(v) / len(v):.1f} | {min(v):.1f} | {max(v):.1f} |")
        timed_spans = read_trace_timed(os.path.join(tdir, "trace_kernel_trace.csv"), spans=True)
        spans = call_spans(timed_spans, e8, mode)
        lines += ["", "Per call over the timed steps: the span from the call's first kernel start to its last kernel "
                  "end (what HIP events around the call measure, gaps between its kernels included):", "",
                  "| call | avg span us |", "|---|---|"]
        for key in sorted(spans):
            lines.append(f"| {key} | {spans[key]:.1f} |")
        if bench:
            rf = bench["roofline"]
            gk = rf["kernel"]
            gemm_api = [key for key in spans if key.startswith(("gemm", "grouped")) and key.endswith(f"[{mode}]")]
            ms_ev = bench["kernels"][gk]["ms"]
            lines += ["", "## The bench line of the traced run", "",
                      f"    roofline: bound {rf['bound']}, achieved {rf['achieved']:.1f} {rf['unit']}, "
                      f"peak {rf['peak']}, frac {rf['frac']:.4f}",
                      f"    {gk}: {ms_ev * 1e3:.1f} us per call (HIP events); "
                      f"ms_per_step {bench['ms_per_step']:.4f}", ""]
            ce = bench.get("ceilings") or {}
            if "mfma_fp8_tflops" in ce and "mfma_fp16_tflops" in ce:
                # boxes differ by several percent in clock; the loop rates of
                # the same run say which kind of box the trace came from
                lines += [f"Matrix-core loop rates of the same run (register-only, two waves per SIMD): FP8 "
                          f"{ce['mfma_fp8_tflops']:.0f} TFLOP/s at {ce['mfma_fp8_sclk_ghz']:.2f} GHz, FP16 "
                          f"{ce['mfma_fp16_tflops']:.0f} TFLOP/s at {ce['mfma_fp16_sclk_ghz']:.2f} GHz.", ""]
            if gemm_api:
                us_tr = spans[gemm_api[0]]
                frac_tr = rf["frac"] * (ms_ev * 1e3) / us_tr
                lines += [f"Recomputed from the trace: {gemm_api[0]} {us_tr:.1f} us per call, so frac = "
                          f"{rf['frac']:.4f} x {ms_ev * 1e3:.1f} / {us_tr:.1f} = {frac_tr:.4f} "
                          f"({(frac_tr / rf['frac'] - 1) * 100:+.1f}% against the line).", ""]
                if abs(frac_tr / rf["frac"] - 1) > 0.03:
                    g0, g1, go = call_gaps(timed_spans, e8, mode, gemm_api[0])
                    fmt = lambda g: "-" if g is None else f"{g:.1f} us"
                    lines += [f"The difference, {ms_ev * 1e3 - us_tr:.1f} us per call, lies outside the call's "
                              f"kernels: in this trace the GPU idles {fmt(g0)} before the call's first kernel and "
                              f"{fmt(g1)} after its last, where the HIP event markers of the timed call are "
                              f"processed, against {fmt(go)} on average between the other kernels of a step. The "
                              "events include that processing, the span does not.", ""]
    lines += ["## Kernel trace of the whole run (`--kernel-trace --stats`; includes warm-up calls)", "",
              "| kernel | calls | avg us | min us | max us | % of GPU time |", "|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, pct in stats:
        lines.append(f"| {name} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.1f} |")
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
    if util_passes:
        um = util_metrics({p: read_counters(path) for p, path in util_passes.items()})
        names = ["clock GHz", "MFMA busy", "co-issue / MFMA busy", "VALU inst / MFMA inst", "LDS inst / MFMA inst",
                 "waiting", "waiting to issue", "LDS conflict", "L2 hit"]
        lines += ["", "## Utilisation counters per launch (averaged over the launches of each kernel)", "",
                  "| kernel | " + " | ".join(names) + " |", "|---" * (len(names) + 1) + "|"]
        for k in sorted(um):
            vals = []
            for n in names:
                v = um[k].get(n)
                vals.append("-" if v is None else (f"{v:.2f}" if n.endswith(("GHz", "inst")) else f"{v * 100:.1f}%"))
            lines.append(f"| {k} | " + " | ".join(vals) + " |")
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
