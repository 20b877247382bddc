"""A short, fixed run of the hot path for hardware-counter profiling:

    rocprofv3 --pmc <counters> -- python -m fine_grained_fp8_quant_amd.profile_workload [--workload prefill] [--scales e8m0]

Quantises (or, for the dispatch workload, quantises and dispatches) the
workload's inputs, runs each GEMM mode --reps times, and runs
one 1 GiB device copy (fgq_debug_copy) whose FETCH_SIZE / WRITE_SIZE
calibrate the traffic counters (known size: 1 GiB read, 1 GiB written).
"""
import argparse
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--workload", default="prefill",
                   choices=["prefill", "decode", "grouped_up", "fused_down", "dispatch", "moe_decode"])
    p.add_argument("--reps", type=int, default=3)
    p.add_argument("--scales", default="f32", choices=["f32", "e8m0"])
    p.add_argument("--modes", default=None, help="GEMM modes to run (default: both of the scale format)")
    args = p.parse_args()
    e8 = args.scales == "e8m0"
    if args.modes is None:
        args.modes = "promote,incore" if e8 else "exact,fp8core"
    import torch

    import fine_grained_fp8_quant_amd as fgq
    from synth import make_workload

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    d = make_workload(args.workload)
    sfx = "_e8m0" if e8 else ""
    if args.workload == "fused_down":
        getattr(fgq, "fused_rmsnorm_quant" + sfx)(dev(d["X"]), dev(d["gamma"]), d["eps"])
    if args.workload in ("dispatch", "moe_decode"):
        qa, sa, off, _, _ = getattr(fgq, "quant_dispatch_1x128" + sfx)(dev(d["X"]), torch.from_numpy(d["ids"]).cuda(),
                                                                        d["E"])
    else:
        qa, sa = getattr(fgq, "quant_act_1x128" + sfx)(dev(d["A"]))
        off = torch.from_numpy(d["offsets"]).cuda() if "offsets" in d else None
    qw, sw = getattr(fgq, "quant_w_128x128" + sfx)(dev(d["W"]))
    modes = {"exact": fgq.GEMM_EXACT, "fp8core": fgq.GEMM_FP8_CORE, "promote": fgq.E8M0_PROMOTE,
             "incore": fgq.E8M0_IN_CORE}
    for name in args.modes.split(","):
        mode = modes[name]
        for _ in range(args.reps):
            if e8 and off is None:
                fgq.gemm_fp8_e8m0(qa, sa, qw, sw, accumulate=mode)
            elif e8:
                fgq.grouped_gemm_fp8_e8m0(qa, sa, qw, sw, off, accumulate=mode)
            elif off is None:
                fgq.gemm_fp8_blockscaled(qa, sa, qw, sw, mode=mode)
            else:
                fgq.grouped_gemm_fp8_blockscaled(qa, sa, qw, sw, off, mode=mode)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    fgq.debug_copy(src, dst)
    torch.cuda.synchronize()
    print("profile_workload done", args.workload, args.scales, flush=True)


if __name__ == "__main__":
    main()
