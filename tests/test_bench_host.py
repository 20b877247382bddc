"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the
source-hash gate on the committed traffic counters, and the shape of the
committed counter table."""
import json
import os
import re
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_is_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    table = {
        "prefill/gemm_fp8_blockscaled[exact]": {"bytes_per_launch": 123.0, "source_sha": bench.sha(bench.GEMM_SOURCE)},
        "decode/gemm_fp8_blockscaled[exact]": {"bytes_per_launch": 456.0, "source_sha": "0" * 16},
        "prefill/quant_act_1x128": {"bytes_per_launch": 7.0, "source_sha": bench.sha(bench.QUANT_SOURCE)},
        "dispatch/quant_dispatch_1x128": {"bytes_per_launch": 8.0, "source_sha": bench.sha(bench.QUANT_SOURCE)},
    }
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(table))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.traffic_for("prefill/gemm_fp8_blockscaled[exact]") == 123.0
    assert bench.traffic_for("decode/gemm_fp8_blockscaled[exact]") is None      # another source's counters
    assert bench.traffic_for("prefill/quant_act_1x128") == 7.0
    assert bench.traffic_for("dispatch/quant_dispatch_1x128") is None           # checked against dispatch.hip
    assert bench.traffic_for("grouped_up/grouped_gemm_fp8_blockscaled[exact]") is None  # no entry
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("prefill/gemm_fp8_blockscaled[exact]") is None


def test_committed_traffic_table_is_well_formed():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        table = json.load(f)
    key = re.compile(r"^(prefill|decode|grouped_up|fused_down|dispatch|moe_decode)/\w+(\[(exact|fp8core|promote|incore)\])?$")
    for k, v in table.items():
        assert key.match(k), k
        assert re.fullmatch(r"[0-9a-f]{16}", v["source_sha"]), k
        assert v["read_bytes"] > 0 and v["write_bytes"] > 0, k
        assert abs(v["bytes_per_launch"] - v["read_bytes"] - v["write_bytes"]) <= 1e-6 * v["bytes_per_launch"], k
    # the default bench line's roofline kernel has counters
    assert "prefill/gemm_fp8_blockscaled[exact]" in table
