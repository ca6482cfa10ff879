"""bench.py's host logic on the CPU: the algorithmic work it divides by (closed forms of a
hand-built routing), the rocprofv3 summary (kernel table, copy-calibrated counter scales,
FFN sums), the traffic figure's source-hash gate, the oracle sample's sizing, and the refusal
of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from synth import MoEConfig  # noqa: E402


def test_algorithmic_work_closed_forms():
    # 4 tokens, K = 2, experts 1..2 local of 0..3: pairs (t, k) local where the id is 1 or 2
    cfg = MoEConfig("hand", 4, 256, 128, 4, 1, 2, 2, 16)
    idx = np.array([[1, 2], [0, 3], [2, 0], [3, 1]])
    w = bench.algorithmic_work(cfg, idx)
    N, T_act, H, I, K, T = 4, 3, 256, 128, 2, 4
    assert w["pairs"] == N
    assert w["ffn_flops"] == 6 * N * H * I
    assert w["dispatch_bytes"] == T_act * H * 2 + N * H * 2
    assert w["combine_bytes"] == N * H * 2 + T * H * 2 + T * K * 8
    assert w["ffn_bytes"] == 2 * 3 * H * I * 2 + N * H * 2 + 2 * N * I * 2 + N * H * 2
    fp8 = bench.algorithmic_work(cfg.with_(dtype="fp8"), idx)
    assert fp8["dispatch_bytes"] == T_act * H * 2 + N * H * (1 + 4 / 128)


def _write_csv(path, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=list(rows[0].keys()))
        wr.writeheader()
        wr.writerows(rows)


def test_summarize_profiles(tmp_path, monkeypatch):
    trace, fetch, write, out = (tmp_path / n for n in ("trace", "fetch", "write", "out"))
    for d in (trace, fetch, write):
        d.mkdir()
    A = "void moe::ffn_big_kernel<128, 8, false, true, true, false, 0, true>(moe::FfnArgs)"
    Y = "void moe::ffn_big_kernel<128, 8, false, false, true, false, 0, true>(moe::FfnArgs)"
    C = "void moe::combine_kernel<8>(moe::CombineArgs)"
    _write_csv(trace / "run_kernel_stats.csv", [
        {"Name": A, "Calls": "4", "AverageNs": "3000000", "MinNs": "2900000", "MaxNs": "3100000"},
        {"Name": Y, "Calls": "4", "AverageNs": "1500000", "MinNs": "1400000", "MaxNs": "1600000"},
        {"Name": C, "Calls": "4", "AverageNs": "240000", "MinNs": "230000", "MaxNs": "250000"},
    ])
    GiB_KiB = float(1 << 20)
    copy = "__amd_rocclr_copyBuffer"
    for d, name, half in ((fetch, "FETCH_SIZE", True), (write, "WRITE_SIZE", False)):
        reading = GiB_KiB / 2 if half else GiB_KiB      # FETCH_SIZE reads half of a copy's bytes here
        _write_csv(d / "run_counter_collection.csv", [
            {"Kernel_Name": copy, "Counter_Name": name, "Counter_Value": str(reading)} for _ in range(3)
        ] + [
            {"Kernel_Name": A, "Counter_Name": name, "Counter_Value": "1000"},
            {"Kernel_Name": A, "Counter_Name": name, "Counter_Value": "3000"},
            {"Kernel_Name": Y, "Counter_Name": name, "Counter_Value": "500"},
            {"Kernel_Name": C, "Counter_Name": name, "Counter_Value": "7777"},
        ])
    bench.summarize_profiles("hand", str(trace), str(fetch), str(write), str(out), ["cmd one", "cmd two"])
    txt = (out / "moe_layer_hand.txt").read_text()
    assert "cmd one" in txt and "cmd two" in txt
    assert "x2.000" in txt and "x1.000" in txt
    js = json.loads((out / "ffn_traffic_hand.json").read_text())
    # per-kernel average KiB x 1024 x scale, summed over the ffn_ kernels only
    assert js["fetch_bytes"] == pytest.approx(((1000 + 3000) / 2 + 500) * 1024 * 2.0)
    assert js["write_bytes"] == pytest.approx(((1000 + 3000) / 2 + 500) * 1024 * 1.0)
    assert js["hbm_bytes_per_ffn_call"] == pytest.approx(js["fetch_bytes"] + js["write_bytes"])
    assert js["ffn_avg_us"] == pytest.approx(4500.0)
    assert js["ffn_source_sha256_16"] == bench.kernel_source_hash()
    # the traffic figure is read back only while the FFN source is the one profiled
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "ffn_traffic_hand.json").write_text(json.dumps(js))
    assert bench.read_traffic("hand", js["ffn_source_sha256_16"]) == pytest.approx(js["hbm_bytes_per_ffn_call"])
    assert bench.read_traffic("hand", "0" * 16) is None
    assert bench.read_traffic("other", js["ffn_source_sha256_16"]) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_sizing(monkeypatch):
    # a stand-in oracle whose time per token falls with the sample size (as the real one's
    # matrix products do): the two probes size a first sample, which finishes in under half
    # the target, so it is grown once by the ratio and timed again
    import types

    clock = {"t": 0.0}

    def moe_layer(inp, tokens):
        n = len(tokens)
        clock["t"] += 0.5 + n * (0.004 if n <= 256 else 0.001)
        return types.SimpleNamespace(out=np.zeros((n, 4)))

    fake = types.SimpleNamespace(moe_layer=moe_layer, bf16_to_f64=lambda x: x, max_norm_rel_err=lambda a, b: 0.0)
    monkeypatch.setitem(sys.modules, "oracle", fake)
    monkeypatch.setattr(bench.time, "perf_counter", lambda: clock["t"])
    out = bench.cpu_baseline(None, max_tokens=100000, target_s=15.0)
    # probes: 64 -> 0.756 s, 256 -> 1.524 s: 4 ms per token, 0.5 s fixed -> 3624 tokens (14.5 / 0.004,
    # rounded down), which take 4.124 s (< 7.5 s) -> grown to 3624 * 15 / 4.124 = 13181 tokens, 13.68 s
    assert out["sample"].startswith("tokens 0..13180 ")
    assert "3624 tokens took 4.1 s" in out["sample"]
    assert out["value"] == pytest.approx(13181 / (0.5 + 13.181))
    # a sample capped by the workload is not grown
    clock["t"] = 0.0
    capped = bench.cpu_baseline(None, max_tokens=2000, target_s=15.0)
    assert capped["sample"].startswith("tokens 0..1999 ") and "took" not in capped["sample"]
