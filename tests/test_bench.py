"""bench.py's contract: the one-GPU refusal, the traffic record it reports only
for the kernel source the counters were taken on, the admitted-pair count
behind the feature FLOPs (CPU), the JSON line itself and the lines of the
build-comparison and head-count modes (GPU)."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr and res.stdout == ""


def test_source_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.h"
    a.write_text("int f(int x) {\n  return x + 1; // one more\n}\n/* block\n comment */\n")
    b.write_text("#define K 3\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(a), str(b)])
    h0 = bench.kernel_source_hash()
    a.write_text("int f(int x) {   return x + 1;   // a different comment\n}\n\n\n")
    assert bench.kernel_source_hash() == h0
    a.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    # the committed record belongs to the committed kernel source
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    assert bench.measured_traffic(2, False) == float(rec["hbm_bytes_per_launch"])
    # and it is within 1 % of the algorithmic bytes (Q, K, V read once, O and LSE written once)
    assert abs(rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"] - 1) < 0.01
    assert bench.measured_traffic(2, True) is None and bench.measured_traffic(3, True) is None
    stale = dict(rec, kernel_source_sha256="0" * 64)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.measured_traffic(2, False) is None


@pytest.mark.parametrize("L", [1, 2, 7, 64, 130])
@pytest.mark.parametrize("wl,wr,causal", [(-1, -1, False), (-1, -1, True), (0, 0, False), (3, 5, False),
                                          (10, 0, False), (-1, 4, False), (6, -1, False), (200, 200, False)])
def test_admitted_pairs_brute_force(L, wl, wr, causal):
    n = 0
    for i in range(L):
        for j in range(L):
            ok = (wl < 0 or j >= i - wl) and (wr < 0 or j <= i + wr)
            if causal:
                ok = ok and j <= i
            n += ok
    assert bench.admitted_pairs(L, wl, wr, causal) == n


def _run_bench(args):
    res = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                         text=True, timeout=600, cwd=ROOT)
    print(res.stderr[-1500:], flush=True)
    assert res.returncode == 0
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, "bench.py prints exactly one line"
    return json.loads(lines[0])


@pytest.mark.gpu
def test_bench_json_line():
    d = _run_bench(["--steps", "20", "--warmup", "20", "--cpu-stride", "256"])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 20
    assert d["unit"] == "TFLOP/s" and d["higher_is_better"] is True and d["vs_baseline"] is None
    assert d["dtype"] == "f16" and d["data"] == "synthetic" and "workload" in d["config"]
    flops = 4.0 * 4 * 8 * 4096 * 4096 * 64
    assert d["value"] == pytest.approx(flops / (d["ms_per_step"] * 1e-3) / 1e12, rel=1e-3)
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2516.6
    assert r["frac"] == pytest.approx(r["achieved"] / r["peak"], abs=1e-4)
    assert 0 < r["frac"] < 1
    # warm: the kernel duration is the back-to-back step time; the per-launch
    # event pairs are reported beside it and also time each launch's latency
    lt = d["launch_timing"]
    assert r["achieved"] == pytest.approx(d["value"], rel=1e-3)
    assert lt["step_us"] == pytest.approx(d["ms_per_step"] * 1e3, abs=0.01)
    assert lt["achieved_from"] == "the step time of back-to-back launches"
    assert 0 < lt["event_pair_min_us"] <= lt["event_pair_median_us"]
    assert r["traffic"] == bench.measured_traffic(2, False)
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "TFLOP/s" and c["cores"] >= 1 and c["value"] > 0
    assert "every 256th query row" in c["sample"]
    gt = d["graph_timing"]
    assert gt["launches_per_graph"] == 100 and gt["rounds"] == 9
    assert 0 < gt["min_us"] <= gt["median_us"] <= gt["max_us"]
    assert gt["tflops_at_median"] == pytest.approx(flops / (gt["median_us"] * 1e-6) / 1e12, rel=1e-3)
    # the graph's per-launch time and the back-to-back step time measure the same kernel
    assert gt["median_us"] == pytest.approx(d["ms_per_step"] * 1e3, rel=0.35)


@pytest.mark.gpu
def test_bench_feature_line():
    d = _run_bench(["--feature", "varlen", "--causal", "--steps", "10", "--warmup", "10", "--no-cpu-baseline",
                    "--graph", "20", "--graph-rounds", "3"])
    assert d["value"] > 0 and d["cpu_baseline"] is None and d["roofline"]["traffic"] is None
    assert d["graph_timing"]["launches_per_graph"] == 20 and d["graph_timing"]["median_us"] > 0
    assert d["config"]["causal"] is True and d["config"]["sequences"] == 24
    d0 = _run_bench(["--workload", "1", "--steps", "5", "--warmup", "5", "--no-cpu-baseline", "--graph", "0"])
    assert d0["graph_timing"] is None


@pytest.mark.gpu
def test_bench_compare_and_scan_lines():
    """The two diagnostic modes: one JSON line per build (--compare) and per
    head count (--scan-heads), each with its median per-launch time."""
    import attention_forward_fa2_amd as fa2
    lib = os.path.join(ROOT, "attention_forward_fa2_amd", "libfa2.so")
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "4", "--compare",
                          f"{lib},{lib}", "--steps", "40", "--block", "10", "--settle-ms", "50"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-1500:]
    lines = [json.loads(ln) for ln in res.stdout.splitlines() if ln.strip()]
    assert [d["build_index"] for d in lines] == [0, 1]
    for d in lines:
        assert d["rounds"] == 4 and d["median_us_per_launch"] > 0 and d["tflops"] > 0
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "4", "--scan-heads", "4,12",
                          "--steps", "40", "--block", "10", "--settle-ms", "50"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-1500:]
    lines = [json.loads(ln) for ln in res.stdout.splitlines() if ln.strip()]
    assert [d["scan_heads"] for d in lines] == [4, 12]
    for d in lines:
        assert d["workgroups"] == fa2.fa2_kernel_config(16, d["scan_heads"], 1000, 64, 0)["blocks"]
        assert d["median_us_per_launch"] > 0
        flops = 4.0 * 16 * d["scan_heads"] * 1000 * 1000 * 64
        assert d["tflops"] == pytest.approx(flops / (d["median_us_per_launch"] * 1e-6) / 1e12, rel=2e-3)
