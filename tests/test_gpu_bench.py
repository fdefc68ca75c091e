"""The benchmark's JSON line on the GPU: one small run of bench.py in a child
process (the tiny workload, a short CPU baseline, the graph replay leg),
checked field by field against the contract the line follows."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_tiny():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--config", "tiny", "--steps", "5",
           "--warmup", "2", "--cpu-budget", "0.5", "--configs", "tiny_zipf", "--graph"]
    print("bench:", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=110, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["unit"] == "GB/s" and d["value"] > 0
    assert d["ms_per_step"] > 0 and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny")
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] <= 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["in_step_us"] > 0 and 0 < rf["in_step_frac"] <= 1
    want = rf["algorithmic_bytes"] / (rf["in_step_us"] * 1e3) / rf["peak"]
    assert abs(rf["in_step_frac"] - want) < 1e-4 + 1e-2 * want
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["sample"]
    assert cb["threads"] == 1 and cb["host_nproc"] >= 1 and isinstance(cb["host_cpu_model"], str)
    assert d["graph_step_us"] > 0
    # the headline is the mean of the K flushed steps
    assert len(d["us_p10_p50_p90"]) == 3 and d["back_to_back_us_per_step"] > 0
    assert abs(d["us_per_dispatch_combine"] - 1e3 * d["ms_per_step"]) < 0.01
    par = d["parity"]
    assert par["pass"] is True and par["plan_tables"] == "bit-exact"
    assert par["out_tokens_vs_oracle"] == 4 * 16 and par["out_elements_off"] == 0
    assert par["grouped_rows_checked"] == 4 * 16 * 2 and par["grouped_rows_bad"] == 0
    assert par["out_tokens_closed_form"] == 64 and par["out_tokens_closed_form_bad"] == 0
    c = d["configs"]["tiny_zipf"]
    assert c["flushed"] is False and c["us_back_to_back"] > 0 and c["parity"]["pass"] is True
    assert c["steps"] == 200 and c["effective_GBps"] > 0
