"""The benchmark's command-line contract: one JSON line with its fixed set
of fields (metric, value, roofline, CPU baseline ...), and a clear refusal
of more than one GPU."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stdout


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    print("bench contract: python bench.py --steps 4 --warmup 1 --cpu-seconds 1", flush=True)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4",
                        "--warmup", "1", "--cpu-seconds", "1"],
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=110)
    assert p.returncode == 0, p.stderr[-3000:]
    lines = [x for x in p.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, p.stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 4 and d["warmup"] == 1
    assert d["value"] > 0 and d["unit"] == "GB/s" and d["higher_is_better"] is True
    assert d["config"]["workload"] == "llama13b_bf16"
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1 and c["sample"]
