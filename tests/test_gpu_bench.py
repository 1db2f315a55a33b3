"""bench.py end to end on the GPU (needs an MI355X): one short run of the
small fp32 workload prints exactly one JSON line with every field of the
result record, a roofline of the forward kernel and the CPU oracle baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    print(f"\n[gpu-bench] bench.py {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


@pytest.mark.timeout(300)
def test_result_record_fields():
    d = run_bench("--workload", "tiny_f32", "--steps", "5", "--warmup", "1", "--cpu-rows", "16")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "ms_p50",
              "ms_min", "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 1
    assert d["unit"] == "tokens/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["dtype"] == "f32" and d["config"]["workload"] == "tiny_f32"
    assert d["vs_baseline"] is None            # the pages quote no figure for this shape
    assert d["ms_min"] <= d["ms_p50"] and d["ms_per_step"] > 0
    # value and ms_per_step are rounded separately
    assert abs(d["value"] - d["config"]["n"] / (d["ms_per_step"] * 1e-3)) <= 5e-3 * d["value"]
    r = d["roofline"]
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 157.3
    assert r["achieved"] > 0 and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None                # counters are committed for the headline shape only
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["unit"] == "tokens/s" and c["value"] > 0 and c["cores"] >= 1
    assert "first 16 of" in c["sample"]


@pytest.mark.timeout(300)
def test_logits_record_fields():
    d = run_bench("--workload", "ce_logits_llama3_8b_seq", "--steps", "3", "--warmup", "1",
                  "--cpu-rows", "16")
    assert d["config"]["workload"] == "ce_logits_llama3_8b_seq" and d["n_gpus"] == 1
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["frac"] < 1 and r["achieved"] > 0
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0
    assert "first 2 of" in c["sample"]        # the logits leg samples an eighth of --cpu-rows
