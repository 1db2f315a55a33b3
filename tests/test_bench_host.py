"""bench.py's host-side logic on the CPU: the one-GPU refusal, the guard that
drops committed HBM-traffic counters taken on other kernel sources or another
workload, and the shape of the CPU oracle baseline record (all threads and
one thread)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (module import touches no GPU)
from linear_cross_entropy_bf16_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a configuration that was not measured


def write_summary(tmp_path, **fields):
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(fields))
    return str(p)


@pytest.mark.parametrize("kernel", sorted(bench.TRAFFIC))
def test_traffic_is_used_only_for_its_sources_and_workload(tmp_path, monkeypatch, kernel):
    path = write_summary(tmp_path, workload="wl_a", kernel_source_hash=bench.kernel_source_hash(kernel),
                         hbm_bytes_per_launch=12345)
    monkeypatch.setitem(bench.TRAFFIC, kernel, (path, bench.TRAFFIC[kernel][1]))
    assert bench.measured_traffic("wl_a", kernel) == 12345
    assert bench.measured_traffic("wl_b", kernel) is None          # another workload
    path = write_summary(tmp_path, workload="wl_a", kernel_source_hash="0" * 16,
                         hbm_bytes_per_launch=12345)
    assert bench.measured_traffic("wl_a", kernel) is None          # other kernel sources
    monkeypatch.setitem(bench.TRAFFIC, kernel, (str(tmp_path / "missing.json"), bench.TRAFFIC[kernel][1]))
    assert bench.measured_traffic("wl_a", kernel) is None          # no summary


@pytest.mark.parametrize("kernel", sorted(bench.TRAFFIC))
def test_source_hash_covers_every_listed_source(kernel):
    names = bench.TRAFFIC[kernel][1]
    assert all(os.path.exists(os.path.join(bench._CSRC, n)) for n in names)
    assert len(bench.kernel_source_hash(kernel)) == 16


def test_committed_summaries_name_their_workloads():
    for kernel, (path, _) in bench.TRAFFIC.items():
        t = json.load(open(path))
        assert t["workload"] in W.WORKLOADS or t["workload"] in W.CE_WORKLOADS, kernel
        assert t["hbm_bytes_per_launch"] > 0


def test_cpu_baseline_record():
    wl = W.WORKLOADS["tiny_f32"]
    inp = W.generate(wl)
    rec = bench.cpu_baseline(wl, inp, 32)
    assert rec["kind"] == "oracle" and rec["unit"] == "tokens/s"
    assert rec["value"] > 0 and rec["cores"] >= 1
    assert "first 32 of" in rec["sample"]
    assert rec["nproc"] >= 1
    assert rec["one_thread"]["rows"] == 16 and rec["one_thread"]["value"] > 0


def test_cpu_baseline_record_logits():
    wl = next(iter(W.CE_WORKLOADS.values()))
    inp = W.generate_logits(wl, n=8)
    rec = bench.cpu_baseline_ce(wl, inp, 4)
    assert rec["kind"] == "oracle" and rec["value"] > 0
    assert "first 4 of" in rec["sample"]
    assert rec["one_thread"]["rows"] == 1 and rec["one_thread"]["value"] > 0
