"""Host-side checks of bench.py (no GPU needed): the one-GPU refusal, the
traffic figure's source-hash gate, and the CPU-oracle baseline on a small
sample of a workload."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import kda_inputs  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_source_it_was_counted_on(tmp_path, monkeypatch):
    summary = {"kernel_source_sha256_16": "0123456789abcdef",
               "launches": {"f32_n64_rows1": {"hbm_bytes_per_launch": 102748081}}}
    path = tmp_path / "pmc.txt"
    path.write_text(json.dumps(summary))
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(path))
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0123456789abcdef")
    assert bench.pmc_traffic("f32_n64_rows1") == 102748081
    assert bench.pmc_traffic("f16_n64_rows1") is None          # no entry for that launch
    monkeypatch.setattr(bench, "kernel_hash", lambda: "fedcba9876543210")
    assert bench.pmc_traffic("f32_n64_rows1") is None          # counted on other sources
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.pmc_traffic("f32_n64_rows1") is None


def test_kernel_hash_covers_the_kernel_source_and_its_headers():
    from kda_gated_delta_decode_amd import profiling
    assert bench.kernel_hash() == profiling.kernel_hash()
    assert len(bench.kernel_hash()) == 16
    assert "kda_launch.h" in profiling.KERNEL_HEADERS and "kda_device.h" in profiling.KERNEL_HEADERS


def test_cpu_baseline_reports_the_oracle_on_a_bounded_sample():
    oracle = pytest.importorskip("oracle.kda_oracle")
    oracle.lib()
    inp = kda_inputs.make_inputs("small", 12, 4, 2, "f32", H=2, seed=3)
    res = bench.cpu_baseline(inp, 0.2)
    assert res["kind"] == "oracle" and res["unit"] == "GB/s" and res["cores"] == 1
    assert res["value"] > 0 and res["us_per_full_step"] > 0
    assert "of the 4 requests" in res["sample"]
    assert res["host_cpus_available"] >= 1 and isinstance(res["cpu_model"], str) and res["cpu_model"]
    par = res["parallel"]
    assert par["cores"] >= 1 and par["value"] > 0
    other = res["other_configs"]
    assert set(other) == {"batched_f32", "batched_f16", "spec_verify_f16", "layers69_f32_one_pass"}
    assert all(v["us_per_step"] > 0 and v["state_GB/s"] > 0 for v in other.values())
