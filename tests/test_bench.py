"""The benchmark's contract, on the CPU: the workload it times, the per-unit
figures of its roofline, the traffic record it trusts, the refusal of more
than one GPU, and the CPU oracle leg's fields."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_default_workload_spans_m_1_to_8192():
    cases = bench._cases("serving")
    assert len(cases) == 42
    ms = sorted({c[1] for c in cases})
    assert ms[0] == 1 and ms[-1] == 8192
    assert {c[0] for c in cases} == {"decode", "prefill", "hadamard"}
    names = [bench._case_name(c[0], c[2], c[1], c[5]) for c in cases]
    assert len(set(names)) == 42
    assert "prefill/gate_up/M=8192" in names and "hadamard/down/M=4096/hb=128" in names


def test_case_filter_and_unknown_case():
    only = {"decode/qkv/M=1", "prefill/down/M=2048"}
    got = {bench._case_name(c[0], c[2], c[1], c[5]) for c in bench._cases("serving", only=only)}
    assert got == only
    with pytest.raises(SystemExit):
        bench._cases("serving", only={"decode/qkv/M=3"})


def test_algorithmic_bytes_per_call():
    # 0.5625 B per weight element (E2M1 codes + one E4M3 scale per 16), 2 B per
    # activation and output element, 2 B per bias element
    M, N, K = 8, 6144, 4096
    assert bench._alg_bytes(M, N, K, True) == 0.5625 * N * K + 2 * M * K + 2 * M * N + 2 * N
    assert bench._alg_bytes(M, N, K, False, "mxfp4") == 0.53125 * N * K + 2 * M * K + 2 * M * N


def test_traffic_record_is_trusted_only_for_the_current_sources(monkeypatch):
    rec = None
    for path in bench.TRAFFIC_SUMMARIES:
        for line in open(path).read().splitlines():
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
    assert rec is not None and rec["bytes_per_launch"] > 0
    if rec["source_sha256"] == bench.source_digest():
        assert bench.measured_traffic(rec["kernel"]) == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_digest", lambda: "0" * 64)
    assert bench.measured_traffic(rec["kernel"]) is None
    assert bench.measured_traffic("no_such_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_fields_on_a_small_sample():
    out = bench.cpu_baseline("tiny", "nvfp4", n_rows=64, m_rows=16, runs=1)
    assert out["kind"] == "oracle" and out["unit"] == "TFLOP/s"
    assert out["value"] > 0 and out["cores"] >= 1
    assert out["one_thread"]["cores"] == 1 and out["one_thread"]["value"] > 0
    assert set(out["pass_seconds"]) == {"quantize", "gemm"}
    assert "tiny" in out["sample"]
