"""Host-side checks of the benchmark's contract (no GPU): a request for more than one GPU
is refused with a message, and the HBM traffic figure comes from the committed counter
summaries only when they were taken on the GEMM source that is built."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

WORKLOADS = ("ffn_up_T57600_5120x13824_k128", "ffn_up_T4096_5120x13824_k64", "ffn_down_T4096_13824x5120_k64")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("workload", WORKLOADS)
def test_traffic_read_from_profiles(workload, tmp_path, monkeypatch):
    """Each committed summary parses to a positive byte count; a summary whose GEMM
    source digest differs from the current source gives no figure, and so does a missing
    one."""
    for kernel in ("gemm_w4a4", "actprep"):
        path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
        assert os.path.exists(path), path
    # the parser, against a summary with a known figure and digest
    prof = tmp_path / "profiles"
    prof.mkdir()
    text = open(os.path.join(ROOT, "profiles", f"gemm_w4a4_{workload}_hbm_counters.md")).read()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "gemm_source_digest", lambda: "0123456789abcdef")
    fixed = "\n".join("source digest: 0123456789abcdef" if l.startswith("source digest:") else
                      ("hbm bytes per launch: 1.234500e+09" if l.startswith("hbm bytes per launch:") else l)
                      for l in text.splitlines())
    (prof / f"gemm_w4a4_{workload}_hbm_counters.md").write_text(fixed)
    assert bench.measured_traffic("gemm_w4a4", workload) == pytest.approx(1.2345e9)
    monkeypatch.setattr(bench, "gemm_source_digest", lambda: "fedcba9876543210")
    assert bench.measured_traffic("gemm_w4a4", workload) is None
    assert bench.measured_traffic("gemm_w4a4", "no_such_workload") is None
