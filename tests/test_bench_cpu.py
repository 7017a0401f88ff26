"""bench.py's host-side contract, without a GPU: the one-GPU guard, and that committed rocprofv3
counters are used only for the kernel source they were taken on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                         env={**os.environ, **env}, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""                       # no JSON line for a run that did not happen


def _write_counters(tmp_path, monkeypatch, sha):
    path = tmp_path / "counters.json"
    path.write_text(json.dumps({"kernel_source_sha256": sha, "hbm_bytes_per_dispatch": 2176700000}))
    monkeypatch.setattr(bench, "counters_path", lambda workload: str(path))


def test_counters_of_the_current_kernel_source_are_used(tmp_path, monkeypatch):
    _write_counters(tmp_path, monkeypatch, bench.kernel_source_hash())
    assert bench.measured_traffic("any", 1) == 2176700000


def test_counters_of_another_kernel_source_are_ignored(tmp_path, monkeypatch):
    _write_counters(tmp_path, monkeypatch, "0" * 64)
    assert bench.measured_traffic("any", 1) is None


def test_missing_counters_give_no_traffic(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "counters_path", lambda workload: str(tmp_path / "absent.json"))
    assert bench.measured_traffic("any", 1) is None
