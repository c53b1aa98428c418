"""Host logic of bench.py (CPU only): the one-GPU guard and the CPU share the oracle baseline uses."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("affinity,omp,want", [(32, "4", 4), (8, "16", 8), (12, "", 12), (12, "x", 12)])
def test_cpu_share_is_the_smallest_limit(monkeypatch, affinity, omp, want):
    monkeypatch.setattr(os, "sched_getaffinity", lambda pid: set(range(affinity)))
    monkeypatch.setenv("OMP_NUM_THREADS", omp)
    real_open = open

    def no_cgroup(path, *a, **k):   # no cgroup CPU quota file: the affinity mask and OMP only
        if str(path) == "/sys/fs/cgroup/cpu.max":
            raise FileNotFoundError(path)
        return real_open(path, *a, **k)

    monkeypatch.setattr("builtins.open", no_cgroup)
    cores, note = bench.cpu_share()
    assert cores == want
    assert "affinity %d" % affinity in note


def test_cpu_share_honours_a_cgroup_quota(monkeypatch, tmp_path):
    monkeypatch.setattr(os, "sched_getaffinity", lambda pid: set(range(64)))
    monkeypatch.delenv("OMP_NUM_THREADS", raising=False)
    quota = tmp_path / "cpu.max"
    quota.write_text("600000 100000\n")        # six CPUs' worth of time per period
    real_open = open
    monkeypatch.setattr("builtins.open",
                        lambda path, *a, **k: real_open(quota if str(path) == "/sys/fs/cgroup/cpu.max" else path,
                                                        *a, **k))
    cores, note = bench.cpu_share()
    assert cores == 6
    assert "cgroup quota 6" in note
