"""Host-side behaviour of bench.py (no GPU): the counter-calibration path and the clock sampler start
no other program, and no process is started at all while a profiler's settings are in the
environment."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _forbid_processes(monkeypatch):
    def boom(*a, **k):
        raise AssertionError("a process was started")
    monkeypatch.setattr(subprocess, "Popen", boom)
    monkeypatch.setattr(subprocess, "run", boom)
    monkeypatch.setattr(subprocess, "call", boom)
    monkeypatch.setattr(subprocess, "check_output", boom)
    for name in ("system", "fork", "forkpty", "posix_spawn", "posix_spawnp", "execv", "execve", "execvp",
                 "execvpe", "execl", "execlp", "spawnv", "spawnvp"):
        if hasattr(os, name):
            monkeypatch.setattr(os, name, boom)


def test_calibrate_copy_starts_no_process(monkeypatch, capsys):
    _forbid_processes(monkeypatch)
    bench.main(["--calibrate-copy", "1", "--steps", "2", "--device", "cpu"])
    out = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert out == {"calibrate_copy_bytes": 1 << 20, "copies": 2}


def test_no_sampler_under_profiler(monkeypatch):
    monkeypatch.setenv("ROCPROF_COUNTERS", "FETCH_SIZE")
    assert bench.under_profiler()
    _forbid_processes(monkeypatch)
    s = bench.ClockSampler(enabled=True)
    assert s.proc is None and s() is None
    s.close()


def test_sampler_disabled_starts_nothing(monkeypatch):
    for k in [k for k in os.environ if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    _forbid_processes(monkeypatch)
    s = bench.ClockSampler(enabled=False)
    assert s.proc is None and s() is None


def test_more_than_one_gpu_is_refused(capsys):
    with pytest.raises(SystemExit) as e:
        bench.main(["--gpus", "2"])
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
