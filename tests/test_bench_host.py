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


def _write_counters(path, counter, kernel, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, v in enumerate(values):
            f.write(f'{i},"{kernel}",{counter},{v}\n')
            f.write(f'{i},"other_kernel",{counter},1\n')


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """HBM bytes = FETCH_SIZE and WRITE_SIZE of the kernel's launches (KiB, median over dispatches),
    each scaled so that a plain copy of known size reads as that size; the summary records the
    kernel source hash that bench.py checks before it reports the traffic."""
    pmc = tmp_path / "pmc"
    _write_counters(pmc / "FETCH_SIZE_copy", "FETCH_SIZE", "copyBuffer", [512 * 1024] * 3)     # half of 1 GiB
    _write_counters(pmc / "WRITE_SIZE_copy", "WRITE_SIZE", "copyBuffer", [1024 * 1024] * 3)
    k = "void bss::(anonymous namespace)::attn_fwd_sg_kernel<256, false>(bss::GroupParams)"
    # dispatch 0 is the warm-up, 1-3 the timed grouped launches, later ones the per-mask protocol
    _write_counters(pmc / "FETCH_SIZE_swa576_d256", "FETCH_SIZE", k, [900.0, 100.0, 300.0, 200.0, 5.0, 5.0])
    _write_counters(pmc / "WRITE_SIZE_swa576_d256", "WRITE_SIZE", k, [900.0, 50.0, 50.0, 70.0, 5.0])
    path = bench.traffic_summary("swa576_d256", str(pmc), out_dir=str(tmp_path))
    txt = open(path).read()
    assert os.path.basename(path) == "attn_fwd_swa576_d256_swa576_traffic.txt"
    assert "hbm_bytes_per_launch: %d" % ((200.0 * 2 + 50.0) * 1024) in txt
    assert f"kernel_source_sha256_16: {bench._kernel_hash('single')}" in txt
    alg = 2 * 131072 * 256 * (2 * 16 + 2 * 4)
    assert f"algorithmic_bytes_per_launch: {alg}" in txt
    with pytest.raises(SystemExit):
        bench.traffic_summary("vit896", str(pmc), out_dir=str(tmp_path))   # no counters for its kernel
