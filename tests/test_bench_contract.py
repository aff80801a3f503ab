"""The benchmark script's host-side contract (CPU only): it refuses more than
one GPU with a message and status 2 before touching a device; the oracle
timing record carries the host's model, thread count and the one-thread runs;
and the traffic figure is read from the committed counter summary only while
that summary's kernel-source hash matches the sources (else it is None)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_oracle_timing_record():
    import datagen
    import torch
    A = torch.from_numpy(datagen.matrix("uniform", 1, 96, 96))
    B = torch.from_numpy(datagen.matrix("uniform", 2, 96, 96))
    rec = bench.oracle_timing(A, B, datagen, full=True)
    assert rec["threads"] >= 1 and rec["nproc"] >= 1
    assert "cpu_model" in rec
    for key in ("one_thread_256", "one_thread_1024", "all_threads_full_96"):
        assert rec[key]["s"] >= 0 and rec[key]["gflops"] > 0, key
    json.dumps(rec)  # the record goes into the benchmark's JSON line


def test_traffic_is_read_only_for_matching_sources(tmp_path, monkeypatch):
    """A summary with the current hash yields its figure; any other hash, a
    missing kernel section or a missing file yields None."""
    name = "void mgemm::sgemm_kernel<mgemm::CfgMfma128, 2, true, 16>(mgemm::GemmArgs)"
    grid = 1048576
    body = (f"kernel_src_sha256={bench.kernel_source_hash()}\n\n[{name} grid={grid}]\n"
            "FETCH_SIZE=1.0\nhbm_bytes_per_launch=123456789\n")
    (tmp_path / "profiles").mkdir()
    f = tmp_path / "profiles" / os.path.basename(bench.COUNTERS_FILE)
    f.write_text(body)
    h = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: h)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(name, grid) == 123456789.0
    assert bench.measured_traffic(name, grid + 1) is None
    f.write_text(body.replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.measured_traffic(name, grid) is None
    f.unlink()
    assert bench.measured_traffic(name, grid) is None
