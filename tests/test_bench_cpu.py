"""Host logic of the benchmark script (CPU only): the single-GPU contract and
the staleness rule of the committed counter summary that `roofline.traffic`
is read from."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_touching_a_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_is_read_only_for_the_sources_it_was_measured_on(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_grouped_bf16_moe.txt")
    kv = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: kv["source_sha256"])
    t = bench.measured_traffic("grouped_bf16_moe")
    want = (float(kv["fetch_kib_per_launch"]) * float(kv["copy_fetch_factor"]) +
            float(kv["write_kib_per_launch"]) * float(kv["copy_write_factor"])) * 1024
    assert t == want and t > 0
    # any other kernel source -> the counters describe another build: no figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("grouped_bf16_moe") is None
    assert bench.measured_traffic("no_such_kernel") is None


def test_source_hash_covers_the_kernel_sources():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and int(h, 16) >= 0
    assert h == bench.kernel_source_hash()  # deterministic
