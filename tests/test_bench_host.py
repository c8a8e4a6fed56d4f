"""bench.py's host-side logic without a GPU: the one-GPU guard, the FLOP
count, the traffic figure gated on the kernel source, and the CPU count."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_attention_flops():
    # 4 B H Nq Nkv D: two products of 2 Nq Nkv D each
    assert bench.attn_flops(1, 10, 32768, 32768, 128) == 4.0 * 10 * 32768 ** 2 * 128
    assert bench.attn_flops(2, 3, 5, 7, 32) == 4.0 * 2 * 3 * 5 * 7 * 32


def _profile(tmp_path, sha, traffic):
    p = tmp_path / "profile.md"
    p.write_text(f"# x\n\n```\ncounters-for-source-sha256: {sha}\n"
                 f"traffic_bytes_per_launch: {traffic}\n```\n")
    return str(p)


def test_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    import hashlib
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    monkeypatch.setattr(bench, "KERNEL_SRC", str(src))
    monkeypatch.setattr(bench, "COUNTERS_MD", _profile(tmp_path, sha, 123456789))
    assert bench.measured_traffic() == 123456789.0
    src.write_bytes(b"// kernel source, edited\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "COUNTERS_MD", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None


def test_host_cpus():
    usable, affinity, model = bench.host_cpus()
    assert 1 <= usable <= affinity == len(os.sched_getaffinity(0))
    assert isinstance(model, str) and model
