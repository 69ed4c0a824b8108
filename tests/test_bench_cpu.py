"""CPU tests of bench.py's own logic (no GPU): the one-GPU contract and the traffic figure's
source-hash gate."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports numpy only at module level)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    """--gpus N > 1 stops before importing torch or touching a device, with status 2."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_sha_covers_every_file_in_order(tmp_path, monkeypatch):
    (tmp_path / "a.hip").write_bytes(b"kernel a\n")
    (tmp_path / "b.h").write_bytes(b"header b\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.source_sha("a.hip+b.h") == hashlib.sha256(b"kernel a\nheader b\n").hexdigest()
    assert bench.source_sha("b.h+a.hip") != bench.source_sha("a.hip+b.h")


def _summary(src, sha, fetch=1000, write=24):
    return ("# traffic\n\n| kernel | x |\n\n"
            f"- kernel_source = {src}\n- kernel_source_sha256 = {sha}\n"
            f"- fetch_bytes_per_launch = {fetch}\n- write_bytes_per_launch = {write}\n")


def test_measured_traffic_only_while_the_hash_matches(tmp_path, monkeypatch):
    """The committed counter figure is reported while the kernel's sources are the ones it
    was taken on, and null once any of them changes or is missing."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "k.hip").write_bytes(b"v1")
    (tmp_path / "k.h").write_bytes(b"h1")
    sha = bench.source_sha("k.hip+k.h")
    (tmp_path / "profiles" / "traffic_gemm_pc.md").write_text(_summary("k.hip+k.h", sha))
    assert bench.measured_traffic("pc") == 1024.0
    assert bench.measured_traffic("m1") is None  # no summary for this workload
    (tmp_path / "k.h").write_bytes(b"h2")  # a header of the kernel changed
    assert bench.measured_traffic("pc") is None
    (tmp_path / "k.h").unlink()  # a named source is gone
    assert bench.measured_traffic("pc") is None


def test_committed_summaries_name_existing_sources():
    """Every committed traffic summary names sources that exist in the repository and gives
    both per-launch byte counts."""
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.startswith("traffic_gemm_") and f.endswith(".md")]
    assert names
    for f in names:
        text = open(os.path.join(prof, f)).read()
        fields = dict(line[2:].split(" = ", 1) for line in text.splitlines() if line.startswith("- ") and " = " in line)
        assert all(os.path.exists(os.path.join(ROOT, p)) for p in fields["kernel_source"].split("+")), f
        assert int(fields["fetch_bytes_per_launch"]) > 0 and int(fields["write_bytes_per_launch"]) > 0, f
