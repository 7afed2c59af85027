"""The benchmark's command-line contract, checked without a GPU: more than one GPU is refused
with a message, and HBM-traffic figures are taken only from lines measured on the current
kernel sources."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_lookup(tmp_path, monkeypatch):
    """measured_traffic returns fetch + write bytes of a kernel's line only when the line's
    source hash is that of the current kernel sources."""
    sha = bench.kernel_sources_sha()
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic_cfg.txt").write_text(
        "header text\n"
        f"traffic bwd_grad fetch_bytes 4000 write_bytes 1650 sources {sha}\n"
        "traffic dh fetch_bytes 3900 write_bytes 165 sources 0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sources_sha", lambda: sha)
    assert bench.measured_traffic("cfg", "bwd_grad") == 5650.0
    assert bench.measured_traffic("cfg", "dh") is None        # measured on other sources
    assert bench.measured_traffic("cfg", "fwd") is None       # not measured
    assert bench.measured_traffic("other", "bwd_grad") is None


def test_sources_hash_follows_code_not_comments(tmp_path):
    """A comment or reflowed line leaves the kernel-code hash (and so a measured traffic figure)
    as it is; a change to the code gives a new hash."""
    src = tmp_path / "csrc"
    src.mkdir()
    (src / "k.hip").write_text("__global__ void k(int* p) { p[0] = 1; }\n")
    base = bench.kernel_sources_sha(str(src))
    (src / "k.hip").write_text("// writes one\n__global__ void k(int* p) {\n    p[0] = 1;  /* one */\n}\n")
    assert bench.kernel_sources_sha(str(src)) == base
    (src / "k.hip").write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.kernel_sources_sha(str(src)) != base
