"""Host logic of bench.py that needs no GPU: the HBM-traffic figure is taken
from the committed counter summary only while the kernel sources still hash
to the value recorded there, and a request for more than one GPU is refused."""
import hashlib
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tree(tmp_path, sha_ok: bool):
    for rel in bench.TRAFFIC_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copyfile(os.path.join(ROOT, rel), dst)
    h = hashlib.sha256()
    for rel in bench.TRAFFIC_SOURCES:
        h.update((tmp_path / rel).read_bytes())
    sha = h.hexdigest() if sha_ok else "0" * 64
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "hbm_traffic_wl.txt").write_text(
        f"# summary\nsources_sha256: {sha}\n"
        "kernel attn_kernel<128,0>: dispatches 3 fetch_kib 1.0 write_kib 2.0 hbm_bytes 1.2345e+09\n")


def test_traffic_reported_when_sources_match(tmp_path, monkeypatch):
    _tree(tmp_path, sha_ok=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", "attn_kernel<128,0>") == 1.2345e9
    assert bench.measured_traffic("wl", "attn_kernel<128,1>") is None
    assert bench.measured_traffic("other", "attn_kernel<128,0>") is None


def test_traffic_dropped_when_sources_changed(tmp_path, monkeypatch):
    _tree(tmp_path, sha_ok=False)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("wl", "attn_kernel<128,0>") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
