"""Host logic of bench.py (CPU only): the HBM-traffic figure is taken from a
counter summary only while it matches the kernel sources it was measured on,
and runs on more than one GPU are refused."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _tree(tmp_path, sources):
    csrc = tmp_path / "static_block_sparse_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name, text in sources.items():
        (csrc / name).write_text(text)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    sources = {f: f"// {f}\n" for f in bench.FWD_SOURCES}
    root = _tree(tmp_path, sources)
    monkeypatch.setattr(bench, "ROOT", str(root))
    assert bench.read_traffic("w") is None  # no summary
    h = bench.kernel_hash(bench.FWD_SOURCES)
    prof = root / "profiles" / "radial_fwd_kernel_w_hbm.txt"
    prof.write_text(f"# command: ...\nkernel_source_sha256: {h}\nhbm_bytes_per_launch: 12345.0\n")
    assert bench.read_traffic("w") == 12345.0
    # any listed source changing (the mask compiler's grouping included) makes it stale
    for f in bench.FWD_SOURCES:
        (root / "static_block_sparse_amd" / "csrc" / f).write_text(f"// {f} changed\n")
        assert bench.read_traffic("w") is None, f
        (root / "static_block_sparse_amd" / "csrc" / f).write_text(sources[f])
    assert bench.read_traffic("w") == 12345.0
    prof.write_text(f"kernel_source_sha256: {h}\nhbm_bytes_per_launch: not-a-number\n")
    assert bench.read_traffic("w") is None


def test_forward_sources_cover_the_kernel_and_its_grouping():
    for f in ("attn_fwd.hip", "device_common.h", "kernels.h", "mask.cpp", "layout.h"):
        assert f in bench.FWD_SOURCES


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    assert r.stdout.strip() == ""  # no bench line
