"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
staleness rule of the committed HBM-counter summaries."""
import glob
import hashlib
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
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _summary(tmp_path, sources, sha):
    (tmp_path / "profiles").mkdir()
    (tmp_path / "bit_quantized_exact_amd" / "csrc").mkdir(parents=True)
    for name, text in sources.items():
        (tmp_path / "bit_quantized_exact_amd" / "csrc" / name).write_text(text)
    (tmp_path / "profiles" / "fwd_fp16_wl_counters.txt").write_text(
        "# HBM traffic of a kernel\n"
        f"source: {' '.join(sources)}\n"
        f"source_sha256: {sha}\n"
        "hbm_bytes_per_launch: 12345\n")


def test_counters_are_used_only_while_the_kernel_sources_match(tmp_path, monkeypatch):
    sources = {"a.hip": "kernel a\n", "b.h": "header b\n"}
    sha = hashlib.sha256(b"kernel a\nheader b\n").hexdigest()
    _summary(tmp_path, sources, sha)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counters_for("fwd_fp16", "wl") == 12345.0
    # any change to the kernel source or a header it lists makes the figure stale
    (tmp_path / "bit_quantized_exact_amd" / "csrc" / "b.h").write_text("header b, edited\n")
    assert bench.counters_for("fwd_fp16", "wl") is None
    assert bench.counters_for("fwd_int8", "wl") is None   # no summary at all


def test_committed_summaries_name_existing_sources():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "*_counters.txt")))
    if not paths:
        pytest.skip("no committed counter summary")
    for path in paths:
        vals = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
        for name in vals["source"].split():
            assert os.path.exists(os.path.join(ROOT, "bit_quantized_exact_amd", "csrc", name)), (path, name)
        for key in ("source_sha256", "hbm_bytes_per_launch", "algorithmic_bytes_per_launch"):
            assert key in vals, (path, key)


def test_peaks_are_the_published_dense_rates():
    assert bench.PEAK_TFLOPS == {"fp16": 2500.0, "int8": 5000.0}
    assert abs(bench.PEAK_BLEND - 3333.33) < 0.01
    assert bench.HBM_PEAK_GBS == 8000.0
