"""bench.py host logic on the CPU: the one-GPU exit, the counter-profile reader and its
source-hash rule, the clock probe.  No kernel runs here."""

import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_score_source_hash_covers_existing_files():
    b = _bench()
    for name in b.SCORE_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, name)), name
    h = b.score_source_hash()
    assert len(h) == 64 and h == b.score_source_hash()


def test_traffic_reader_honours_the_source_hash(tmp_path, monkeypatch):
    b = _bench()
    k = b.SCORE_KERNELS[0]
    good = tmp_path / "good.txt"
    good.write_text(f"# header\nsource_sha256: {b.score_source_hash()}\ntraffic_bytes_per_launch[{k}]: 123456789\n")
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(good))
    assert b.measured_traffic(b.SCORE_KERNELS) == 123456789.0
    stale = tmp_path / "stale.txt"
    stale.write_text(f"source_sha256: {'0' * 64}\ntraffic_bytes_per_launch[{k}]: 123456789\n")
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(stale))
    assert b.measured_traffic(b.SCORE_KERNELS) is None
    monkeypatch.setattr(b, "TRAFFIC_PROFILE", str(tmp_path / "missing.txt"))
    assert b.measured_traffic(b.SCORE_KERNELS) is None


def test_committed_traffic_profile_parses():
    b = _bench()
    lines = open(b.TRAFFIC_PROFILE).read().splitlines()
    assert any(l.startswith("source_sha256: ") for l in lines)
    vals = {l.split("]:")[0][len("traffic_bytes_per_launch["):]: float(l.split("]:")[1])
            for l in lines if l.startswith("traffic_bytes_per_launch[")}
    for k in b.SCORE_KERNELS:
        # within 1% of the algorithmic bytes of one call (4567597056)
        assert abs(vals[k] - 4567597056) < 0.01 * 4567597056


def test_clock_probe_never_raises():
    b = _bench()
    c = b.gpu_clocks()
    assert c is None or isinstance(c, dict)
