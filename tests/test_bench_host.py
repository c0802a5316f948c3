"""Host-side checks of the benchmark's conventions (CPU only)."""
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def read_timings():
    rows = []
    for line in open(os.path.join(HERE, "golden", "vecdbuf_timings.txt")):
        if line.strip() and not line.startswith("#"):
            n, ms, gf, _ = line.split()
            rows.append((int(n), float(ms), float(gf)))
    return rows


def test_flop_convention_matches_the_pages_printed_gflops():
    """2*N^3 / time reproduces every GFLOPS figure printed on the V3 page to the
    precision of the printed time (3 decimals in ms)."""
    import gemm_inputs as gi
    for n, ms, gf in read_timings():
        p = gi.Problem("x", None, n, n, n, n, n, n, 1.0, 0.0, None, None, None)
        ours = p.flops / (ms * 1e-3) / 1e9
        assert abs(ours - gf) / gf < 0.5e-3 / ms + 1e-5, (n, ms, gf, ours)


def test_gpus_above_one_exits_with_message():
    import subprocess
    import sys
    root = os.path.dirname(HERE)
    proc = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_recorded_traffic_requires_matching_sources(tmp_path, monkeypatch):
    import bench
    d = bench.library_digest()
    f = tmp_path / "x_counters.md"
    f.write_text("- `variant`: `v1`\n- `workload`: `w1`\n- `library_digest`: `%s`\n"
                 "- `traffic_bytes_per_launch`: `123`\n" % d)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("v1", "w1") == 123.0
    assert bench.recorded_traffic("v1", "w2") is None
    f.write_text(f.read_text().replace(d, "0" * 16))
    assert bench.recorded_traffic("v1", "w1") is None


def test_recorded_counters_require_matching_library(tmp_path, monkeypatch):
    import bench
    d = bench.library_digest()
    f = tmp_path / "y_counters.md"
    f.write_text("- `variant`: `v1`\n- `workload`: `w1`\n- `library_digest`: `%s`\n"
                 "- `mfma_util`: `0.9500`\n- `lds_bank_conflict_cycles`: `0`\n" % d)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    c = bench.recorded_counters("v1", "w1")
    assert c["mfma_util"] == 0.95 and c["lds_bank_conflict_cycles"] == 0.0
    assert bench.recorded_traffic("v1", "w1") is None   # not recorded in this file
    f.write_text(f.read_text().replace(d, "0" * 16))
    assert bench.recorded_counters("v1", "w1") is None
