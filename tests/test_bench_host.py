"""Host-side pieces of bench.py (no GPU): the rocprofv3 results parser and the source hash
that keys the measured traffic figures."""

import os
import sqlite3
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _results_db(path, kernels=(), counters=()):
    con = sqlite3.connect(path)
    con.execute("create table kernels (name text, duration integer)")
    con.executemany("insert into kernels values (?, ?)", kernels)
    con.execute("create table counters_collection (dispatch_id integer, kernel_name text, counter_name text, "
                "value real)")
    con.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    con.commit()
    con.close()


def test_profile_summary_reads_kernel_trace_and_counters(tmp_path):
    run = tmp_path / "trace" / "host"
    run.mkdir(parents=True)
    # durations in ns: kernel A 10, 20, 30 us; kernel B 100 us
    _results_db(run / "run_results.db",
                kernels=[("kA", 10_000), ("kA", 20_000), ("kA", 30_000), ("kB", 100_000)],
                # FETCH_SIZE of one dispatch arrives split over several rows (per XCD): they add up
                counters=[(1, "kA", "FETCH_SIZE", 100.0), (1, "kA", "FETCH_SIZE", 28.0),
                          (2, "kA", "FETCH_SIZE", 64.0), (3, "kB", "WRITE_SIZE", 512.0)])
    text = bench.profile_summary(str(tmp_path))
    lines = text.splitlines()
    ka = next(l for l in lines if l.rstrip().endswith("kA") and "dispatches" not in l)
    kb = next(l for l in lines if l.rstrip().endswith("kB") and "dispatches" not in l)
    calls, avg, median, lo, hi, pct = ka.split()[:6]
    assert (int(calls), float(avg), float(median), float(lo), float(hi)) == (3, 20.0, 20.0, 10.0, 30.0)
    assert abs(float(pct) - 37.5) < 1e-9 and kb.split()[:2] == ["1", "100.0"]
    fetch = next(l for l in lines if "FETCH_SIZE" in l)
    assert "2 dispatches" in fetch and "96.0 KiB" in fetch  # (128 + 64) / 2
    assert any("WRITE_SIZE" in l and "512.0 KiB" in l for l in lines)


def test_profile_summary_skips_missing_views(tmp_path):
    con = sqlite3.connect(tmp_path / "x_results.db")
    con.execute("create table other (a integer)")
    con.commit()
    con.close()
    assert bench.profile_summary(str(tmp_path)) == ""


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    csrc = tmp_path / "exact_attention_35_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (csrc / "k.hip").write_text("int a = 1;  // one\n\n/* block\n comment */ int b = 2;\n")
    h1 = bench.sources_sha256(["k.hip"])
    (csrc / "k.hip").write_text("int a = 1;  // a different comment\n/* other */ int b = 2;\n\n\n")
    assert bench.sources_sha256(["k.hip"]) == h1
    (csrc / "k.hip").write_text("int a = 1;\nint b = 3;\n")
    assert bench.sources_sha256(["k.hip"]) != h1
