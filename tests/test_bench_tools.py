"""Host-side checks of bench.py's profile tools (no GPU): the stored traffic figure is
reported only while the kernel sources still match the hash taken with the counters."""
import json

import bench


def test_measured_traffic_follows_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    entry = "sparse_attn_decode"
    f.write_text(json.dumps({"entries": {entry: {"bytes_per_launch": 1234,
                                                  "source_hash": bench.source_hash(entry)}}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic(entry) == 1234
    f.write_text(json.dumps({"entries": {entry: {"bytes_per_launch": 1234, "source_hash": "stale"}}}))
    assert bench.measured_traffic(entry) is None
    assert bench.measured_traffic("score_blocks") is None


def test_missing_traffic_file_gives_none(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic("score_blocks") is None


def test_gpus_above_one_exits_with_message(capsys):
    import sys
    old = sys.argv
    sys.argv = ["bench.py", "--gpus", "2"]
    try:
        bench.main()
    except SystemExit as e:
        assert e.code == 2
    finally:
        sys.argv = old
    assert "one GPU" in capsys.readouterr().err


def test_counter_summary_rates_from_counter_and_trace_databases(tmp_path):
    """Issued MFMA rate = flops per dispatch over the kernel's average traced duration; kernels
    without counter activity are left out."""
    import sqlite3
    pmc, trace = tmp_path / "pmc.db", tmp_path / "trace.db"
    con = sqlite3.connect(pmc)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    rows = [("void infllmv2::attn_k<4>(int)", "MfmaFlopsBF16", 2.0e12), ("void infllmv2::attn_k<4>(int)",
            "MfmaFlopsBF16", 1.0e12), ("void infllmv2::attn_k<4>(int)", "MfmaUtil", 40.0),
            ("void infllmv2::attn_k<4>(int)", "MfmaUtil", 20.0), ("fill_k(int)", "MfmaFlopsBF16", 0.0),
            ("fill_k(int)", "MfmaUtil", 0.0)]
    con.executemany("insert into counters_collection values (?, ?, ?)", rows)
    con.commit()
    con = sqlite3.connect(trace)
    con.execute("create table kernels (name text, duration real)")
    con.executemany("insert into kernels values (?, ?)", [("void infllmv2::attn_k<4>(int)", 1.0e6)] * 3)
    con.commit()
    md = bench.summarize_counters(str(pmc), str(trace), "t", "cmd")
    line = next(x for x in md.splitlines() if "attn_k<4>" in x)
    cells = [c.strip() for c in line.strip("|").split("|")]
    # dispatches 2; MfmaFlopsBF16 1.5e12 per dispatch; MfmaUtil 30; 1 ms -> 1500 TFLOP/s = 60% of 2.5 PF
    assert cells[1] == "2" and cells[2] == "1.5e+12" and cells[3] == "30"
    assert cells[4] == "1000.0" and cells[5] == "1500" and cells[6] == "60.0%"
    assert "fill_k" not in md


def test_trace_durations_give_traced_roofline_while_sources_match(tmp_path, monkeypatch):
    """A launch's traced duration is the sum of its kernels' average traced durations (one call
    each per launch); the traced fraction is reported only while the kernel sources match."""
    import sqlite3
    db = tmp_path / "trace.db"
    con = sqlite3.connect(db)
    con.execute("create table kernels (name text, duration real)")
    con.executemany("insert into kernels values (?, ?)",
                    [("void infllmv2::decode_split_kernel<128, 1, 32>(int)", 18.0e3)] * 2 +
                    [("void infllmv2::decode_split_kernel<128, 1, 32>(int)", 20.0e3)] * 2 +
                    [("void infllmv2::decode_combine_kernel<128, 8>(int)", 5.0e3)] * 4 +
                    [("void infllmv2::score_kernel<128, 4, 1>(int)", 17.0e3)] * 4 +
                    [("__amd_rocclr_copyBuffer", 600.0e3)])
    con.commit()
    t = bench.store_trace_durations({"decode": str(db)})
    e = t["entries"]["sparse_attn_decode_scores"]
    assert e["launch_us"] == 24.0 and set(e["kernels"]) == {"decode_split_kernel<128, 1, 32>",
                                                             "decode_combine_kernel<128, 8>"}
    assert t["entries"]["score_blocks"]["launch_us"] == 17.0
    assert "sparse_attn_prefill" not in t["entries"]
    f = tmp_path / "durations.json"
    f.write_text(json.dumps(t))
    monkeypatch.setattr(bench, "TRACE_FILE", str(f))
    # 48 MB per launch over 24 us = 2000 GB/s = 25% of 8 TB/s
    got = bench.traced_fields("sparse_attn_decode_scores", 48e6 / 1e3, 8000.0)
    assert got == {"traced_launch_us": 24.0, "frac_traced": 0.25}
    t["entries"]["sparse_attn_decode_scores"]["source_hash"] = "stale"
    f.write_text(json.dumps(t))
    assert bench.traced_fields("sparse_attn_decode_scores", 1.0, 1.0) == {"traced_launch_us": None,
                                                                           "frac_traced": None}
