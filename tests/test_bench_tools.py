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
