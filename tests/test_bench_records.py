"""Host-side checks of bench.py's bookkeeping (no GPU): the digest that ties a
committed rocprof record to the kernel sources ignores comments and blank
space but not code, and every committed decode record names sources that
exist."""
import json
import os

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_source_digest_ignores_comments_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    a = tmp_path / "k.hip"
    a.write_text("int f(int x) {  // add one\n  return x + 1; /* done */\n}\n")
    d0 = bench.source_digest(["k.hip"])
    a.write_text("// a new comment\nint f(int x) {\n  return x + 1;\n}\n")
    assert bench.source_digest(["k.hip"]) == d0
    a.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_digest(["k.hip"]) != d0


def test_committed_decode_records_name_existing_sources():
    pdir = os.path.join(ROOT, "profiles")
    recs = [f for f in os.listdir(pdir) if f.startswith("decode_traffic_")]
    assert recs
    for f in recs:
        rec = json.load(open(os.path.join(pdir, f)))
        assert rec["sources"] and all(os.path.exists(os.path.join(ROOT, s)) for s in rec["sources"])
        assert rec["traffic_bytes"] > 0 and rec["rocprof_avg_us"] > 0
        assert len(rec["source_digest"]) == 64
