"""Host-side checks of bench.py's bookkeeping (no GPU): the digest that ties a
committed rocprof record to the kernel sources ignores comments and blank
space but not code, every committed decode record names sources that exist,
and the extra measurements run as child processes whose failure is reported
in the line instead of ending the run."""
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


def test_extra_leg_runs_in_a_child_and_its_failure_is_reported(monkeypatch):
    calls = []

    class Done:
        def __init__(self, rc, out):
            self.returncode, self.stdout = rc, out

    def fake_run(cmd, stdout=None, text=None):
        calls.append(cmd)
        if "continuous_batching" in cmd:
            return Done(-9, "")
        return Done(0, 'some log line\n{"decode_step_us": 47.0}\n')

    monkeypatch.setattr(bench.subprocess, "run", fake_run)
    assert bench.leg_in_child("llama8b_c4k", 4, 256) == {"decode_step_us": 47.0}
    assert "error" in bench.leg_in_child("continuous_batching", 4, 512)
    # a fresh interpreter running this same script, one leg
    assert all(c[1].endswith("bench.py") and c[2:4] == ["--leg", c[3]] for c in calls)
    assert calls[0][3] == "llama8b_c4k" and "--replicas" in calls[0]
