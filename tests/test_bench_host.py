"""bench.py host logic: the traffic figure comes from the committed counter summary only while
every source file of the kernel still has the recorded hash."""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _records():
    out = []
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            out += [json.loads(l.split(":", 1)[1]) for l in f if l.startswith("traffic-record:")]
    return out


def test_traffic_records_are_well_formed():
    recs = _records()
    assert recs, "no traffic record under profiles/"
    for r in recs:
        assert r["bytes_per_launch"] == r["fetch_bytes_per_launch"] + r["write_bytes_per_launch"]
        assert r["sources"], "a record names the files its kernel is built from"
        for rel in r["sources"]:
            assert os.path.exists(os.path.join(ROOT, rel)), rel


def test_traffic_follows_source_hash():
    for r in _records():
        same = True
        for rel, sha in r["sources"].items():
            with open(os.path.join(ROOT, rel), "rb") as f:
                same &= hashlib.sha256(f.read()).hexdigest() == sha
        got = bench.recorded_traffic(r["workload"], r["kernel"])
        assert got == (r["bytes_per_launch"] if same else None)
    assert bench.recorded_traffic("no_such_workload", "no_such_kernel") is None
