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


class _FakeEvent:
    def __init__(self, enable_timing=True):
        self.t = None

    def record(self):
        self.t = _FakeCuda.clock

    def elapsed_time(self, end):
        return 1.0


class _FakeCuda:
    """The parts of torch.cuda that queued_ahead uses, recording the order of calls."""
    clock = 0
    calls = []
    Event = _FakeEvent

    @classmethod
    def _sleep(cls, cycles):
        cls.calls.append(("sleep", int(cycles)))

    @classmethod
    def synchronize(cls):
        cls.calls.append(("sync",))


class _FakeTorch:
    cuda = _FakeCuda


def test_queued_ahead_order_and_bounded_sleep():
    """Every group of steps is issued after one sleep and before one synchronisation, the steps
    run in order after the untimed steps that measure the host's cost (body(-1), three of them),
    and each sleep stays under its cap."""
    _FakeCuda.calls = []
    seen = []
    bench.queued_ahead(_FakeTorch, 7, lambda i: seen.append(i), group=3)
    assert seen == [-1, -1, -1, 0, 1, 2, 3, 4, 5, 6]
    sleeps = [c for c in _FakeCuda.calls if c[0] == "sleep"]
    # one for the clock calibration (two timed sleeps of the same length), then one per group
    groups = sleeps[2:]
    assert len(groups) == 3
    cpm = sleeps[1][1] / 1.0            # cycles per ms from the fake events' 1 ms
    assert all(0 < c[1] <= 500.0 * cpm for c in groups)
    # a synchronisation ends every group
    tail = _FakeCuda.calls[-1]
    assert tail == ("sync",)
