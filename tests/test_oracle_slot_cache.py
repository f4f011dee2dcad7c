"""Pins for the oracle's slot-pool simulation: a hand-worked trace, a
move-to-front LRU list (textbook), the inclusion property and the S >= E case."""
import os

import numpy as np
import pytest

from oracle.slot_cache import LRUSlotCache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_worked_trace():
    rows = []
    for line in open(os.path.join(GOLDEN, "lru_trace.txt")):
        line = line.split("#")[0].strip()
        if line:
            rows.append(tuple(int(v) for v in line.split()))
    c = LRUSlotCache(4, 2)
    got = []
    for step, touched in enumerate([{0, 1}, {1, 2}, {0, 3}, {0, 1, 2}], start=1):
        plan = c.step(touched)
        for w, wave in enumerate(plan.waves):
            for ent in wave:
                got.append((step, w, ent.expert, ent.slot, int(ent.hit), ent.evicted))
    assert got == rows
    assert (c.stats.hits, c.stats.misses, c.stats.evictions, c.stats.waves) == (2, 7, 5, 5)


def _mtf_run(steps, E, S):
    """Move-to-front list: index 0 is the most recent. Same access order as the oracle."""
    lst = []
    hits = misses = ev = 0
    victims = []
    for touched in steps:
        touched = sorted(set(touched))
        order = [e for e in touched if e in lst] + [e for e in touched if e not in lst]
        for e in order:
            if e in lst:
                hits += 1
                lst.remove(e)
            else:
                misses += 1
                if len(lst) == S:
                    victims.append(lst.pop())
                    ev += 1
            lst.insert(0, e)
    return hits, misses, ev, victims, sorted(lst)


@pytest.mark.parametrize("E,S,k", [(8, 3, 2), (16, 4, 3), (64, 16, 8), (128, 32, 8)])
def test_matches_move_to_front(E, S, k):
    rng = np.random.default_rng(E * S)
    steps = [rng.choice(E, size=(rng.integers(1, 6), k)).ravel() for _ in range(80)]
    c = LRUSlotCache(E, S)
    victims = []
    for st in steps:
        for wave in c.step(st).waves:
            assert len(wave) <= S
            victims += [en.evicted for en in wave if en.evicted >= 0]
            slots = [en.slot for en in wave]
            assert len(set(slots)) == len(slots)          # a wave never reuses a slot
    h, m, ev, vic, res = _mtf_run(steps, E, S)
    assert (c.stats.hits, c.stats.misses, c.stats.evictions) == (h, m, ev)
    assert victims == vic
    assert c.resident() == res
    # slot table consistency
    for e in range(E):
        if c.slot_of[e] >= 0:
            assert c.owner[c.slot_of[e]] == e


def test_inclusion_property():
    rng = np.random.default_rng(11)
    steps = [rng.choice(40, size=12) for _ in range(200)]
    misses = []
    for S in range(1, 41):
        c = LRUSlotCache(40, S)
        for st in steps:
            c.step(st)
        misses.append(c.stats.misses)
    assert all(a >= b for a, b in zip(misses, misses[1:]))


def test_pool_holding_all_experts_only_cold_misses():
    rng = np.random.default_rng(12)
    steps = [rng.choice(30, size=5) for _ in range(50)]
    c = LRUSlotCache(30, 30)
    for st in steps:
        c.step(st)
    assert c.stats.misses == len(set(np.concatenate(steps).tolist()))
    assert c.stats.evictions == 0
