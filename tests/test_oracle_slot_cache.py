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


# ---------------------------------------------------------------- prefetch --

def _prefetch_sequence():
    return [("S", {0, 1}), ("P", [2, 3, 4]), ("S", {2, 3}), ("P", [4, 5, 1]), ("S", {1, 4})]


def test_prefetch_hand_worked_trace():
    want_s, want_p, want_t = [], [], None
    for line in open(os.path.join(GOLDEN, "lru_prefetch_trace.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tag, *vals = line.split()
        vals = tuple(int(v) for v in vals)
        {"S": want_s, "P": want_p}.get(tag, []).append(vals)
        if tag == "T":
            want_t = vals
    c = LRUSlotCache(6, 3)
    got_s, got_p = [], []
    n_s = n_p = 0
    for kind, arg in _prefetch_sequence():
        if kind == "S":
            n_s += 1
            for w, wave in enumerate(c.step(arg).waves):
                got_s += [(n_s, w, en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
        else:
            n_p += 1
            got_p += [(n_p,) + cp for cp in c.prefetch(arg)]
    assert got_s == want_s and got_p == want_p
    st = c.stats
    assert (st.hits, st.misses, st.evictions, st.prefetches, st.prefetch_used) == want_t


def _mtf_prefetch_run(ops, S):
    """Move-to-front list (index 0 = most recent) with prefetch: a prediction goes to the
    front; its victim is the deepest entry outside the protected set (the last step's
    experts and everything predicted since)."""
    lst, protected, from_pf = [], set(), set()
    hits = misses = ev = pf = used = 0
    for kind, arg in ops:
        if kind == "S":
            touched = sorted(set(arg))
            protected = set()
            for e in [e for e in touched if e in lst] + [e for e in touched if e not in lst]:
                protected.add(e)
                if e in lst:
                    hits += 1
                    used += e in from_pf
                    from_pf.discard(e)
                    lst.remove(e)
                else:
                    misses += 1
                    if len(lst) == S:
                        from_pf.discard(lst.pop())
                        ev += 1
                lst.insert(0, e)
        else:
            for e in arg:
                if e in lst:
                    lst.remove(e)
                    lst.insert(0, e)
                    protected.add(e)
                    continue
                if len(lst) == S:
                    free = [i for i, v in enumerate(lst) if v not in protected]
                    if not free:
                        break
                    from_pf.discard(lst.pop(free[-1]))
                    ev += 1
                lst.insert(0, e)
                protected.add(e)
                from_pf.add(e)
                pf += 1
    return (hits, misses, ev, pf, used), sorted(lst)


@pytest.mark.parametrize("E,S,k", [(8, 3, 2), (16, 5, 3), (64, 16, 8), (128, 32, 8)])
def test_prefetch_matches_move_to_front(E, S, k):
    rng = np.random.default_rng(E + S)
    ops, prev = [], None
    for i in range(120):
        touched = rng.choice(E, size=(rng.integers(1, 5), k)).ravel()
        ops.append(("S", touched))
        if i % 3 != 2:
            pred = rng.choice(E, size=rng.integers(0, S + 3)).tolist()
            if prev is not None and i % 2:
                pred = sorted(set(prev.tolist()))[:S] + pred   # previous step's set first
            ops.append(("P", pred))
        prev = touched
    c = LRUSlotCache(E, S)
    for kind, arg in ops:
        if kind == "S":
            before = set(c.resident())
            plan = c.step(arg)
            for wave in plan.waves:
                for en in wave:
                    assert bool(en.hit) == (en.expert in before)
        else:
            last_step = {en.expert for wave in plan.waves for en in wave if c.slot_of[en.expert] >= 0}
            c.prefetch(arg)
            # a prefetch never evicts an expert the last step ran
            assert last_step <= set(c.resident())
    st = c.stats
    want, res = _mtf_prefetch_run(ops, S)
    assert (st.hits, st.misses, st.evictions, st.prefetches, st.prefetch_used) == want
    assert c.resident() == res
    for e in range(E):
        if c.slot_of[e] >= 0:
            assert c.owner[c.slot_of[e]] == e


def test_prefetch_of_the_next_set_removes_its_misses():
    """A perfect prediction with room for it: the next step is all hits, each one used."""
    rng = np.random.default_rng(21)
    E, S = 64, 40
    c = LRUSlotCache(E, S)
    steps = [rng.choice(E, size=16, replace=False) for _ in range(30)]
    for cur, nxt in zip(steps, steps[1:]):
        c.step(cur)
        pf0 = c.stats.prefetches
        c.prefetch(sorted(set(nxt.tolist())))
        h0, m0, u0 = c.stats.hits, c.stats.misses, c.stats.prefetch_used
        c.step(nxt)
        assert c.stats.misses == m0
        assert c.stats.hits - h0 == len(set(nxt.tolist()))
        # every bundle the last prefetch copied was used by this step
        assert c.stats.prefetch_used - u0 == c.stats.prefetches - pf0
    assert c.stats.prefetch_used == c.stats.prefetches


def test_prefetch_of_resident_or_nothing_changes_no_residency():
    c = LRUSlotCache(10, 4)
    c.step([1, 2, 3])
    slots = list(c.slot_of)
    assert c.prefetch([]) == [] and c.prefetch([3, 1]) == []
    assert c.slot_of == slots and c.stats.prefetches == 0 and c.stats.evictions == 0


# ------------------------------------------------------------- layer order --

def test_layer_order_hand_worked_trace():
    want_s, want_t = [], None
    for line in open(os.path.join(GOLDEN, "lru_layer_order_trace.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tag, *vals = line.split()
        vals = tuple(int(v) for v in vals)
        if tag == "S":
            want_s.append(vals)
        else:
            want_t = vals
    c = LRUSlotCache(6, 3, n_layers=2)
    got = []
    for step, touched in enumerate([{3}, {0}, {4}, {1}, {3, 4}], start=1):
        for w, wave in enumerate(c.step(touched).waves):
            got += [(step, w, en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
    assert got == want_s
    assert (c.stats.hits, c.stats.misses, c.stats.evictions) == want_t
    plain = LRUSlotCache(6, 3)
    for touched in [{3}, {0}, {4}, {1}, {3, 4}]:
        plain.step(touched)
    assert (plain.stats.hits, plain.stats.misses) == (1, 5)


def _furthest_next_use_misses(seq, S):
    """Offline replacement in the textbook MIN manner, under the pool's constraint that a step's
    experts stay resident while it runs (each step here is one wave): on a miss with a full pool,
    evict, among the entries the step does not touch, the one whose next step lies furthest ahead
    (never used again counts as furthest). Computed from the future of the sequence itself."""
    cache, misses = set(), 0
    for i, touched in enumerate(seq):
        for e in sorted(touched):
            if e in cache:
                continue
            misses += 1
            if len(cache) == S:
                def next_use(v):
                    for j in range(i + 1, len(seq)):
                        if v in seq[j]:
                            return j
                    return len(seq) + 1
                cache.remove(max((v for v in cache if v not in touched), key=lambda v: (next_use(v), -v)))
            cache.add(e)
    return misses


@pytest.mark.parametrize("L,per,size,S", [(3, 8, 4, 6), (4, 16, 6, 16), (4, 32, 10, 24), (5, 8, 3, 9)])
def test_layer_order_is_optimal_on_a_fixed_cycle(L, per, size, S):
    """Each layer touches the same set every cycle: the layer order then makes exactly as many
    misses as evicting by furthest next use read off the future sequence, and plain LRU (which
    evicts what comes next) makes more."""
    rng = np.random.default_rng(L * per + S)
    sets = [set((l * per + rng.choice(per, size=size, replace=False)).tolist()) for l in range(L)]
    seq = [sets[i % L] for i in range(L * 12)]
    c = LRUSlotCache(L * per, S, n_layers=L)
    lru = LRUSlotCache(L * per, S)
    for touched in seq:
        c.step(touched)
        lru.step(touched)
    assert c.stats.misses == _furthest_next_use_misses(seq, S)
    assert lru.stats.misses > c.stats.misses


def test_layer_order_rejects_a_step_across_layers():
    c = LRUSlotCache(8, 4, n_layers=2)
    with pytest.raises(ValueError):
        c.step([1, 5])


# --------------------------------------------------------- routing frequency --

def test_frequency_hand_worked_trace():
    want_s, want_t = [], None
    for line in open(os.path.join(GOLDEN, "lru_frequency_trace.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tag, *vals = line.split()
        vals = tuple(int(v) for v in vals)
        if tag == "S":
            want_s.append(vals)
        else:
            want_t = vals
    c = LRUSlotCache(4, 2, freq_decay=0.5)
    got = []
    steps = [[0, 0, 0, 1], [2], [0, 3, 3], [1, 2]]       # one id per routed row
    for step, rows in enumerate(steps, start=1):
        for w, wave in enumerate(c.step(rows).waves):
            got += [(step, w, en.expert, en.slot, int(en.hit), en.evicted) for en in wave]
    assert got == want_s
    assert (c.stats.hits, c.stats.misses, c.stats.evictions) == want_t
    assert c.freq == [0.875, 1.125, 1.25, 1.0]


def _lfu_run(steps, S):
    """Textbook LFU over a recency list (index 0 = most recent): a miss with a full cache evicts,
    among the entries outside the step's wave, the one routed the fewest rows so far, the deepest
    in the list among equals. Same access order as the pool (resident ascending, then others)."""
    lst, total = [], {}
    hits = misses = 0
    for rows in steps:
        for e in rows:
            total[e] = total.get(e, 0) + 1
        touched = sorted(set(rows))
        order = [e for e in touched if e in lst] + [e for e in touched if e not in lst]
        for w0 in range(0, len(order), S):
            wave = order[w0:w0 + S]
            for e in wave:
                if e in lst:
                    hits += 1
                    lst.remove(e)
                else:
                    misses += 1
                    if len(lst) == S:
                        cand = [i for i, v in enumerate(lst) if v not in wave]
                        fewest = min(total[lst[i]] for i in cand)
                        lst.pop(max(i for i in cand if total[lst[i]] == fewest))
                lst.insert(0, e)
    return hits, misses


@pytest.mark.parametrize("E,S,k", [(8, 3, 2), (16, 5, 3), (64, 16, 8)])
def test_frequency_without_decay_is_textbook_lfu(E, S, k):
    rng = np.random.default_rng(3 * E + S)
    p = rng.dirichlet(np.full(E, 0.3))
    steps = [rng.choice(E, size=(rng.integers(1, 5) * k), p=p).tolist() for _ in range(80)]
    c = LRUSlotCache(E, S, freq_decay=1.0)
    for rows in steps:
        c.step(rows)
    assert (c.stats.hits, c.stats.misses) == _lfu_run(steps, S)


def test_frequency_is_the_decayed_sum_of_routed_rows():
    rng = np.random.default_rng(5)
    E, d = 12, 0.8
    steps = [rng.choice(E, size=10).tolist() for _ in range(40)]
    c = LRUSlotCache(E, 4, freq_decay=d)
    for rows in steps:
        c.step(rows)
    counts = np.stack([np.bincount(r, minlength=E) for r in steps])
    closed = (d ** np.arange(len(steps))[::-1, None] * counts).sum(axis=0)
    assert np.allclose(c.freq, closed, rtol=1e-12, atol=0)
