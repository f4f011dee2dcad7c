"""Exact simulation of the expert slot pool (oracle side, test infrastructure only).

The pages' expert cache keeps whole expert bundles resident in VRAM, checks
residency for the experts the router returned and evicts the least recently
used bundles on a miss; a step that needs more experts than there are slots
finishes each wave's copies before that wave computes ("Running 35B MoE Models
on 8GB GPUs: How vvllm-ms Caches Experts in System RAM", section "Technical
Insight"); only
experts that actually run are loaded ("NovaLLM: Running Massive MoE Models
Fully In-Memory", section 3, Optimization #1).

Readings taken where the pages are silent:

* the pool holds n_slots bundles and starts empty;
* per step the touched set is the distinct experts in topk_idx; they are
  accessed in the order: experts resident at the start of the step (ascending
  id), then the non-resident ones (ascending id);
* that sequence is cut into transfer waves of at most n_slots consecutive
  experts; a wave's transfers complete before its experts run;
* each access is a textbook LRU access: a hit refreshes the expert's recency;
  a miss fills the lowest free slot, else evicts the least recently accessed
  expert and reuses its slot;
* weights are read-only, so an eviction is a table update with no copy back.

Under this order an eviction never removes an expert of the wave being formed:
every expert accessed in the wave is more recent than any candidate victim,
and a wave holds at most n_slots experts.

Prefetch (the "next" row of the residency design): predicted experts are
fetched ahead of the layer that will run them, in the background while the
current layer computes ("NovaLLM", section 3, Optimization #1), only when not
already resident, the experts most in demand first ("The Billion-Token
Bottleneck", sections "Predictive Prefetching: Looking into the Future" and
"The Orchestration Layer"). The prediction is an input (a priority-ordered
list). Readings taken:

* a predicted expert that is resident only has its recency refreshed;
* a non-resident one takes the lowest free slot, else the slot of the least
  recently used expert that neither the most recent step touched (that step's
  kernels may still be reading its experts) nor a prediction since that step
  named (a prediction does not undo itself); when no such expert exists the
  rest of the prediction is dropped;
* a prefetch is neither a hit nor a miss; a later step that touches a
  prefetched expert before it is evicted counts a hit and a "prefetch used".

Layer order (beyond the pages, whose cache is plain LRU and which call that
naive, "Running 35B MoE Models on 8GB GPUs", section "Gotcha"): the entries may
be L layer-major groups of a stack whose layers run in the cyclic order
0..L-1. A step then touches one layer's entries, and every victim choice (a
miss's or a prefetch's) takes, among the entries it may evict, one of the layer
whose next step comes last, i.e. the largest (layer - current - 1) mod L, the
least recently used within it. With L = 1 this is plain LRU.

Routing frequency (beyond the pages, likewise): with a decay in (0, 1], every
step first sets freq[e] = decay * freq[e] + (rows routed to e in the step) for
all entries, and a victim (after the layer order, if any) is the entry with
the smallest freq, the least recently used among equals. The pages' cache is
recency alone ("Technical Insight"), which they call blind to upcoming needs
("Gotcha").
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class WaveEntry:
    expert: int
    slot: int
    hit: bool
    evicted: int  # expert evicted to make room, or -1


@dataclass
class StepPlan:
    waves: list = field(default_factory=list)   # list[list[WaveEntry]]


@dataclass
class CacheStats:
    hits: int = 0
    misses: int = 0
    evictions: int = 0
    waves: int = 0
    steps: int = 0
    prefetches: int = 0
    prefetch_used: int = 0


class LRUSlotCache:
    def __init__(self, n_experts: int, n_slots: int, n_layers: int = 1, freq_decay: float = 0.0):
        if n_slots < 1 or n_experts < 1 or n_experts % n_layers or not 0.0 <= freq_decay <= 1.0:
            raise ValueError("need an expert, a slot, layers that divide the entries and a decay in [0, 1]")
        self.E, self.S, self.L, self.decay = n_experts, n_slots, n_layers, freq_decay
        self.reset()

    def reset(self):
        self.slot_of = [-1] * self.E
        self.owner = [-1] * self.S
        self.last = [0] * self.E
        self.clock = 0
        self.layer = 0                # layer of the most recent step
        self.freq = [0.0] * self.E    # decayed rows routed per entry (used when decay > 0)
        self.step_touched = set()     # experts the most recent step accessed, or predicted since
        self.from_prefetch = set()    # prefetched, not yet touched by a step
        self.stats = CacheStats()

    def resident(self):
        return [e for e in range(self.E) if self.slot_of[e] >= 0]

    def _victim(self, candidates):
        """The layer whose next step comes last, then the least recently used."""
        per = self.E // self.L
        ahead = lambda v: (v // per - self.layer - 1) % self.L
        f = (lambda v: self.freq[v]) if self.decay > 0 else (lambda v: 0.0)
        return max(candidates, key=lambda v: (ahead(v), -f(v), -self.last[v]))

    def _access(self, e: int, wave) -> WaveEntry:
        self.clock += 1
        self.step_touched.add(e)
        if self.slot_of[e] >= 0:
            self.last[e] = self.clock
            self.stats.hits += 1
            if e in self.from_prefetch:
                self.from_prefetch.discard(e)
                self.stats.prefetch_used += 1
            return WaveEntry(e, self.slot_of[e], True, -1)
        self.stats.misses += 1
        evicted = -1
        free = [s for s in range(self.S) if self.owner[s] < 0]
        if free:
            slot = free[0]
        else:
            evicted = self._victim([v for v in self.resident() if v not in wave])
            slot = self.slot_of[evicted]
            self.slot_of[evicted] = -1
            self.from_prefetch.discard(evicted)
            self.stats.evictions += 1
        self.owner[slot] = e
        self.slot_of[e] = slot
        self.last[e] = self.clock
        return WaveEntry(e, slot, False, evicted)

    def step(self, touched_experts) -> StepPlan:
        rows = [int(e) for e in touched_experts]
        touched = sorted(set(rows))
        if self.decay > 0:
            routed = [0] * self.E
            for e in rows:
                routed[e] += 1
            self.freq = [self.decay * f + r for f, r in zip(self.freq, routed)]
        layers = {e // (self.E // self.L) for e in touched}
        if len(layers) > 1:
            raise ValueError("a step touches entries of several layers")
        if layers:
            self.layer = layers.pop()
        self.step_touched = set()
        order = [e for e in touched if self.slot_of[e] >= 0] + [e for e in touched if self.slot_of[e] < 0]
        plan = StepPlan()
        for w0 in range(0, len(order), self.S):
            wave = order[w0:w0 + self.S]
            plan.waves.append([self._access(e, wave) for e in wave])
        self.stats.waves += len(plan.waves)
        self.stats.steps += 1
        return plan

    def prefetch(self, predicted):
        """Inserts the predicted experts (priority order) between steps. Returns the copies it
        implies as (expert, slot, evicted) in issue order."""
        copies = []
        for e in (int(v) for v in predicted):
            if self.slot_of[e] >= 0:
                self.clock += 1
                self.last[e] = self.clock
                self.step_touched.add(e)
                continue
            free = [s for s in range(self.S) if self.owner[s] < 0]
            evicted = -1
            if free:
                slot = free[0]
            else:
                candidates = [v for v in self.resident() if v not in self.step_touched]
                if not candidates:
                    break
                evicted = self._victim(candidates)
                slot = self.slot_of[evicted]
                self.slot_of[evicted] = -1
                self.from_prefetch.discard(evicted)
                self.stats.evictions += 1
            self.clock += 1
            self.owner[slot] = e
            self.slot_of[e] = slot
            self.last[e] = self.clock
            self.step_touched.add(e)
            self.from_prefetch.add(e)
            self.stats.prefetches += 1
            copies.append((e, slot, evicted))
        return copies
