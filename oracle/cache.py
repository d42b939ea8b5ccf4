"""A device expert cache in front of an external expert store: which slot
holds which expert, what each batch must fetch (pure Python, integers only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Hugging Face card "K3-Stuff" (llama-cpp-patches item 2) runs K3 with the
routed experts paged in from disk on demand, the OS page cache acting as the
hot-expert cache with least-recently-used eviction; the lucebox page
"feat(kimi-k3): add DSpark Q8 artifact and shared speculative runtime"
("Runtime validation") runs the target with SSD-routed experts behind an
8 GiB device expert cache.  Neither page specifies the policy beyond LRU
eviction; the reading used here and by the GPU library:

* the cache has C slots; each holds one expert (all three matrices) or
  nothing; slot_of[e] is the slot holding expert e (-1: not cached),
  expert_in[s] the expert in slot s (-1: empty);
* order[0 .. C-1] lists the slots from least to most recently used; at the
  start the slots are empty and listed 0, 1, ..., C-1;
* a batch uses the distinct ids in [0, E) its routed entries name (repeats
  and out-of-range ids use nothing); a used expert already cached is a hit,
  the others are misses, taken in increasing expert order;
* the i-th miss goes to the i-th slot of order that no hit of this batch
  holds (empty slots are listed first, so they fill before anything is
  evicted); the expert it held, if any, is evicted;
* the new order is: the slots this batch did not touch (in their old order),
  then the hit slots (in their old order), then the filled slots (in miss
  order); so a batch needs C >= its number of distinct experts;
* every routed entry is renamed to its expert's slot (entries that use
  nothing become -1), and the batch fetches the (expert, slot) pairs of its
  misses.
"""

from __future__ import annotations

import numpy as np


class ExpertCacheRef:
    """The cache state and its update, one batch at a time."""

    def __init__(self, E: int, C: int):
        self.E, self.C = E, C
        self.slot_of = [-1] * E
        self.expert_in = [-1] * C
        self.order = list(range(C))
        self.step = 0
        self.hits_total = 0
        self.misses_total = 0

    def route(self, ids: np.ndarray):
        """Apply one batch of routed ids [T, k].

        Returns (slot_ids int32 [T, k], fetch list [(expert, slot)], hits,
        misses)."""
        ids = np.asarray(ids, dtype=np.int64)
        used = sorted({int(e) for e in ids.reshape(-1) if 0 <= e < self.E})
        if len(used) > self.C:
            raise ValueError("batch uses more experts than the cache has slots")
        hit_slots = {self.slot_of[e] for e in used if self.slot_of[e] >= 0}
        misses = [e for e in used if self.slot_of[e] < 0]
        free = [s for s in self.order if s not in hit_slots]  # least recently used first
        victims = free[: len(misses)]
        fetch = []
        for e, s in zip(misses, victims):
            old = self.expert_in[s]
            if old >= 0:
                self.slot_of[old] = -1
            self.expert_in[s] = e
            self.slot_of[e] = s
            fetch.append((e, s))
        hits_in_order = [s for s in self.order if s in hit_slots]
        self.order = free[len(misses):] + hits_in_order + victims
        self.step += 1
        self.hits_total += len(hit_slots)
        self.misses_total += len(misses)
        slot_ids = np.full(ids.shape, -1, dtype=np.int32)
        for q, e in np.ndenumerate(ids):
            if 0 <= e < self.E:
                slot_ids[q] = self.slot_of[int(e)]
        return slot_ids, fetch, len(hit_slots), len(misses)
