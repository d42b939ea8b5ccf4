"""Pins of the expert-cache oracle (CPU only): a hand-worked sequence, and
agreement with an independent least-recently-used simulation that keeps a
last-use time per slot instead of an ordered list."""

import numpy as np
import pytest

from oracle.cache import ExpertCacheRef


def test_hand_worked_sequence():
    # 3 slots, 10 experts
    c = ExpertCacheRef(10, 3)
    # batch 1 uses 4, 7: two misses fill the empty slots 0, 1
    sid, fetch, h, m = c.route(np.array([[7, 4], [4, -1]]))
    assert fetch == [(4, 0), (7, 1)] and (h, m) == (0, 2)
    assert sid.tolist() == [[1, 0], [0, -1]]
    assert c.order == [2, 0, 1]
    # batch 2 uses 7 (hit, slot 1) and 2 (miss): empty slot 2 first
    sid, fetch, h, m = c.route(np.array([[7, 2]]))
    assert fetch == [(2, 2)] and (h, m) == (1, 1)
    assert sid.tolist() == [[1, 2]]
    assert c.order == [0, 1, 2]
    # batch 3 uses 9 and 5: both miss; slots 0 (expert 4) and 1 (expert 7) are
    # the least recently used and are evicted, 5 -> 0, 9 -> 1
    sid, fetch, h, m = c.route(np.array([[9, 5, 9]]))
    assert fetch == [(5, 0), (9, 1)] and (h, m) == (0, 2)
    assert sid.tolist() == [[1, 0, 1]]
    assert c.slot_of[4] == -1 and c.slot_of[7] == -1 and c.expert_in == [5, 9, 2]
    assert c.order == [2, 0, 1]
    # batch 4 uses 2 and 5 (both hits): untouched slot 1 first, then the hit
    # slots in their old order (2 before 0)
    _, fetch, h, m = c.route(np.array([[5, 2]]))
    assert fetch == [] and (h, m) == (2, 0)
    assert c.order == [1, 2, 0]
    assert (c.hits_total, c.misses_total, c.step) == (3, 5, 4)


class LastUseLRU:
    """Independent simulation: every slot carries a recency key compared as a
    tuple, no ordered list.  Never used: (-1, slot index); hit at step t:
    (t, 0, its previous key); filled at step t: (t, 1, miss index).  Victims
    are the non-hit slots with the smallest keys."""

    def __init__(self, E, C):
        self.E, self.C = E, C
        self.exp = [-1] * C
        self.key = [(-1, s) for s in range(C)]
        self.t = 0

    def route(self, ids):
        self.t += 1
        used = sorted({int(e) for e in np.asarray(ids).reshape(-1) if 0 <= e < self.E})
        where = {e: s for s, e in enumerate(self.exp) if e >= 0}
        hits = {where[e] for e in used if e in where}
        misses = [e for e in used if e not in where]
        cand = sorted((s for s in range(self.C) if s not in hits), key=lambda s: self.key[s])
        fetch = list(zip(misses, cand[: len(misses)]))
        for s in hits:
            self.key[s] = (self.t, 0, self.key[s])
        for i, (e, s) in enumerate(fetch):
            self.exp[s] = e
            self.key[s] = (self.t, 1, i)
        return fetch

    def order(self):
        return sorted(range(self.C), key=lambda s: self.key[s])


@pytest.mark.parametrize("E,C,T,k", [(896, 160, 8, 16), (40, 12, 3, 4), (6, 6, 2, 3), (1000, 600, 1, 16)])
def test_matches_independent_lru(E, C, T, k):
    g = np.random.default_rng(E + C)
    a, b = ExpertCacheRef(E, C), LastUseLRU(E, C)
    hot = g.choice(E, size=max(1, C // 2), replace=False)
    for _ in range(40):
        ids = g.integers(-2, E + 2, size=(T, k))
        ids[:, 0] = g.choice(hot, size=T)  # a hot set, so hits happen
        slot_ids, fetch, h, m = a.route(ids)
        assert fetch == b.route(ids)
        assert a.expert_in == b.exp
        assert a.order == b.order()
        # invariants: the two tables agree, every used expert is cached, the
        # renamed entries name the slots holding their experts
        for s, e in enumerate(a.expert_in):
            assert e < 0 or a.slot_of[e] == s
        assert sorted(a.order) == list(range(C))
        used = {int(e) for e in ids.reshape(-1) if 0 <= e < E}
        assert h + m == len(used)
        for (t, j), e in np.ndenumerate(ids):
            assert slot_ids[t, j] == (a.slot_of[int(e)] if 0 <= e < E else -1)


def test_batch_larger_than_cache_is_refused():
    c = ExpertCacheRef(10, 2)
    with pytest.raises(ValueError):
        c.route(np.array([[1, 2, 3]]))
