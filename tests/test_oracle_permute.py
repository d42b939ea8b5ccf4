"""Pins of the grouping oracle (CPU only)."""

import numpy as np

from oracle.permute import permute_ref, valid_entries


def brute_force(ids, E):
    T, k = ids.shape
    per_expert = {e: [] for e in range(E)}
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(ids[t, j])
            if 0 <= e < E and e not in seen:
                per_expert[e].append((t, j))
            seen.add(e)
    rows = [q for e in range(E) for q in per_expert[e]]
    slot_row = np.full(T * k, -1, np.int32)
    for r, (t, j) in enumerate(rows):
        slot_row[t * k + j] = r
    counts = np.array([len(per_expert[e]) for e in range(E)], np.int32)
    return counts, np.array([t for t, _ in rows], np.int32), slot_row


def test_matches_brute_force_with_invalid_entries():
    g = np.random.default_rng(5)
    for T, k, E in [(1, 16, 896), (8, 16, 896), (37, 3, 11), (100, 4, 6)]:
        ids = g.integers(-2, E + 2, size=(T, k)).astype(np.int32)
        counts, offsets, row_tok, slot_row = permute_ref(ids, E)
        c2, rt2, sr2 = brute_force(ids, E)
        assert np.array_equal(counts, c2)
        assert np.array_equal(row_tok, rt2)
        assert np.array_equal(slot_row, sr2)
        assert offsets[0] == 0 and offsets[-1] == counts.sum() == row_tok.size


def test_invariants():
    g = np.random.default_rng(6)
    T, k, E = 300, 16, 896
    ids = np.stack([g.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    assert valid_entries(ids, E).all()
    counts, offsets, row_tok, slot_row = permute_ref(ids, E)
    assert counts.sum() == T * k and np.all(slot_row >= 0)
    q = np.arange(T * k)
    assert np.array_equal(row_tok[slot_row], q // k)  # each entry's row holds its token
    assert np.array_equal(np.sort(slot_row), q)  # a permutation of the rows
    for e in range(E):
        seg = row_tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)  # tokens ascending inside an expert's segment
        assert np.all((ids[seg] == e).any(axis=1))  # every token in the segment routed to e


def test_duplicates_keep_first_slot():
    ids = np.array([[3, 1, 3, 1], [1, 1, 1, 1]], np.int32)
    ok = valid_entries(ids, 4)
    assert ok.tolist() == [[True, True, False, False], [True, False, False, False]]
    counts, offsets, row_tok, slot_row = permute_ref(ids, 4)
    assert counts.tolist() == [0, 2, 0, 1]
    assert row_tok.tolist() == [0, 1, 0]
    assert slot_row.tolist() == [2, 0, -1, -1, 1, -1, -1, -1]
