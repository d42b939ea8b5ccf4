"""Pins of the verify-width oracle (CPU only): brute force with Python sets,
closed forms, and a hand-worked choice."""

import numpy as np
import pytest

from oracle.verify import expected_committed, verify_distinct_ref, verify_width_choose_ref


def brute_force(ids, S, W, E):
    out = []
    for w in range(W):
        seen = set()
        for s in range(S):
            for p in range(w + 1):
                for e in ids[s * W + p]:
                    if 0 <= int(e) < E:
                        seen.add(int(e))
        out.append(len(seen))
    return np.array(out)


@pytest.mark.parametrize("S,W,k,E", [(16, 8, 16, 896), (1, 1, 4, 8), (3, 5, 2, 6), (4, 8, 16, 40)])
def test_distinct_matches_brute_force(S, W, k, E):
    g = np.random.default_rng(S * 100 + W)
    ids = g.integers(-3, E + 3, size=(S * W, k)).astype(np.int32)
    got = verify_distinct_ref(ids, S, W, E)
    assert np.array_equal(got, brute_force(ids, S, W, E))
    assert np.all(np.diff(got) >= 0)  # more rows never route to fewer experts


def test_distinct_closed_forms():
    S, W, k, E = 4, 6, 3, 1000
    # every row routes to the same k experts: k at every width
    same = np.tile(np.array([[7, 8, 9]], np.int32), (S * W, 1))
    assert np.array_equal(verify_distinct_ref(same, S, W, E), np.full(W, k))
    # every row routes to its own k experts: S * (w + 1) * k
    own = np.arange(S * W * k, dtype=np.int32).reshape(S * W, k)
    assert np.array_equal(verify_distinct_ref(own, S, W, E), S * k * np.arange(1, W + 1))
    # only invalid ids: zero
    assert np.array_equal(verify_distinct_ref(np.full((S * W, k), -1, np.int32), S, W, E), np.zeros(W))
    # the whole batch: the number of distinct valid ids
    g = np.random.default_rng(3)
    ids = g.integers(0, 50, size=(S * W, k)).astype(np.int32)
    assert verify_distinct_ref(ids, S, W, 50)[-1] == np.unique(ids).size


def test_expected_committed():
    # width 1 commits the target's own token only
    assert expected_committed([0.5, 0.5], 1) == 1.0
    # 1 + a1 + a1 a2
    assert expected_committed([0.5, 0.4], 3) == pytest.approx(1 + 0.5 + 0.2)
    assert expected_committed([1.0] * 7, 8) == 8.0


def test_choose_hand_worked():
    # S = 2 sequences, 3 positions; distinct experts 10, 14, 30; 1 MB per
    # expert, 1e9 B/s, fixed 2 ms; acceptance 0.9 then 0.2:
    #   w=1: 2 * 1      / (0.002 + 0.010) = 166.67 tok/s
    #   w=2: 2 * 1.9    / (0.002 + 0.014) = 237.5
    #   w=3: 2 * 2.08   / (0.002 + 0.030) = 130.0
    best, rates = verify_width_choose_ref([10, 14, 30], 2, [0.9, 0.2], 1e6, 1e9, 0.002)
    assert best == 2
    assert rates == pytest.approx([2 / 0.012, 3.8 / 0.016, 4.16 / 0.032])


def test_choose_limits():
    # nothing accepted: every pass commits one token per sequence, wider only costs
    best, _ = verify_width_choose_ref([16, 20, 30, 40], 4, [0.0] * 3, 1e6, 1e9, 0.0)
    assert best == 1
    # everything accepted and no extra bytes: the widest pass wins
    best, _ = verify_width_choose_ref([16, 16, 16, 16], 4, None, 1e6, 1e9, 0.0)
    assert best == 4
    # equal rates: the smallest width
    best, _ = verify_width_choose_ref([10, 20], 1, [1.0], 1e6, 1e9, 0.0)
    assert best == 1
