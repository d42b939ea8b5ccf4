"""Pins of the routing oracle (CPU only)."""

import math

import numpy as np

from oracle.route import route_ref, scores


def python_topk(z, b, k):
    """Textbook selection with Python's sorted(): key (-score, index)."""
    T, E = z.shape
    ids = []
    for t in range(T):
        s = [1.0 / (1.0 + math.exp(-float(z[t, e]))) + (float(b[e]) if b is not None else 0.0) for e in range(E)]
        ids.append(sorted(range(E), key=lambda e: (-s[e], e))[:k])
    return np.array(ids, dtype=np.int32)


def test_matches_python_sorted():
    g = np.random.default_rng(1)
    for T, E, k in [(16, 40, 5), (7, 8, 2), (3, 896, 16)]:
        z = g.standard_normal((T, E)).astype(np.float32)
        b = (g.standard_normal(E) * 0.3).astype(np.float32)
        ids, w = route_ref(z, b, k)
        assert np.array_equal(ids, python_topk(z, b, k))
        ids0, _ = route_ref(z, None, k)
        assert np.array_equal(ids0, python_topk(z, None, k))


def test_hand_worked_example():
    # z = [0, 0, 2, -1], b = [0, .5, 0, 0]: scores .5, 1.0, 0.8808, 0.2689 -> experts 1 then 2.
    z = np.array([[0.0, 0.0, 2.0, -1.0]], np.float32)
    b = np.array([0.0, 0.5, 0.0, 0.0], np.float32)
    ids, w = route_ref(z, b, 2)
    assert ids.tolist() == [[1, 2]]
    s2 = 1.0 / (1.0 + math.exp(-2.0))  # 0.8807970779778823
    assert np.allclose(w, [[0.5 / (0.5 + s2), s2 / (0.5 + s2)]], rtol=0, atol=1e-7)
    # the bias steers selection only: the weight of expert 1 is sigmoid(0) = 0.5 before normalizing
    _, wu = route_ref(z, b, 2, normalize=False)
    assert np.allclose(wu, [[0.5, s2]], rtol=1e-7)


def test_zero_bias_is_topk_of_logits():
    g = np.random.default_rng(2)
    z = g.random((64, 896), dtype=np.float32)  # U[0,1) fp32 has exact duplicates in some rows
    ids, _ = route_ref(z, np.zeros(896, np.float32), 16)
    ref = np.argsort(-z.astype(np.float64), axis=1, kind="stable")[:, :16]
    assert np.array_equal(ids, ref)


def test_all_equal_and_full_k():
    z = np.zeros((3, 10), np.float32)
    ids, w = route_ref(z, np.zeros(10, np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3
    assert np.all(w == np.float32(0.25))
    g = np.random.default_rng(3)
    z = g.standard_normal((5, 12)).astype(np.float32)
    ids, w = route_ref(z, None, 12)
    assert all(sorted(r) == list(range(12)) for r in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)


def test_invariants_and_scale():
    g = np.random.default_rng(4)
    z = g.standard_normal((50, 896)).astype(np.float32)
    b = (g.standard_normal(896) * 0.5).astype(np.float32)
    ids, w = route_ref(z, b, 16)
    assert np.all((ids >= 0) & (ids < 896))
    assert all(len(set(r)) == 16 for r in ids.tolist())
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
    s = scores(z, b)
    sel = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    assert np.all(np.diff(sel, axis=1) <= 0)  # emitted in descending score
    ids2, w2 = route_ref(z, b, 16, route_scale=2.5)
    assert np.array_equal(ids, ids2) and np.allclose(w2, 2.5 * w, rtol=1e-6)


def test_nan_ranks_last_and_ties_go_to_lower_index():
    z = np.array([[np.nan, 1.0, 1.0, 0.5]], np.float32)
    ids, _ = route_ref(z, None, 4)
    assert ids.tolist() == [[1, 2, 3, 0]]
