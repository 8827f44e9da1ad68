"""Pins for the oracle's retrieval: scoring and top-k selection (CPU only).

score() is the exact inner product rounded once to fp64: pinned against exact
rational arithmetic (fractions.Fraction) and by order independence.
select_topk() is pinned against a brute-force selection written differently
(repeated scan for the best remaining item), numpy.lexsort, and argmax for
k = 1, including exact ties from duplicated embedding rows.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import decisive_gap, retrieve, score, select_topk


def _exact_dot(e32, q32):
    s = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(e32, q32)), Fraction(0))
    return float(s)           # float(Fraction) rounds to nearest


def test_score_is_exactly_rounded():
    rng = np.random.default_rng(29)
    for E in (1, 3, 16, 96):
        emb = rng.standard_normal((20, E)).astype(np.float32)
        q = rng.standard_normal(E).astype(np.float32)
        s = score(emb, q)
        for i in range(20):
            assert s[i] == _exact_dot(emb[i], q)


def test_score_with_heavy_cancellation():
    # terms that cancel to a tiny remainder: naive fp64 summation loses it
    q = np.array([1.0, 1.0, 1.0], np.float32)
    emb = np.array([[2.0**20, 2.0**-20, -2.0**20]], np.float32)
    assert score(emb, q)[0] == 2.0**-20
    emb2 = np.array([[1e30, 1.0, -1e30]], np.float32)
    assert score(emb2, q)[0] == 1.0


def test_score_independent_of_column_order():
    rng = np.random.default_rng(31)
    emb = rng.standard_normal((50, 768)).astype(np.float32)
    q = rng.standard_normal(768).astype(np.float32)
    perm = rng.permutation(768)
    assert np.array_equal(score(emb, q), score(emb[:, perm], q[perm]))


def _brute_topk(s, k):
    left = list(range(len(s)))
    out = []
    while left and len(out) < k:
        best = left[0]
        for i in left[1:]:
            if s[i] > s[best] or (s[i] == s[best] and i < best):
                best = i
        out.append(best)
        left.remove(best)
    return out


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 64))
    # few distinct values so that ties are frequent
    s = rng.integers(0, max(1, N // 3), N).astype(np.float64) / 7.0
    for k in (0, 1, 2, 5, N - 1, N, N + 3):
        if k < 0:
            continue
        assert select_topk(s, k) == _brute_topk(list(s), k)


def test_topk_lexsort_and_argmax():
    rng = np.random.default_rng(37)
    s = np.round(rng.standard_normal(2000), 2)      # many exact ties
    ref = np.lexsort((np.arange(s.size), -s))
    for k in (1, 5, 50, 2000):
        assert select_topk(s, k) == list(ref[:k])
    assert select_topk(s, 1) == [int(np.argmax(s))]


def test_duplicate_embedding_rows_tie_by_index():
    rng = np.random.default_rng(41)
    emb = rng.standard_normal((30, 64)).astype(np.float32)
    q = emb[7].copy()                 # row 7 is the best match ...
    emb[3] = emb[7]                   # ... and so is its duplicate at row 3
    emb[20] = emb[7]
    s = score(emb, q)
    assert s[3] == s[7] == s[20]
    top = select_topk(s, 3)
    assert top == [3, 7, 20]


def test_retrieve_pads_small_users():
    rng = np.random.default_rng(43)
    emb = rng.standard_normal((10, 16)).astype(np.float32)
    ufb = np.array([0, 4, 10])
    q = rng.standard_normal(16).astype(np.float32)
    ids, sc = retrieve(emb, ufb, 0, q, 6)
    assert list(ids[4:]) == [-1, -1] and np.all(np.isneginf(sc[4:]))
    assert sorted(ids[:4]) == [0, 1, 2, 3]
    ids1, _ = retrieve(emb, ufb, 1, q, 3)
    assert np.all((ids1 >= 4) & (ids1 < 10))
    ids0, _ = retrieve(emb, ufb, 1, q, 0)
    assert ids0.size == 0


def test_decisive_gap():
    assert decisive_gap([3.0, 1.0, 2.0], 1) == 1.0
    assert decisive_gap([3.0, 3.0, 1.0], 2) == 2.0
    assert decisive_gap([1.0, 1.0], 1) == math.inf
