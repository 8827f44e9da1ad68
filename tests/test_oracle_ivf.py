"""Pins of oracle.ivf_probe, the exact answer of an inverted-file probe, and
of oracle.ivf_init / ivf_update, the build's centroid rules.

ivf_probe is checked against the flat retrieval it must equal when every
list is probed, against brute force on tiny indexes (every subset of lists
enumerated by hand), and on exact ties across lists (lower fact id first).
ivf_init and ivf_update are checked on hand cases (picked rows, orthogonal
pairs, empty and cancelling lists) and against the Cauchy-Schwarz optimum
the update must reach."""

from __future__ import annotations

import itertools
import math

import numpy as np
import pytest

import oracle


def _index(rng, n, nlist, dim):
    emb = rng.standard_normal((n, dim)).astype(np.float32)
    emb /= np.linalg.norm(emb, axis=1, keepdims=True)
    assign = rng.integers(0, nlist, n)
    assign[:nlist] = np.arange(nlist)                 # no empty list
    members = np.concatenate([np.flatnonzero(assign == c) for c in range(nlist)])
    list_begin = np.concatenate([[0], np.cumsum(np.bincount(assign, minlength=nlist))])
    cent = rng.standard_normal((nlist, dim)).astype(np.float32)
    return emb, cent, list_begin, members


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_all_lists_equals_flat_retrieval(seed):
    rng = np.random.default_rng(seed)
    emb, cent, lb, mem = _index(rng, 300, 7, 12)
    q = rng.standard_normal(12).astype(np.float32)
    for k in (1, 10, 300, 400):
        ids, sc = oracle.ivf_probe(emb, cent, lb, mem, q, 7, k)
        f_ids, f_sc = oracle.retrieve(emb, np.array([0, 300]), 0, q, k)
        assert np.array_equal(ids, f_ids)
        assert np.array_equal(sc[: min(k, 300)], f_sc[: min(k, 300)])


def test_brute_force_on_tiny_indexes():
    rng = np.random.default_rng(3)
    emb, cent, lb, mem = _index(rng, 40, 5, 6)
    q = rng.standard_normal(6).astype(np.float32)
    cs = [float(np.dot(cent[c].astype(float), q.astype(float))) for c in range(5)]
    rank = sorted(range(5), key=lambda c: (-cs[c], c))
    for nprobe in range(1, 6):
        cand = sorted(itertools.chain.from_iterable(mem[lb[c]:lb[c + 1]] for c in rank[:nprobe]))
        s = {f: float(np.dot(emb[f].astype(float), q.astype(float))) for f in cand}
        want = sorted(cand, key=lambda f: (-s[f], f))[:8]
        ids, _ = oracle.ivf_probe(emb, cent, lb, mem, q, nprobe, 8)
        assert list(ids[: len(want)]) == want
        assert np.all(ids[len(want):] == -1)


def test_ties_across_lists_go_to_the_lower_fact_id():
    dim = 4
    emb = np.zeros((6, dim), np.float32)
    emb[:, 0] = [0.5, 0.9, 0.5, 0.9, 0.1, 0.5]        # equal first components tie
    emb[:, 1] = [1, -1, 2, 3, 0, -2]                   # other components differ
    members = np.array([5, 3, 0, 1, 2, 4])             # lists {5, 3}, {0, 1}, {2, 4}
    list_begin = np.array([0, 2, 4, 6])
    cent = np.eye(3, dim, dtype=np.float32)
    q = np.array([1, 0, 0, 0], np.float32)             # score = first component
    ids, sc = oracle.ivf_probe(emb, cent, list_begin, members, q, 3, 6)
    assert list(ids) == [1, 3, 0, 2, 5, 4]


# ---- the build's centroid rules: ivf_init and ivf_update -------------------

def test_ivf_init_picks_evenly_spaced_rows_at_unit_length():
    emb = np.arange(1, 25, dtype=np.float32).reshape(8, 3)
    c = oracle.ivf_init(emb, 3)                       # rows 0, 2, 5
    for got, r in zip(c, (0, 2, 5)):
        want = emb[r].astype(np.float64)
        assert np.allclose(got, want / math.sqrt(float(want @ want)), rtol=0, atol=1e-15)
    z = np.zeros((4, 2), np.float32)
    assert np.all(oracle.ivf_init(z, 2) == 0.0)


def test_ivf_update_closed_forms():
    a, b = np.array([1.0, 0.0, 0.0]), np.array([0.0, 1.0, 0.0])
    emb = np.stack([a, b, -a, 3 * b]).astype(np.float32)
    prev = np.eye(3)[:3]
    # list 0 = {a, b}: (a + b) / sqrt 2; list 1 = {3b}: b; list 2 empty: kept
    lb = np.array([0, 2, 3, 3])
    mem = np.array([0, 1, 3])
    c = oracle.ivf_update(emb, lb, mem, prev)
    assert np.allclose(c[0], (a + b) / math.sqrt(2.0), rtol=0, atol=1e-15)
    assert np.allclose(c[1], b, rtol=0, atol=1e-15)
    assert np.array_equal(c[2], prev[2])
    # a list whose rows cancel keeps its centroid
    c2 = oracle.ivf_update(emb, np.array([0, 1, 3]), np.array([1, 0, 2]), prev[:2])
    assert np.array_equal(c2[1], prev[1])


def test_ivf_update_maximises_the_members_inner_products():
    """Cauchy-Schwarz: over unit vectors u, sum_r <x_r, u> = <sum_r x_r, u> is
    largest at u = sum / |sum|, so no random unit vector beats the update."""
    rng = np.random.default_rng(3)
    emb = rng.standard_normal((40, 16)).astype(np.float32)
    lb = np.array([0, 13, 13, 40])
    mem = rng.permutation(40)
    c = oracle.ivf_update(emb, lb, mem, np.eye(3, 16))
    for li in (0, 2):
        rows = emb[mem[lb[li]:lb[li + 1]]].astype(np.float64)
        best = (rows @ c[li]).sum()
        u = rng.standard_normal((500, 16))
        u /= np.linalg.norm(u, axis=1, keepdims=True)
        assert np.all((rows @ u.T).sum(axis=0) <= best + 1e-12)
        assert abs(np.linalg.norm(c[li]) - 1.0) < 1e-15
