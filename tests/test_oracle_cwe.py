"""Pins of Context-Window Encoding (oracle.cwe_window / capture_rows) with a
random-weight fp64 decoder (tests/_decoder.py).

What the pages fix: each fact is encoded with the w turns before it and only
its own KV is kept, keys before RoPE (gist.science summary, "Phase
Hors-ligne").  Consequences checked here: a window of 0 is independent
encoding; a window covering every earlier turn reproduces exactly the KV a
prefill of the whole conversation gives those tokens, so injecting all facts
and prefilling only the query equals prompting with the conversation
(Theorem 3); the first layer's KV never depends on the window; the stored KV
does not depend on where the window is encoded (RoPE is relative)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from _decoder import Decoder


def test_cwe_window_by_hand():
    lens = [3, 5, 2, 4]
    assert oracle.cwe_window(lens, 2, 0) == (8, 10, 0, 2)
    assert oracle.cwe_window(lens, 2, 1) == (3, 10, 5, 2)
    assert oracle.cwe_window(lens, 2, 5) == (0, 10, 8, 2)     # clipped at the first turn
    assert oracle.cwe_window(lens, 0, 2) == (0, 3, 0, 3)
    w = np.arange(20).reshape(10, 2)
    assert np.array_equal(oracle.capture_rows(w, 3, 4), w[3:7])


def _conversation(rng, lens, dm=24):
    return [rng.standard_normal((n, dm)) for n in lens]


def _encode(dec, turns, j, w, offset=0):
    """CWE of fact j: prefill the window at offset.., keep the fact's rows."""
    lens = [t.shape[0] for t in turns]
    a, b, kb, kl = oracle.cwe_window(lens, j, w)
    x = np.concatenate(turns)[a:b]
    _, kv = dec.prefill(x, offset + np.arange(b - a))
    return [(oracle.capture_rows(k, kb, kl), oracle.capture_rows(v, kb, kl)) for k, v in kv]


@pytest.mark.parametrize("seed", [0, 1])
def test_window_zero_is_independent_encoding(seed):
    rng = np.random.default_rng(seed)
    dec = Decoder(rng)
    turns = _conversation(rng, [4, 6, 3, 5])
    for j in range(4):
        got = _encode(dec, turns, j, 0)
        _, ref = dec.prefill(turns[j], np.arange(turns[j].shape[0]))
        for (gk, gv), (rk, rv) in zip(got, ref):
            assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


@pytest.mark.parametrize("seed", [0, 1])
def test_full_window_equals_conversation_prefill(seed):
    rng = np.random.default_rng(seed)
    dec = Decoder(rng)
    lens = [4, 6, 3, 5]
    turns = _conversation(rng, lens)
    x = np.concatenate(turns)
    _, kv_all = dec.prefill(x, np.arange(x.shape[0]))
    starts = np.concatenate([[0], np.cumsum(lens)])
    for j in range(4):
        got = _encode(dec, turns, j, j, offset=17)         # encoded elsewhere: RoPE is relative
        for (gk, gv), (rk, rv) in zip(got, kv_all):
            assert np.allclose(gk, rk[starts[j]:starts[j + 1]], rtol=0, atol=1e-10)
            assert np.allclose(gv, rv[starts[j]:starts[j + 1]], rtol=0, atol=1e-10)


def test_first_layer_ignores_the_window_and_deeper_layers_do_not():
    rng = np.random.default_rng(2)
    dec = Decoder(rng)
    turns = _conversation(rng, [5, 4, 6])
    e0 = _encode(dec, turns, 2, 0)
    e2 = _encode(dec, turns, 2, 2)
    assert np.array_equal(e0[0][0], e2[0][0]) and np.array_equal(e0[0][1], e2[0][1])
    assert not np.allclose(e0[1][0], e2[1][0], atol=1e-6)   # context reached layer 2


@pytest.mark.parametrize("start", [0, 29])
def test_cwe_memory_injected_equals_prompting_with_the_conversation(start):
    # every fact encoded with all earlier turns, stored, injected in order at
    # start.., then only the query is prefilled: Theorem 3
    rng = np.random.default_rng(11)
    dec = Decoder(rng)
    lens = [4, 6, 3, 5]
    turns = _conversation(rng, lens)
    qry = rng.standard_normal((3, 24))
    x = np.concatenate(turns + [qry])
    h_full, _ = dec.prefill(x, start + np.arange(x.shape[0]))
    per_fact = [_encode(dec, turns, j, j) for j in range(4)]
    mem_kv = [(np.concatenate([f[l][0] for f in per_fact]), np.concatenate([f[l][1] for f in per_fact]))
              for l in range(len(dec.W))]
    lm = sum(lens)
    h_inj = dec.prefill_over_injected(qry, start + lm + np.arange(3), mem_kv, start + np.arange(lm))
    assert np.allclose(h_inj, h_full[lm:], rtol=0, atol=1e-10)
