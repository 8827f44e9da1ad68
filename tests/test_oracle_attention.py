"""Pins of the oracle's attention read (causal_attention, attend_prefill).

Checked against what the mathematics fixes, not against the oracle itself:
a masked-softmax matrix formula written independently, closed forms (one key,
equal scores), the paged layout against contiguous rows, the GQA head
mapping, and Theorem 3 as the pages describe it (gist.science summary,
"Contributions Clés"): in a causal decoder, KV states injected at the
intended positions give the query tokens exactly the outputs a prefill of the
memory as prompt gives.  The last check runs a random-weight two-layer
decoder in fp64 whose RoPE is written with complex numbers, independently of
the oracle's rotate-half code."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from _decoder import Decoder, rope_complex


def _masked_softmax_attention(q, k, v, qpos, kpos, scale):
    s = scale * (q @ k.T)
    s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w / w.sum(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_causal_attention_matches_masked_softmax(seed):
    rng = np.random.default_rng(seed)
    nq, nk, D = 7, 23, 16
    q, k, v = rng.standard_normal((nq, D)), rng.standard_normal((nk, D)), rng.standard_normal((nk, D))
    kpos = np.sort(rng.choice(100, nk, replace=False)) + 3
    qpos = np.sort(rng.choice(np.arange(kpos[0], 130), nq, replace=False))
    got = oracle.causal_attention(q, k, v, qpos, kpos, 0.3)
    ref = _masked_softmax_attention(q, k, v, qpos, kpos, 0.3)
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


def test_causal_attention_closed_forms():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((5, 8))
    k = rng.standard_normal((5, 8))
    # a query that sees exactly one key gets that key's value
    out = oracle.causal_attention(rng.standard_normal((1, 8)), k, v, [10], [10, 11, 12, 13, 14], 1.0)
    assert np.array_equal(out[0], v[0])
    # a zero query scores every key equally: the mean of the visible values
    out = oracle.causal_attention(np.zeros((1, 8)), k, v, [12], [10, 11, 12, 13, 14], 1.0)
    assert np.allclose(out[0], v[:3].mean(axis=0), atol=1e-15)


def _bits(x):
    return oracle.f64_to_bf16(x)


def test_attend_prefill_paged_equals_contiguous_and_maps_gqa_heads():
    rng = np.random.default_rng(4)
    D, hkv, group, bs, nb = 16, 2, 3, 4, 20
    hq = hkv * group
    ctx_begin, q_pos, tq, theta, scale = 5, 17, 6, 1e4, 0.25
    kc = _bits(rng.standard_normal((nb, bs, hkv, D)))
    vc = _bits(rng.standard_normal((nb, bs, hkv, D)))
    table = rng.permutation(nb)
    q_pre = _bits(rng.standard_normal((tq, hq, D)))
    got = oracle.attend_prefill(q_pre, kc, vc, table, bs, ctx_begin, q_pos, theta, scale)
    # contiguous rows in position order, read through the table by hand
    pos = np.arange(ctx_begin, q_pos + tq)
    krow = np.stack([kc[table[p // bs], p % bs] for p in pos])
    vrow = np.stack([vc[table[p // bs], p % bs] for p in pos])
    qpos = q_pos + np.arange(tq)
    for h in range(hq):
        g = h // group
        qr = oracle.bf16_to_f64(_bits(oracle.rope_rotate(oracle.bf16_to_f64(q_pre[:, h]), qpos, theta)))
        ref = _masked_softmax_attention(qr, oracle.bf16_to_f64(krow[:, g]), oracle.bf16_to_f64(vrow[:, g]),
                                        qpos, pos, scale)
        assert np.allclose(got[:, h], ref, atol=1e-13), f"head {h}"
    # query heads of different groups really read different KV heads
    assert not np.allclose(got[:, 0], got[:, group])


# ---- Theorem 3 with a random-weight decoder ---------------------------------

@pytest.mark.parametrize("seed, start", [(0, 0), (1, 37), (2, 1000)])
def test_theorem3_injected_memory_equals_prompt(seed, start):
    rng = np.random.default_rng(seed)
    dec = Decoder(rng)
    lm, tq = 11, 5
    mem = rng.standard_normal((lm, 24))
    qry = rng.standard_normal((tq, 24))
    # prompt: memory then query tokens, prefilled together at start..
    full_pos = start + np.arange(lm + tq)
    h_full, _ = dec.prefill(np.concatenate([mem, qry]), full_pos)
    # memory encoded once, alone, at offset 0: its pre-RoPE K/V are stored
    _, mem_kv = dec.prefill(mem, np.arange(lm))
    # injected at start.. and read by a prefill of the query tokens only
    h_inj = dec.prefill_over_injected(qry, start + lm + np.arange(tq), mem_kv, start + np.arange(lm))
    assert np.allclose(h_inj, h_full[lm:], rtol=0, atol=1e-10)


def test_theorem3_needs_the_intended_positions():
    # injected one position too late, the outputs differ: the check has teeth
    rng = np.random.default_rng(9)
    dec = Decoder(rng)
    lm, tq, start = 9, 4, 20
    mem, qry = rng.standard_normal((lm, 24)), rng.standard_normal((tq, 24))
    h_full, _ = dec.prefill(np.concatenate([mem, qry]), start + np.arange(lm + tq))
    _, mem_kv = dec.prefill(mem, np.arange(lm))
    h_bad = dec.prefill_over_injected(qry, start + lm + np.arange(tq), mem_kv, start - 1 + np.arange(lm))
    assert not np.allclose(h_bad, h_full[lm:], atol=1e-6)


# ---- encode once, inject anywhere -------------------------------------------

@pytest.mark.parametrize("shift", [1, 37, 4096])
def test_encode_once_inject_anywhere(shift):
    """The pages store each fact's pre-RoPE K once and place it at any
    position later (gist.science summary, "Phase Hors-ligne" and "Rotation
    Dynamique").  That rests on translation invariance: a RoPE decoder fed the
    same tokens at positions shifted by s computes the same pre-RoPE K and V in
    every layer, and its post-RoPE keys are the stored keys rotated to the new
    positions, which is what the oracle's Chunked RoPE computes."""
    rng = np.random.default_rng(shift)
    dec = Decoder(rng, layers=3)
    lm = 13
    x = rng.standard_normal((lm, 24))
    _, kv0 = dec.prefill(x, np.arange(lm))
    pos = shift + np.arange(lm)
    _, kvs = dec.prefill(x, pos)
    for (k0, v0), (ks, vs) in zip(kv0, kvs):
        assert np.allclose(ks, k0, rtol=0, atol=1e-10)
        assert np.allclose(vs, v0, rtol=0, atol=1e-10)
        post = rope_complex(ks, pos, dec.theta)
        assert np.allclose(oracle.rope_rotate(k0, pos[:, None], dec.theta), post, rtol=0, atol=1e-10)


def test_absolute_positions_break_encode_once():
    # with an absolute position signal in the input, the stored K would depend
    # on where the fact was encoded: the invariance above is not automatic
    rng = np.random.default_rng(8)
    dec = Decoder(rng, layers=2)
    lm = 9
    x = rng.standard_normal((lm, 24))
    p_emb = lambda p: np.sin(np.outer(p, np.arange(1, 25)) * 0.01)
    _, kv0 = dec.prefill(x + p_emb(np.arange(lm)), np.arange(lm))
    _, kvs = dec.prefill(x + p_emb(50 + np.arange(lm)), 50 + np.arange(lm))
    assert not np.allclose(kvs[1][0], kv0[1][0], atol=1e-6)
