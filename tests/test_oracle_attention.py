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

def _rope_complex(x, pos, theta):
    """RoPE as multiplication of (x_i + i x_{i+D/2}) by exp(i p w_i)."""
    D = x.shape[-1]
    h = D // 2
    w = theta ** (-2.0 * np.arange(h) / D)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, float)[:, None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


class _Decoder:
    def __init__(self, rng, layers=2, dm=24, hq=4, hkv=2, D=8, theta=1e4):
        self.hq, self.hkv, self.D, self.theta = hq, hkv, D, theta
        self.scale = 1.0 / np.sqrt(D)
        s = 0.3
        self.W = [dict(q=rng.standard_normal((dm, hq * D)) * s, k=rng.standard_normal((dm, hkv * D)) * s,
                       v=rng.standard_normal((dm, hkv * D)) * s, o=rng.standard_normal((hq * D, dm)) * s,
                       u=rng.standard_normal((dm, 2 * dm)) * s, d=rng.standard_normal((2 * dm, dm)) * s)
                  for _ in range(layers)]

    def _qkv(self, h, W):
        n = h.shape[0]
        return ((h @ W["q"]).reshape(n, self.hq, self.D), (h @ W["k"]).reshape(n, self.hkv, self.D),
                (h @ W["v"]).reshape(n, self.hkv, self.D))

    def _finish(self, h, att, W):
        h = h + att.reshape(h.shape[0], -1) @ W["o"]
        return h + np.tanh(h @ W["u"]) @ W["d"]

    def prefill(self, x, pos):
        """Full causal prefill (textbook); returns the last hidden states and
        every layer's pre-RoPE K and V."""
        h, kv = x, []
        g = self.hq // self.hkv
        for W in self.W:
            q, k, v = self._qkv(h, W)
            kv.append((k, v))
            qr, kr = _rope_complex(q, pos, self.theta), _rope_complex(k, pos, self.theta)
            att = np.stack([_masked_softmax_attention(qr[:, i], kr[:, i // g], v[:, i // g], pos, pos, self.scale)
                            for i in range(self.hq)], axis=1)
            h = self._finish(h, att, W)
        return h, kv

    def prefill_over_injected(self, x, pos, mem_kv, mem_pos):
        """Query-only prefill: each layer's attention reads the injected memory
        (pre-RoPE K rotated by Chunked RoPE to mem_pos, raw V) and the query
        tokens' own K/V, through the oracle's rotation and attention."""
        h = x
        g = self.hq // self.hkv
        kpos = np.concatenate([mem_pos, pos])
        for W, (mk, mv) in zip(self.W, mem_kv):
            q, k, v = self._qkv(h, W)
            keys = np.concatenate([oracle.rope_rotate(mk, mem_pos[:, None], self.theta),
                                   oracle.rope_rotate(k, pos[:, None], self.theta)])
            vals = np.concatenate([mv, v])
            qr = oracle.rope_rotate(q, pos[:, None], self.theta)
            att = np.stack([oracle.causal_attention(qr[:, i], keys[:, i // g], vals[:, i // g], pos, kpos, self.scale)
                            for i in range(self.hq)], axis=1)
            h = self._finish(h, att, W)
        return h


@pytest.mark.parametrize("seed, start", [(0, 0), (1, 37), (2, 1000)])
def test_theorem3_injected_memory_equals_prompt(seed, start):
    rng = np.random.default_rng(seed)
    dec = _Decoder(rng)
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
    dec = _Decoder(rng)
    lm, tq, start = 9, 4, 20
    mem, qry = rng.standard_normal((lm, 24)), rng.standard_normal((tq, 24))
    h_full, _ = dec.prefill(np.concatenate([mem, qry]), start + np.arange(lm + tq))
    _, mem_kv = dec.prefill(mem, np.arange(lm))
    h_bad = dec.prefill_over_injected(qry, start + lm + np.arange(tq), mem_kv, start - 1 + np.arange(lm))
    assert not np.allclose(h_bad, h_full[lm:], atol=1e-6)
