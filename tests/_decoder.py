"""A random-weight causal decoder in fp64, for the pins of the attention read
and of Context-Window Encoding.  Its RoPE is written with complex numbers,
independently of the oracle's rotate-half code; its full prefill uses a
masked-softmax matrix formula, independently of oracle.causal_attention.
Test infrastructure only."""

from __future__ import annotations

import numpy as np

import oracle


def masked_softmax_attention(q, k, v, qpos, kpos, scale):
    s = scale * (q @ k.T)
    s = np.where(kpos[None, :] <= qpos[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w / w.sum(axis=1, keepdims=True)) @ v


def rope_complex(x, pos, theta):
    """RoPE as multiplication of (x_i + i x_{i+D/2}) by exp(i p w_i)."""
    D = x.shape[-1]
    h = D // 2
    w = theta ** (-2.0 * np.arange(h) / D)
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, float)[:, None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


class Decoder:
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
            qr, kr = rope_complex(q, pos, self.theta), rope_complex(k, pos, self.theta)
            att = np.stack([masked_softmax_attention(qr[:, i], kr[:, i // g], v[:, i // g], pos, pos, self.scale)
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


