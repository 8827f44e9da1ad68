"""Seeded synthetic inputs for the KV-injection hot path.

This module draws random numbers and lays them out in the shapes the serving
workloads use.  It holds none of the method's arithmetic: no scoring, no
selection, no rotation and no placement.  Tests, the bench and the CPU oracle's
callers all take their inputs from here, so both sides of a parity check see
the same bytes.

Workloads (model shapes follow the three open-weight models the InferScale
pages evaluate on, "Résultats"/"Resultados" sections of the gist.science
summaries; the pages publish no fact counts, lengths or embedding sizes, so
those are chosen here and recorded in the config table below):

  tiny        1 layer, 8 KV heads, head_dim 128, theta 5e5, 256 facts x 16 tokens,
              384-d embeddings, k=5, 64 blocks (a permutation), start_pos 37
  llama       Llama-3.1-8B shape: 32 layers, 8 KV heads, head_dim 128, theta 5e5,
              2,000 facts of U[12,48] tokens, 768-d, one request, k=50
  qwen        Qwen2.5-7B shape: 28 layers, 4 KV heads, theta 1e6, 5,000 facts,
              768-d, one request, k in {5,10,20,50}
  concurrent  Llama shape, 100 users x 1,000 facts, 100 requests (one per user),
              k=50, start_pos U[0,512), one shared pool of 20,000 blocks
  large       Mistral-7B shape: 32 layers, 8 KV heads, theta 1e6, 20,000 facts of
              U[16,44] tokens, 1024-d, 32 requests of one user, k=50

Random streams: numpy.random.SeedSequence(seed) spawns one child per named
stream (lengths, emb, query, start_pos, block_table, kv) so each part can be
regenerated alone.  Embeddings and queries are fp32 N(0,1) rows normalised in
fp64 and rounded to fp32.  K/V arenas are bf16 N(0,1) drawn by torch's
generator on the device that will hold them (the CPU oracle reads the bytes
back, never regenerates them).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

STREAMS = ("lengths", "emb", "query", "start_pos", "block_table", "kv", "sentinel")

# bf16 bit pattern written over every cache byte before an injection, so that
# any slot the injection must not touch can be checked byte for byte.
SENTINEL_BITS = 0xFFFF


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    num_layers: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    embed_dim: int
    num_users: int
    facts_per_user: int
    len_lo: int              # inclusive
    len_hi: int              # inclusive
    batch: int
    k: int
    start_lo: int            # inclusive
    start_hi: int            # exclusive
    pool_blocks: int         # physical blocks per layer in the paged cache
    table: str               # "permuted" | "free" | "shared_pool"
    block_size: int = 16
    one_user: bool = False   # every request of the batch belongs to user 0

    @property
    def num_facts(self) -> int:
        return self.num_users * self.facts_per_user

    @property
    def max_blocks(self) -> int:
        """Block-table width: enough logical blocks for the latest start
        position plus k facts of the longest length (the permuted table of the
        tiny case spans the whole pool)."""
        if self.table == "permuted":
            return self.pool_blocks
        worst = (self.start_hi - 1) + self.k * self.len_hi
        return -(-worst // self.block_size)


CONFIGS: Dict[str, Shape] = {
    "tiny": Shape("tiny", 1, 8, 128, 5e5, 384, 1, 256, 16, 16, 1, 5, 37, 38, 64,
                  "permuted"),
    "llama": Shape("llama", 32, 8, 128, 5e5, 768, 1, 2000, 12, 48, 1, 50, 0, 256,
                   512, "free"),
    "qwen": Shape("qwen", 28, 4, 128, 1e6, 768, 1, 5000, 12, 48, 1, 50, 0, 256,
                  512, "free"),
    "concurrent": Shape("concurrent", 32, 8, 128, 5e5, 768, 100, 1000, 12, 48, 100,
                        50, 0, 512, 20000, "shared_pool"),
    "large": Shape("large", 32, 8, 128, 1e6, 1024, 1, 20000, 16, 44, 32, 50, 0,
                   512, 6000, "shared_pool", one_user=True),
}

DEFAULT_SEEDS = {"tiny": 1000, "llama": 1001, "qwen": 1002, "concurrent": 1003,
                 "large": 1004}


def _rngs(seed: int) -> Dict[str, np.random.Generator]:
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.default_rng(c) for name, c in zip(STREAMS, children)}


def _torch_seed(seed: int, *tag: int) -> int:
    ss = np.random.SeedSequence([seed, 0x6B76, *tag])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 62) - 1))


def _unit_rows(rng: np.random.Generator, n: int, dim: int) -> np.ndarray:
    x = rng.standard_normal((n, dim), dtype=np.float32)
    norms = np.sqrt(np.einsum("ij,ij->i", x.astype(np.float64), x.astype(np.float64)))
    return (x.astype(np.float64) / norms[:, None]).astype(np.float32)


@dataclasses.dataclass
class Workload:
    """One store plus one batch of requests (host arrays)."""
    shape: Shape
    seed: int
    fact_len: np.ndarray          # int32 [F]
    user_fact_begin: np.ndarray   # int64 [U+1]
    emb: np.ndarray               # float32 [F, E]
    users: np.ndarray             # int32 [B]
    queries: np.ndarray           # float32 [B, E]
    start_pos: np.ndarray         # int32 [B]
    block_table: np.ndarray       # int32 [B, max_blocks]
    k: int

    @property
    def num_tokens(self) -> int:
        return int(self.fact_len.sum(dtype=np.int64))

    @property
    def fact_token_begin(self) -> np.ndarray:
        """Token offset of every fact in the arenas (facts are stored back to
        back in fact order); int64 [F+1].  Layout bookkeeping only."""
        out = np.zeros(self.fact_len.size + 1, np.int64)
        np.cumsum(self.fact_len, out=out[1:])
        return out


def make_workload(shape: Shape | str, seed: Optional[int] = None, *,
                  k: Optional[int] = None, batch: Optional[int] = None,
                  num_users: Optional[int] = None,
                  facts_per_user: Optional[int] = None) -> Workload:
    """Draw the host-side part of a workload (everything except the K/V
    arenas).  ``batch``/``num_users``/``facts_per_user`` shrink a shape for
    quick tests; ``k`` picks the retrieval budget (default: the shape's)."""
    if isinstance(shape, str):
        if seed is None:
            seed = DEFAULT_SEEDS[shape]
        shape = CONFIGS[shape]
    if seed is None:
        seed = DEFAULT_SEEDS.get(shape.name, 0)
    repl = {}
    if batch is not None:
        repl["batch"] = batch
    if num_users is not None:
        repl["num_users"] = num_users
    if facts_per_user is not None:
        repl["facts_per_user"] = facts_per_user
    if repl:
        shape = dataclasses.replace(shape, **repl)
    k = shape.k if k is None else k
    r = _rngs(seed)

    F = shape.num_facts
    fact_len = r["lengths"].integers(shape.len_lo, shape.len_hi + 1, size=F).astype(np.int32)
    user_fact_begin = (np.arange(shape.num_users + 1, dtype=np.int64) * shape.facts_per_user)
    emb = _unit_rows(r["emb"], F, shape.embed_dim)

    users, queries, start_pos, table = _draw_requests(shape, r)
    return Workload(shape, seed, fact_len, user_fact_begin, emb, users, queries,
                    start_pos, table, k)


def _draw_requests(shape: Shape, r: Dict[str, np.random.Generator]):
    B = shape.batch
    if shape.one_user or shape.num_users == 1:
        users = np.zeros(B, np.int32)
    else:
        if B > shape.num_users:
            raise ValueError("one request per user needs batch <= num_users")
        users = np.arange(B, dtype=np.int32)
    queries = _unit_rows(r["query"], B, shape.embed_dim)
    start_pos = r["start_pos"].integers(shape.start_lo, shape.start_hi, size=B).astype(np.int32)

    mb = shape.max_blocks
    rb = r["block_table"]
    if shape.table == "permuted":
        table = np.stack([rb.permutation(shape.pool_blocks)[:mb] for _ in range(B)])
    elif shape.table == "free":
        table = np.stack([rb.choice(shape.pool_blocks, size=mb, replace=False)
                          for _ in range(B)])
    elif shape.table == "shared_pool":
        if B * mb > shape.pool_blocks:
            raise ValueError("shared pool too small for the batch")
        table = rb.permutation(shape.pool_blocks)[: B * mb].reshape(B, mb)
    else:
        raise ValueError(shape.table)
    return users, queries, start_pos, table.astype(np.int32)


def request_sets(wl: Workload, n: int, seed: int) -> List[Dict[str, np.ndarray]]:
    """``n`` further (query, start_pos, block_table) sets for the same store,
    used to vary the requests between timed steps."""
    out = []
    for i in range(n):
        _, queries, start_pos, table = _draw_requests(wl.shape, _rngs(seed + 7919 * (i + 1)))
        out.append({"queries": queries, "start_pos": start_pos, "block_table": table})
    return out


# --------------------------------------------------------------------------
# K/V arenas and paged caches (torch tensors; torch is only the allocator and
# the random-number source here)
# --------------------------------------------------------------------------

def make_arenas(wl: Workload, layers: Sequence[int], device, *, pinned: bool = False):
    """Per-layer pre-RoPE key and value arenas, bf16 [T, H, D], N(0,1).

    ``layers`` selects which of the shape's layers to materialise (the rest are
    not allocated).  With ``pinned`` the arenas live in page-locked host memory;
    they are drawn on ``device`` first and copied over.
    Returns (k_list, v_list) aligned with ``layers``."""
    import torch
    s = wl.shape
    T = wl.num_tokens
    ks, vs = [], []
    for l in layers:
        pair = []
        for which in (0, 1):
            g = torch.Generator(device=device)
            g.manual_seed(_torch_seed(wl.seed, l, which))
            t = torch.randn((T, s.num_kv_heads, s.head_dim), generator=g,
                            device=device, dtype=torch.bfloat16)
            if pinned:
                h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
                h.copy_(t)
                del t
                t = h
            pair.append(t)
        ks.append(pair[0])
        vs.append(pair[1])
    return ks, vs


def make_caches(wl: Workload, layers: Sequence[int], device, num_blocks: Optional[int] = None):
    """Per-layer paged K and V caches, bf16 [num_blocks, block_size, H, D],
    every byte set to the sentinel pattern."""
    import torch
    s = wl.shape
    nb = s.pool_blocks if num_blocks is None else num_blocks
    shape = (nb, s.block_size, s.num_kv_heads, s.head_dim)
    kc, vc = [], []
    for _ in layers:
        for lst in (kc, vc):
            t = torch.empty(shape, dtype=torch.int16, device=device)
            t.fill_(np.int16(np.uint16(SENTINEL_BITS).view(np.int16)).item())
            lst.append(t.view(torch.bfloat16))
    return kc, vc


def bf16_bits(t) -> np.ndarray:
    """Host uint16 copy of a bf16 tensor's bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def clustered_embeddings(n: int, dim: int, topics: int, spread: float, seed: int):
    """Unit rows drawn around ``topics`` random unit centres (centre +
    spread * N(0, I/dim), normalised in fp64, rounded to fp32), and each row's
    topic.  Stands in for the topical structure of a user's memory, which an
    approximate index relies on; no real text is involved."""
    ss = np.random.SeedSequence(seed)
    g_c, g_t, g_n = [np.random.default_rng(x) for x in ss.spawn(3)]
    centres = g_c.standard_normal((topics, dim))
    centres /= np.linalg.norm(centres, axis=1, keepdims=True)
    topic = g_t.integers(0, topics, n)
    out = np.empty((n, dim), np.float32)
    step = 65536
    for a in range(0, n, step):
        b = min(n, a + step)
        x = centres[topic[a:b]] + spread * g_n.standard_normal((b - a, dim)) / np.sqrt(dim)
        out[a:b] = (x / np.linalg.norm(x, axis=1, keepdims=True)).astype(np.float32)
    return out, topic
