"""Plain fp64 CPU oracle of the InferScale serving-time KV-injection path.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Shares no code with the GPU library.

Sources (the web pages on "InferScale: GPU-Native KV Injection for
Personalized LLM Serving", Li & Pandey, arXiv 2607.27090):
  [abstract]  astralor.com feed item, section "Full text" (the paper's abstract)
  [online]    gist.science technical summary, section "Phase En-ligne : RoPE par
              Morceaux (Chunked RoPE) et Injection de KV" (fr); the same text is
              "Fase Online" (es) and "온라인 단계" (ko)
  [contrib]   gist.science summary, "Contributions Clés" / "Contribuciones Clave"
  [problem]   gist.science summary, "Problématique" / "Planteamiento del Problema"
  [results]   gist.science summary, "Résultats" / "Resultados" (host offload)

What the pages fix, and the readings taken where they are silent:
  * Each fact's keys are stored *before* RoPE, together with the raw values
    and a semantic embedding, on the GPU [abstract; online "Stockage Pré-RoPE"].
  * At serving time the retrieved facts are composed into one contiguous
    segment and each stored key is rotated to its new position [online
    "Rotation Dynamique"].  Reading: the segment starts at the request's
    start position, facts follow in rank order (best score first), with no
    gaps or separators.
  * The composed K/V is scatter-copied into the paged KV cache [online
    "Injection"].  Reading: position p goes to physical block
    block_table[p // block_size], slot p % block_size; nothing else changes.
  * Re-rotation is exact under RoPE (Theorem 6, stated on the pages only in
    words): <R(m)q, R(n)k> = <q, R(n-m)k>.
  * Retrieval picks the top-k facts by semantic similarity with budget k
    [problem; contrib "Conception de Système Native au GPU"].  Reading: the
    similarity is the inner product of L2-normalised fp32 embeddings, exact
    products summed and rounded once to fp64; ties go to the lower fact index.
  * RoPE variant (the pages name the models, not the variant): rotate-half
    pairing (element i with i + D/2), frequency w_i = theta^(-2i/D), no
    frequency scaling.
  * Values are stored and injected unchanged [online]: copied byte for byte.
  * Keys are produced in bf16: the exact fp64 rotation rounded once to the
    nearest bf16, ties to even.

bf16 tensors are handled as numpy uint16 arrays of bit patterns.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = [
    "bf16_to_f64", "f64_to_bf16", "score", "select_topk", "decisive_gap",
    "retrieve", "compose", "segment_rows", "placement", "request_problem",
    "rope_inv_freq", "rope_rotate", "inject_request", "expected_rows",
    "gather_rows", "causal_attention", "attend_prefill", "ivf_probe", "ivf_init", "ivf_update", "cwe_window",
    "capture_rows",
]


# --------------------------------------------------------------------------
# bf16 <-> fp64
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of each bf16 bit pattern (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even, in ONE step
    (never through an fp32 intermediate).  Returns uint16 bit patterns.

    bf16 carries 8 significant bits over fp32's exponent range: in the binade
    [2^(e-1), 2^e) its spacing is 2^(e-8), and it never gets finer than the
    subnormal spacing 2^-133.  Scaling by that spacing is exact, np.rint rounds
    to the nearest integer with ties to even, and the rounded value is exactly
    representable in fp32, so the final cast only changes the container.
    Values whose rounding exceeds the largest bf16 become +-inf."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    r = np.rint(np.ldexp(x, -q))
    y = np.ldexp(r, q)
    with np.errstate(over="ignore"):
        f = y.astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# Retrieval: score + top-k
# --------------------------------------------------------------------------

def score(emb_rows: np.ndarray, query: np.ndarray) -> np.ndarray:
    """Similarity of one query with each fact embedding [problem; contrib]:
    s_i = sum_j e_ij * q_j.  Every fp32*fp32 product is exact in fp64 and
    math.fsum returns the exactly rounded sum, so s_i is the exact inner
    product rounded once to fp64 (independent of summation order)."""
    e = np.asarray(emb_rows, dtype=np.float32).astype(np.float64)
    q = np.asarray(query, dtype=np.float32).astype(np.float64)
    prods = e * q[None, :]
    return np.array([math.fsum(row) for row in prods.tolist()], dtype=np.float64)


def select_topk(scores: Sequence[float], k: int) -> List[int]:
    """The min(k, N) highest-scoring positions, best first; equal scores are
    ordered by lower position [problem: retrieval budget k]."""
    s = list(map(float, scores))
    order = sorted(range(len(s)), key=lambda i: (-s[i], i))
    return order[: max(0, min(k, len(s)))]


def decisive_gap(scores: Sequence[float], k: int) -> float:
    """Smallest score difference that decides the top-k answer: between
    neighbours inside the selected ranks and between rank k and rank k+1.
    Exact ties (gap 0) are decided by the index rule, so they are skipped.
    Returns +inf when nothing is decided by a score difference."""
    s = np.sort(np.asarray(scores, dtype=np.float64))[::-1]
    kk = min(k, s.size)
    m = min(kk + 1, s.size)
    d = s[: m - 1] - s[1:m]
    d = d[d > 0]
    return float(d.min()) if d.size else math.inf


def retrieve(emb: np.ndarray, user_fact_begin: np.ndarray, user: int,
             query: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Top-k facts of one user's store for one query: the retrieval step that
    runs when a request is served [abstract].  Returns (global fact ids,
    scores), both of length k with -1 / -inf padding past min(k, N_user)."""
    a, b = int(user_fact_begin[user]), int(user_fact_begin[user + 1])
    s = score(emb[a:b], query)
    local = select_topk(s, k)
    ids = np.full(max(k, 0), -1, np.int64)
    sc = np.full(max(k, 0), -np.inf, np.float64)
    ids[: len(local)] = np.asarray(local, np.int64) + a
    sc[: len(local)] = s[local]
    return ids, sc


# --------------------------------------------------------------------------
# Composition and placement
# --------------------------------------------------------------------------

def compose(ids: Sequence[int], fact_len: np.ndarray) -> Tuple[List[int], int]:
    """Composition of the retrieved facts into one contiguous segment
    [online "Rotation Dynamique"]: fact j starts at offset off_j = sum of the
    lengths of the facts before it.  Padding ids (-1) end the list.
    Returns (offsets [k'+1], total length L)."""
    off = [0]
    for f in ids:
        if f < 0:
            break
        off.append(off[-1] + int(fact_len[f]))
    return off, off[-1]


def segment_rows(ids: Sequence[int], fact_len: np.ndarray,
                 fact_token_begin: np.ndarray) -> np.ndarray:
    """Arena row of every token of the composed segment, in segment order."""
    rows = []
    for f in ids:
        if f < 0:
            break
        b = int(fact_token_begin[f])
        rows.extend(range(b, b + int(fact_len[f])))
    return np.asarray(rows, dtype=np.int64)


def placement(pos, block_table: np.ndarray, block_size: int):
    """Paged-cache address of absolute position p [online "Injection"]:
    (block_table[p // block_size], p % block_size)."""
    pos = np.asarray(pos, dtype=np.int64)
    return np.asarray(block_table, np.int64)[pos // block_size], pos % block_size


def request_problem(ids: Sequence[int], user_range: Tuple[int, int],
                    fact_len: np.ndarray, start_pos: int, block_table: np.ndarray,
                    num_blocks: int, block_size: int) -> List[str]:
    """Reasons a request cannot be placed (empty list when it can):
    'fact_id'     an id outside the request's user, or padding before a real id
    'start_pos'   negative start position or a position past int32
    'block_short' the table has fewer than ceil((s+L)/block_size) entries
    'block_id'    a table entry the segment uses is outside [0, num_blocks)"""
    out = []
    a, b = user_range
    seen_pad = False
    for f in ids:
        if f < 0:
            seen_pad = True
            continue
        if seen_pad or not (a <= f < b):
            out.append("fact_id")
            break
    if out:
        return out
    _, L = compose(ids, fact_len)
    if start_pos < 0 or start_pos + L > 2**31 - 1:
        return ["start_pos"]
    if L == 0:
        return []
    first, last = start_pos // block_size, (start_pos + L - 1) // block_size
    if last >= len(block_table):
        return ["block_short"]
    used = np.asarray(block_table[first:last + 1], np.int64)
    if np.any((used < 0) | (used >= num_blocks)):
        return ["block_id"]
    return []


# --------------------------------------------------------------------------
# Chunked RoPE
# --------------------------------------------------------------------------

def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """w_i = theta^(-2i/D), i < D/2 (the RoPE frequencies)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / head_dim)


def rope_rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """R(p) applied to fp64 vectors x[..., D] at integer positions ``pos``
    (broadcast against x[..., 0]) — the rotation Chunked RoPE applies at
    serving time [online "Rotation Dynamique"], rotate-half pairing:
        y_i       = x_i cos(p w_i) - x_{i+D/2} sin(p w_i)
        y_{i+D/2} = x_{i+D/2} cos(p w_i) + x_i sin(p w_i)"""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    a = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(D, theta)
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# Injection
# --------------------------------------------------------------------------

def expected_rows(k_pre_rows: np.ndarray, v_rows: np.ndarray, pos, theta: float):
    """Cache contents for composed tokens: K = bf16(R(p) k_pre), V = the raw
    value bytes.  k_pre_rows / v_rows are uint16 [..., H, D]; pos is one
    position per leading index."""
    x = bf16_to_f64(k_pre_rows)
    p = np.asarray(pos, dtype=np.int64)[..., None]        # broadcast over heads
    k = f64_to_bf16(rope_rotate(x, p, theta))
    return k, np.array(v_rows, dtype=np.uint16, copy=True)


def inject_request(k_pre: Sequence[np.ndarray], v: Sequence[np.ndarray],
                   k_cache: Sequence[np.ndarray], v_cache: Sequence[np.ndarray],
                   ids: Sequence[int], fact_len: np.ndarray,
                   fact_token_begin: np.ndarray, start_pos: int,
                   block_table: np.ndarray, block_size: int, theta: float,
                   layers: Sequence[int]) -> int:
    """One request's injection into the paged cache, all given layers
    [online "Rotation Dynamique" + "Injection"].  Arrays are uint16 bit
    patterns: k_pre[l], v[l] are [T, H, D]; k_cache[l], v_cache[l] are
    [num_blocks, block_size, H, D] and are updated in place (lists indexed by
    the position in ``layers``).  Returns the segment length L."""
    rows = segment_rows(ids, fact_len, fact_token_begin)
    L = rows.size
    if L == 0:
        return 0
    pos = start_pos + np.arange(L, dtype=np.int64)
    blk, slot = placement(pos, block_table, block_size)
    for i, _ in enumerate(layers):
        kk, vv = expected_rows(k_pre[i][rows], v[i][rows], pos, theta)
        k_cache[i][blk, slot] = kk
        v_cache[i][blk, slot] = vv
    return L


# --------------------------------------------------------------------------
# Host offload
# --------------------------------------------------------------------------

def gather_rows(arena: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Fetching selected facts from a host-resident store [results: the KV
    store can be offloaded to host DRAM] moves bytes only: the staged rows are
    the arena rows, unchanged."""
    return np.array(arena[np.asarray(rows, np.int64)], copy=True)


# --------------------------------------------------------------------------
# Attention read of the injected cache
# --------------------------------------------------------------------------

def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos, k_pos,
                     scale: float) -> np.ndarray:
    """Softmax attention of queries over keys at positions not after their own
    (a causal decoder's attention, the setting of Theorem 3 as the pages state
    it [contrib]), in fp64: for query i,
        out_i = sum_j a_ij v_j,  a_ij = exp(scale <q_i, k_j>) / sum_j' (...)
    over the keys j with k_pos[j] <= q_pos[i].  q [Nq, D], k and v [Nk, D]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    q_pos = np.asarray(q_pos, np.int64)
    k_pos = np.asarray(k_pos, np.int64)
    out = np.zeros((q.shape[0], v.shape[1]))
    for i in range(q.shape[0]):
        sel = k_pos <= q_pos[i]
        s = scale * (k[sel] @ q[i])
        w = np.exp(s - s.max())
        out[i] = (w / w.sum()) @ v[sel]
    return out


def attend_prefill(q_pre: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                   block_table: np.ndarray, block_size: int, ctx_begin: int, q_pos: int,
                   theta: float, scale: float) -> np.ndarray:
    """One request's prefill attention over one layer's paged cache.

    q_pre: uint16 bf16 bits [Tq, Hq, D], before RoPE; token j is at position
    q_pos + j and is rotated by R(q_pos + j) and rounded once to bf16 (the
    same treatment the injected keys get).  k_cache / v_cache: uint16 bits
    [num_blocks, block_size, Hkv, D]; position p is read from
    (block_table[p // block_size], p % block_size).  Query head h reads KV head
    h // (Hq / Hkv).  Token j attends to positions ctx_begin .. q_pos + j.
    Returns fp64 [Tq, Hq, D]."""
    tq, hq, D = q_pre.shape
    hkv = k_cache.shape[2]
    group = hq // hkv
    qpos = q_pos + np.arange(tq, dtype=np.int64)
    qr = bf16_to_f64(f64_to_bf16(rope_rotate(bf16_to_f64(q_pre), qpos[:, None], theta)))
    kpos = np.arange(ctx_begin, q_pos + tq, dtype=np.int64)
    blk, slot = placement(kpos, block_table, block_size)
    kr = bf16_to_f64(k_cache[blk, slot])             # [N, Hkv, D]
    vr = bf16_to_f64(v_cache[blk, slot])
    out = np.zeros((tq, hq, D))
    for h in range(hq):
        g = h // group
        out[:, h] = causal_attention(qr[:, h], kr[:, g], vr[:, g], qpos, kpos, scale)
    return out


# --------------------------------------------------------------------------
# Approximate retrieval through an inverted-file index
# --------------------------------------------------------------------------

def ivf_probe(emb: np.ndarray, centroids: np.ndarray, list_begin: np.ndarray,
              members: np.ndarray, query: np.ndarray, nprobe: int, k: int):
    """What an inverted-file probe returns (the pages keep a GPU-resident
    retrieval index [contrib] and do not describe it; this is the index's own
    definition): lists ranked by (centroid score desc, list index asc); the
    candidates are the facts of the first ``nprobe`` lists; the result is their
    k best by (score desc, fact id asc), scores exact as in ``score``.
    ``members`` holds global fact ids (rows of ``emb``).  Returns (ids padded
    with -1, scores padded with -inf)."""
    cs = score(centroids, query)
    lists = select_topk(cs, nprobe)
    cand = np.concatenate([np.asarray(members[list_begin[c]:list_begin[c + 1]], np.int64)
                           for c in lists]) if len(lists) else np.zeros(0, np.int64)
    s = score(emb[cand], query) if cand.size else np.zeros(0)
    order = np.lexsort((cand, -s))[:k]
    ids = np.full(k, -1, np.int64)
    sc = np.full(k, -np.inf)
    ids[: order.size] = cand[order]
    sc[: order.size] = s[order]
    return ids, sc


def ivf_init(emb: np.ndarray, nlist: int) -> np.ndarray:
    """The index's starting centroids (its own definition, as for
    ``ivf_probe``): centroid c is row floor(c * N / nlist) of ``emb``,
    scaled to unit length in fp64.  Returns fp64 [nlist, E]."""
    n = emb.shape[0]
    rows = np.asarray(emb, np.float64)[[c * n // nlist for c in range(nlist)]]
    norm = np.sqrt((rows * rows).sum(axis=1, keepdims=True))
    return np.where(norm > 0, rows / np.where(norm > 0, norm, 1.0), 0.0)


def ivf_update(emb: np.ndarray, list_begin: np.ndarray, members: np.ndarray,
               prev: np.ndarray) -> np.ndarray:
    """One spherical k-means update (the index's own definition): each
    centroid becomes the unit vector along the sum of its list's embeddings,
    the direction that maximises the sum of the members' inner products with
    a unit vector; an empty list, or a zero sum, keeps the previous centroid.
    ``members`` holds rows of ``emb``.  Returns fp64 [nlist, E]."""
    out = np.array(prev, np.float64, copy=True)
    e64 = np.asarray(emb, np.float64)
    for c in range(len(list_begin) - 1):
        rows = np.asarray(members[list_begin[c]:list_begin[c + 1]], np.int64)
        if rows.size == 0:
            continue
        v = e64[rows].sum(axis=0)
        norm = math.sqrt(float(v @ v))
        if norm > 0:
            out[c] = v / norm
    return out


# --------------------------------------------------------------------------
# Context-Window Encoding: which tokens the encoder sees, which rows are kept
# --------------------------------------------------------------------------

def cwe_window(turn_len: Sequence[int], j: int, w: int) -> Tuple[int, int, int, int]:
    """Context-Window Encoding of fact j (conversation turn j) with a window
    of w turns [offline "Encodage de la Fenêtre de Contexte"]: the encoder
    reads turns max(0, j - w) .. j as one sequence, and only the fact's own
    tokens are kept.  Returns (first token, end token) of the window in the
    conversation, and (keep_begin, keep_len) of the fact inside the window."""
    starts = np.concatenate([[0], np.cumsum(np.asarray(turn_len, np.int64))])
    a = int(starts[max(0, j - w)])
    b = int(starts[j + 1])
    return a, b, int(starts[j]) - a, int(turn_len[j])


def capture_rows(window: np.ndarray, keep_begin: int, keep_len: int) -> np.ndarray:
    """The stored part of a window's pre-RoPE K (or raw V): the fact's rows,
    bytes unchanged; the context rows are discarded."""
    return np.array(window[keep_begin:keep_begin + keep_len], copy=True)
