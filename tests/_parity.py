"""Shared helpers of the GPU parity tests: run the library on a workload and
compare what it wrote with the CPU oracle, element by element."""

from __future__ import annotations

import math
import sys
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
from kv_cache_injection_amd import fs, synth
from kv_cache_injection_amd.workload import DeviceStore, build_store, request_tensors

# K tolerance: at most 1 bf16 ulp from the oracle's correctly rounded value
K_MAX_ULP = 1
# Score tolerance: GPU fp64 accumulation vs the exactly rounded oracle sum.
# |err| <= E * 2^-53 * sum|e_j q_j| <= E * 2^-53 for unit vectors (E <= 1024).
SCORE_ABS_TOL = 1024 * 2.0**-53
# A top-k answer is certified when every score difference that decides it is
# larger than twice the score tolerance; otherwise equal-score candidates may
# legitimately swap and only validity is checked.
CERT_GAP = 2 * SCORE_ABS_TOL


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps between two arrays of bit patterns (+0 == -0)."""
    def ordered(x):
        x = x.astype(np.int32)
        mag = x & 0x7FFF
        return np.where(x & 0x8000, -mag, mag)
    return np.abs(ordered(a) - ordered(b))


def gpu_retrieve(ds: DeviceStore, req, k: int, batch: int):
    dev = req["query"].device
    ids = torch.full((batch, k), -7, dtype=torch.int32, device=dev)
    scores = torch.zeros((batch, k), dtype=torch.float64, device=dev)
    ntok = torch.full((batch,), -7, dtype=torch.int32, device=dev)
    fs.fs_retrieve_topk(ds.store, batch, req["user"], req["query"], k, ids, scores, ntok)
    return ids, scores, ntok


def check_retrieval(wl: synth.Workload, ids_gpu: np.ndarray, scores_gpu: np.ndarray,
                    ntok_gpu: np.ndarray, requests: Sequence[int], k: int) -> Dict[int, np.ndarray]:
    """Compare GPU top-k with the oracle for the given requests.  Returns the
    oracle's ids per request."""
    out = {}
    for b in requests:
        u = int(wl.users[b])
        a, e = int(wl.user_fact_begin[u]), int(wl.user_fact_begin[u + 1])
        s_all = oracle.score(wl.emb[a:e], wl.queries[b])
        local = oracle.select_topk(s_all, k)
        o_ids = np.full(k, -1, np.int64)
        o_sc = np.full(k, -np.inf)
        o_ids[: len(local)] = np.asarray(local, np.int64) + a
        o_sc[: len(local)] = s_all[local]
        out[b] = o_ids
        g_ids = ids_gpu[b].astype(np.int64)
        kk = min(k, e - a)
        gap = oracle.decisive_gap(s_all, k)
        if gap > CERT_GAP:
            assert np.array_equal(g_ids, o_ids), f"request {b}: ids differ"
        else:
            # near-tie: every GPU pick must be a valid fact whose exact score
            # matches the oracle's score at that rank within tolerance
            assert np.all(g_ids[kk:] == -1)
            assert len(set(g_ids[:kk])) == kk and np.all((g_ids[:kk] >= a) & (g_ids[:kk] < e))
            assert np.all(np.abs(s_all[g_ids[:kk] - a] - o_sc[:kk]) <= CERT_GAP)
            say(f"request {b}: near-tie (gap {gap:.3g}), validity checked")
        g_sc = scores_gpu[b]
        assert np.all(np.isneginf(g_sc[kk:]))
        assert np.all(np.abs(g_sc[:kk] - o_sc[:kk]) <= SCORE_ABS_TOL), f"request {b}: scores"
        _, L = oracle.compose(o_ids, wl.fact_len)
        assert int(ntok_gpu[b]) == L, f"request {b}: num_tokens {int(ntok_gpu[b])} != {L}"
    return out


def check_injection(wl: synth.Workload, ds: DeviceStore, kc: list, vc: list,
                    ids_by_req: Dict[int, np.ndarray], layer_idx: Sequence[int],
                    stats: Optional[dict] = None) -> None:
    """Compare the cache rows each listed request wrote with the oracle's
    rows for the same ids (all materialised layers in layer_idx)."""
    s = wl.shape
    ftb = wl.fact_token_begin
    for b, o_ids in ids_by_req.items():
        rows = oracle.segment_rows(o_ids, wl.fact_len, ftb)
        if rows.size == 0:
            continue
        pos = int(wl.start_pos[b]) + np.arange(rows.size)
        blk, slot = oracle.placement(pos, wl.block_table[b], s.block_size)
        rows_t = torch.from_numpy(rows).to(ds.k_pre[0].device)
        blk_t = torch.from_numpy(blk).cuda()
        slot_t = torch.from_numpy(slot).cuda()
        for li in layer_idx:
            kpre = synth.bf16_bits(ds.k_pre[li][rows_t])
            vpre = synth.bf16_bits(ds.v[li][rows_t])
            ek, ev = oracle.expected_rows(kpre, vpre, pos, s.rope_theta)
            gk = synth.bf16_bits(kc[li][blk_t, slot_t])
            gv = synth.bf16_bits(vc[li][blk_t, slot_t])
            assert np.array_equal(gv, ev), f"request {b} layer {li}: V bytes differ"
            d = bf16_ulp_distance(gk, ek)
            worst = int(d.max())
            if stats is not None:
                stats["elements"] = stats.get("elements", 0) + d.size
                stats["ulp1"] = stats.get("ulp1", 0) + int((d == 1).sum())
            assert worst <= K_MAX_ULP, f"request {b} layer {li}: K off by {worst} ulp"


def written_mask(wl: synth.Workload, ids_by_req: Dict[int, np.ndarray], num_blocks: int):
    """Boolean [num_blocks, block_size]: slots some request writes."""
    s = wl.shape
    m = np.zeros((num_blocks, s.block_size), bool)
    for b, o_ids in ids_by_req.items():
        _, L = oracle.compose(o_ids, wl.fact_len)
        if L == 0:
            continue
        pos = int(wl.start_pos[b]) + np.arange(L)
        blk, slot = oracle.placement(pos, wl.block_table[b], s.block_size)
        m[blk, slot] = True
    return m


def check_sentinel(kc: list, vc: list, mask: np.ndarray, layer_idx: Sequence[int]) -> None:
    """Every slot outside ``mask`` still holds the sentinel, in every byte, and
    every slot inside it was written."""
    sent = np.int16(np.uint16(synth.SENTINEL_BITS).view(np.int16)).item()
    keep = torch.from_numpy(~mask).cuda()
    wrote = torch.from_numpy(mask).cuda()
    for li in layer_idx:
        for name, c in (("K", kc[li]), ("V", vc[li])):
            untouched = c.view(torch.int16)[keep]
            bad = int((untouched != sent).sum())
            assert bad == 0, f"layer {li} {name}: {bad} elements changed outside the segment"
            written = c.view(torch.int16)[wrote]
            still = int((written == sent).sum())
            assert still == 0, f"layer {li} {name}: {still} elements of the segment not written"
