"""Glue between a synthetic Workload and the library: allocate the arenas and
caches with torch, describe the store, register it, upload request tensors.
Marshalling only — no step of the hot path runs here."""

from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch

from . import fs, synth


def make_desc(wl: synth.Workload, num_layers: int, *, max_batch: Optional[int] = None,
              max_k: Optional[int] = None, pinned: bool = False,
              staging_layers: int = 0) -> fs.fs_store_desc:
    s = wl.shape
    return fs.make_desc(
        num_layers=num_layers, num_kv_heads=s.num_kv_heads, head_dim=s.head_dim,
        embed_dim=s.embed_dim, rope_theta=float(s.rope_theta), block_size=s.block_size,
        kv_location=fs.FS_KV_PINNED_HOST if pinned else fs.FS_KV_DEVICE,
        num_users=s.num_users, max_batch=max_batch or s.batch,
        max_k=max_k or max(wl.k, 1), staging_layers=staging_layers,
        num_facts=int(wl.fact_len.size), num_tokens=wl.num_tokens)


@dataclasses.dataclass
class DeviceStore:
    wl: synth.Workload
    layers: List[int]                 # which of the shape's layers are materialised
    k_pre: list                       # per materialised layer, bf16 [T, H, D]
    v: list
    emb: torch.Tensor
    store: fs.Store

    def close(self):
        self.store.close()


def build_store(wl: synth.Workload, layers: Sequence[int], *, device="cuda", pinned=False,
                staging_layers: Optional[int] = None, max_batch: Optional[int] = None,
                max_k: Optional[int] = None) -> DeviceStore:
    layers = list(layers)
    k_pre, v = synth.make_arenas(wl, layers, device, pinned=pinned)
    emb = torch.from_numpy(wl.emb).to(device)
    sl = (staging_layers or len(layers)) if pinned else 0
    desc = make_desc(wl, len(layers), max_batch=max_batch, max_k=max_k, pinned=pinned,
                     staging_layers=sl)
    store = fs.fs_create_store(desc, wl.user_fact_begin, wl.fact_len, emb, k_pre, v)
    return DeviceStore(wl, layers, k_pre, v, emb, store)


def request_tensors(wl: synth.Workload, device="cuda", *, queries=None, start_pos=None,
                    block_table=None):
    """Device copies of one batch's request inputs."""
    q = wl.queries if queries is None else queries
    sp = wl.start_pos if start_pos is None else start_pos
    bt = wl.block_table if block_table is None else block_table
    return {
        "user": torch.from_numpy(np.ascontiguousarray(wl.users, np.int32)).to(device),
        "query": torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(device),
        "start_pos": torch.from_numpy(np.ascontiguousarray(sp, np.int32)).to(device),
        "block_table": torch.from_numpy(np.ascontiguousarray(bt, np.int32)).to(device),
    }
