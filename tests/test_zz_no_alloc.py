"""fs_inject_noalloc, the inject entry point that allocates nothing (its
plan lives in the library's static per-GPU buffer), against fs_inject bit
for bit through the C ABI: two calls in a row, the second with fewer
requests, a smaller k and one layer, so it runs over the first call's
leftover plan.  Also its size limit."""

import numpy as np
import pytest
import torch

from _parity import say
from kv_cache_injection_amd import fs, synth
from kv_cache_injection_amd.workload import build_store, request_tensors

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16)


def test_noalloc_inject_matches_fs_inject_twice():
    wl = synth.make_workload("concurrent", num_users=6, facts_per_user=150, batch=6)
    s = wl.shape
    layers = [0, 1, 2]
    B, k = s.batch, wl.k
    mb = wl.block_table.shape[1]
    say("noalloc: building store")
    ds = build_store(wl, layers)
    req = request_tensors(wl)
    ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
    fs.fs_retrieve_topk(ds.store, B, req["user"], req["query"], k, ids, None, None)
    sent = np.int16(np.uint16(synth.SENTINEL_BITS).view(np.int16)).item()
    for call, (b, kk, layer) in enumerate(((B, k, fs.FS_ALL_LAYERS), (2, k // 2, 1))):
        say(f"noalloc: call {call}: batch {b}, k {kk}, layer {layer}")
        args = (b, req["user"][:b], ids[:b, :kk].contiguous(), kk, req["block_table"][:b].contiguous(), mb,
                req["start_pos"][:b])
        kc, vc = synth.make_caches(wl, layers, "cuda")
        rk, rv = synth.make_caches(wl, layers, "cuda")
        nb = kc[0].shape[0]
        fs.fs_inject_noalloc(ds.store, layer, *args, fs.CacheTable(ds.store, kc, vc, nb))
        fs.fs_inject(ds.store, layer, *args, fs.CacheTable(ds.store, rk, rv, nb))
        torch.cuda.synchronize()
        assert fs.fs_poll_errors(ds.store) == 0
        for l in range(len(layers)):
            assert torch.equal(_bits(kc[l]), _bits(rk[l])), f"call {call} layer {l} K"
            assert torch.equal(_bits(vc[l]), _bits(rv[l])), f"call {call} layer {l} V"
            written = bool((_bits(kc[l]) != sent).any())
            assert written == (layer == fs.FS_ALL_LAYERS or layer == l), f"call {call} layer {l}"
    ds.close()


def test_noalloc_inject_refuses_a_plan_beyond_its_buffer():
    # one 48-token fact, 100 requests of k = 64: a plan of about 4.9 MB
    E, T = 16, 48
    emb = torch.nn.functional.normalize(torch.randn((1, E), device="cuda"), dim=1).contiguous()
    k_pre = [torch.zeros((T, 1, 64), dtype=torch.bfloat16, device="cuda")]
    v = [torch.zeros((T, 1, 64), dtype=torch.bfloat16, device="cuda")]
    desc = fs.make_desc(num_layers=1, num_kv_heads=1, head_dim=64, embed_dim=E, rope_theta=1e4,
                        block_size=16, num_users=1, max_batch=100, max_k=64, num_facts=1, num_tokens=T)
    st = fs.fs_create_store(desc, np.array([0, 1], np.int64), np.array([T], np.int32), emb, k_pre, v)
    assert fs.fs_inject_plan_size(st, 100) > fs.FS_NOALLOC_PLAN_BYTES
    assert fs.fs_inject_plan_size(st, 50) <= fs.FS_NOALLOC_PLAN_BYTES
    kc = [torch.zeros((8, 16, 1, 64), dtype=torch.bfloat16, device="cuda")]
    tb = fs.CacheTable(st, kc, [torch.zeros_like(kc[0])], 8)
    user = torch.zeros(100, dtype=torch.int32, device="cuda")
    ids = torch.full((100, 64), -1, dtype=torch.int32, device="cuda")
    ids[:, 0] = 0
    bt = torch.zeros((100, 4), dtype=torch.int32, device="cuda")
    sp = torch.zeros(100, dtype=torch.int32, device="cuda")
    with pytest.raises(fs.FsError) as e:
        fs.fs_inject_noalloc(st, 0, 100, user, ids, 64, bt, 4, sp, tb)
    assert e.value.status == fs.FS_E_RANGE
    torch.cuda.synchronize()
    assert bool((kc[0] == 0).all())
    # within the buffer: every request writes the fact's 48 rows into blocks 0..2
    fs.fs_inject_noalloc(st, 0, 50, user[:50], ids[:50].contiguous(), 64, bt[:50].contiguous(), 4, sp[:50], tb)
    torch.cuda.synchronize()
    assert fs.fs_poll_errors(st) == 0
    st.close()
