"""fs_retrieve_plan on the GPU: retrieval whose selection also writes the
inject plan of the selected ids.

It must write exactly what fs_retrieve_topk writes (ids, scores, segment
lengths) and the plan that fs_plan_inject writes from those ids (header,
per-request length and start, every token's arena row and cache slot), set
the same device error bits, and fs_inject_planned from it must write what
fs_inject writes (which the parity tests compare with the oracle; the Llama
case is also checked against the oracle here).  Covered: every selection
path of the top-k kernel (one-wave sort, ranking, radix select, all-equal
scores, the 1024-thread block, the two-phase selection of a large user),
block tables longer than the prefetched window, k = 0, and each request
rejection the plan checks.
"""

import gc

import numpy as np
import pytest
import torch

from _parity import check_injection, check_retrieval, say
from kv_cache_injection_amd import fs, synth
from kv_cache_injection_amd.workload import build_store, request_tensors

pytestmark = pytest.mark.gpu

PLAN_HEADER = 32
REQ_BYTES = 8
TOK_BYTES = 16


@pytest.fixture(autouse=True)
def _cleanup():
    yield
    gc.collect()
    if torch.cuda.is_available():
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


def _small_store(emb, ufb, fact_len, H=2, D=128, bs=16, max_k=8, max_batch=4, num_layers=1):
    T = int(np.sum(fact_len))
    g = torch.Generator(device="cuda")
    g.manual_seed(int(T))
    k_pre = [torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(num_layers)]
    v = [torch.randn((T, H, D), generator=g, device="cuda").to(torch.bfloat16) for _ in range(num_layers)]
    desc = fs.make_desc(num_layers=num_layers, num_kv_heads=H, head_dim=D, embed_dim=emb.shape[1],
                        rope_theta=1e6, block_size=bs, num_users=len(ufb) - 1, max_batch=max_batch,
                        max_k=max_k, num_facts=emb.shape[0], num_tokens=T)
    e = torch.from_numpy(np.ascontiguousarray(emb, np.float32)).cuda()
    return fs.fs_create_store(desc, ufb, fact_len, e, k_pre, v), (k_pre, v, e)


def _tables(rng, B, mb, num_blocks):
    """Block tables with distinct blocks across all requests."""
    perm = rng.permutation(num_blocks)[:B * mb]
    return perm.reshape(B, mb).astype(np.int32)


def _plan_parts(plan, B):
    """(header bytes, [B] lengths, [B] starts, token area [B][seg][16])."""
    p = plan.cpu().numpy()
    hdr = PLAN_HEADER + (B * REQ_BYTES + 15) // 16 * 16
    seg = (p.size - hdr) // (TOK_BYTES * B)
    req = p[PLAN_HEADER:PLAN_HEADER + B * REQ_BYTES].view(np.int32).reshape(B, 2)
    tok = p[hdr:hdr + B * seg * TOK_BYTES].reshape(B, seg, TOK_BYTES)
    return p[:PLAN_HEADER], req[:, 0].copy(), req[:, 1].copy(), tok


def _compare(st, B, user, q, k, bt, mb, sp, nb, where=""):
    """fs_retrieve_topk + fs_plan_inject against fs_retrieve_plan.  Returns
    the fused call's (ids, scores, lengths, plan, error bits)."""
    ids_a = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    sc_a = torch.zeros((B, k), dtype=torch.float64, device="cuda")
    nt_a = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    plan_a = fs.new_inject_plan(st, B).fill_(0xAA)
    ids_b = torch.full((B, k), -9, dtype=torch.int32, device="cuda")
    sc_b = torch.ones((B, k), dtype=torch.float64, device="cuda")
    nt_b = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    plan_b = fs.new_inject_plan(st, B).fill_(0x55)
    fs.fs_retrieve_topk(st, B, user, q, k, ids_a, sc_a, nt_a)
    if k > 0:                # (an empty ids tensor is a null pointer, which fs_plan_inject refuses)
        fs.fs_plan_inject(st, B, user, ids_a, k, bt, mb, sp, nb, plan_a)
    err_a = fs.fs_poll_errors(st)
    say(f"retrieve+plan {where}: k={k} B={B}")
    fs.fs_retrieve_plan(st, B, user, q, k, ids_b, bt, mb, sp, nb, plan_b, scores=sc_b, num_tokens=nt_b)
    err_b = fs.fs_poll_errors(st)
    assert err_a == err_b, (where, hex(err_a), hex(err_b))
    assert torch.equal(ids_a, ids_b), where
    assert torch.equal(sc_a.view(torch.int64), sc_b.view(torch.int64)), where
    assert torch.equal(nt_a, nt_b), where
    if k == 0:
        # nothing planned by either call
        assert bool((plan_a == 0xAA).all()) and bool((plan_b == 0x55).all()), where
        return ids_b, sc_b, nt_b, plan_b, err_b
    ha, la, sa, ta = _plan_parts(plan_a, B)
    hb, lb, sb, tb = _plan_parts(plan_b, B)
    assert np.array_equal(ha, hb), where
    assert np.array_equal(la, lb) and np.array_equal(sa, sb), (where, la, lb)
    for b in range(B):
        assert np.array_equal(ta[b, :la[b]], tb[b, :lb[b]]), (where, b)
    return ids_b, sc_b, nt_b, plan_b, err_b


def _tie_store(rng, E=96):
    pool = rng.standard_normal((40, E)).astype(np.float32)
    pool /= np.linalg.norm(pool, axis=1, keepdims=True)
    # users of 3000, 40, 1960 and 500 facts; the last user's rows are all
    # one vector (every score equal)
    F = 5500
    emb = pool[rng.integers(0, 40, F)]
    emb[5000:] = pool[11]
    ufb = np.array([0, 3000, 3040, 5000, 5500], np.int64)
    fl = rng.integers(1, 9, F).astype(np.int32)
    return emb, ufb, fl, pool


@pytest.mark.parametrize("k", [1, 50, 64, 65, 200, 1024])
def test_retrieve_plan_matches_retrieve_then_plan_on_every_select_path(k):
    """Rows drawn from 40 distinct vectors, so exact ties straddle every rank
    and the candidate sets range from the one-wave sort to the radix select;
    one user's scores are all equal.  Block tables of 600 entries, segments
    of up to 8192 tokens (512 blocks): entries inside and past the
    prefetched window."""
    rng = np.random.default_rng(200 + k)
    emb, ufb, fl, pool = _tie_store(rng)
    B, mb, nb = 4, 600, 4096
    st, keep = _small_store(emb, ufb, fl, max_k=1024, max_batch=B)
    users = np.array([0, 1, 2, 3], np.int32)
    q = np.stack([pool[3], rng.standard_normal(emb.shape[1]), pool[7], pool[2]]).astype(np.float32)
    q[1] /= np.linalg.norm(q[1])
    bt = _tables(rng, B, mb, nb)
    sp = rng.integers(0, 700, B).astype(np.int32)
    args = (torch.from_numpy(users).cuda(), torch.from_numpy(q).cuda(), k, torch.from_numpy(bt).cuda(), mb,
            torch.from_numpy(sp).cuda(), nb)
    for rep in range(2):
        err = _compare(st, B, args[0], args[1], k, *args[3:], where=f"ties rep {rep}")[-1]
        assert err == 0
    st.close()
    del keep


@pytest.mark.parametrize("n_big", [6000, 70000], ids=["1024-thread block", "two-phase"])
def test_retrieve_plan_large_users_and_k0(n_big):
    """A user of 6000 facts (selected by the 1024-thread block) or of 70,000
    facts (two-phase selection: chunk tops, then the top of the candidates,
    for every user of that store), beside a 300-fact user and an empty user;
    k from 0 to 1024."""
    rng = np.random.default_rng(41 + n_big)
    E = 16
    ufb = np.array([0, 300, 300, 300 + n_big], np.int64)
    F = int(ufb[-1])
    emb = rng.standard_normal((F, E)).astype(np.float32)
    emb /= np.linalg.norm(emb, axis=1, keepdims=True)
    emb[300 + 4095] = emb[300 + n_big - 7]                # a tie across blocks and chunks
    fl = rng.integers(1, 4, F).astype(np.int32)
    B, mb, nb = 4, 300, 2048
    st, keep = _small_store(emb, ufb, fl, H=1, D=64, max_k=1024, max_batch=B)
    users = np.array([2, 0, 1, 2], np.int32)
    q = np.stack([emb[300 + n_big - 7], emb[17], emb[0], rng.standard_normal(E).astype(np.float32)])
    q = np.ascontiguousarray(q, np.float32)
    bt = _tables(rng, B, mb, nb)
    sp = rng.integers(0, 100, B).astype(np.int32)
    u_t, q_t = torch.from_numpy(users).cuda(), torch.from_numpy(q).cuda()
    bt_t, sp_t = torch.from_numpy(bt).cuda(), torch.from_numpy(sp).cuda()
    for k in (0, 1, 50, 300, 1024):
        err = _compare(st, B, u_t, q_t, k, bt_t, mb, sp_t, nb, where=f"{n_big}-fact user")[-1]
        assert err == 0
    st.close()
    del keep


def test_retrieve_plan_rejections_match_plan_inject():
    """Request 0 is served; request 1 names a user past the store, request 2
    starts at -1, request 3's table holds a block id past the cache, request
    4's table is too short for its segment, request 5 belongs to an empty
    user, request 6's segment would run past the last int32 position.  Bits,
    plan lengths and the injection from the plan must equal fs_plan_inject's;
    only request 0 is written."""
    rng = np.random.default_rng(7)
    E = 32
    emb = rng.standard_normal((200, E)).astype(np.float32)
    ufb = np.array([0, 120, 120, 200], np.int64)        # user 1 is empty
    fl = rng.integers(1, 12, 200).astype(np.int32)
    B, mb, nb, k = 7, 40, 512, 20
    st, keep = _small_store(emb, ufb, fl, H=2, D=64, bs=8, max_k=32, max_batch=B)
    users = np.array([0, 5, 2, 0, 2, 1, 0], np.int32)
    q = np.ascontiguousarray(emb[[3, 4, 150, 9, 170, 5, 11]], np.float32)
    bt = _tables(rng, B, mb, nb)
    sp = np.array([13, 0, -1, 40, 200, 0, np.iinfo(np.int32).max - 3], np.int32)
    bt[3, 40 // 8] = nb                            # its first block: one past the cache
    # request 4: 200 + its segment (>= 20 tokens) needs more than 25 blocks of 8
    mb_short = 25
    bt = np.ascontiguousarray(bt[:, :mb_short])
    u_t, q_t = torch.from_numpy(users).cuda(), torch.from_numpy(q).cuda()
    bt_t, sp_t = torch.from_numpy(bt).cuda(), torch.from_numpy(sp).cuda()
    ids, _, _, plan, err = _compare(st, B, u_t, q_t, k, bt_t, mb_short, sp_t, nb, where="rejections")
    assert err == (fs.FS_ERR_USER | fs.FS_ERR_START_POS | fs.FS_ERR_BLOCK_ID | fs.FS_ERR_BLOCK_SHORT), hex(err)
    _, lens, starts, _ = _plan_parts(plan, B)
    assert lens[0] > 0 and np.all(lens[1:] == 0), lens
    assert np.array_equal(starts, sp)
    # the injection from the fused plan writes request 0 only, as from
    # fs_plan_inject's plan
    caches = [torch.zeros((nb, 8, 2, 64), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ref = [torch.zeros((nb, 8, 2, 64), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    plan_ref = fs.new_inject_plan(st, B)
    fs.fs_plan_inject(st, B, u_t, ids, k, bt_t, mb_short, sp_t, nb, plan_ref)
    fs.fs_poll_errors(st)
    fs.fs_inject_planned(st, fs.FS_ALL_LAYERS, B, k, plan, fs.CacheTable(st, [caches[0]], [caches[1]], nb))
    fs.fs_inject_planned(st, fs.FS_ALL_LAYERS, B, k, plan_ref, fs.CacheTable(st, [ref[0]], [ref[1]], nb))
    torch.cuda.synchronize()
    assert fs.fs_poll_errors(st) == 0
    assert torch.equal(caches[0].view(torch.int16), ref[0].view(torch.int16))
    assert torch.equal(caches[1].view(torch.int16), ref[1].view(torch.int16))
    written = set(np.unique(np.nonzero(caches[1].view(torch.int16).abs().sum(dim=(1, 2, 3)).cpu().numpy())[0]))
    assert written and written <= set(bt[0].tolist()), "a rejected request wrote"
    st.close()
    del keep


def test_retrieve_plan_host_checks():
    rng = np.random.default_rng(8)
    emb = rng.standard_normal((10, 16)).astype(np.float32)
    st, keep = _small_store(emb, np.array([0, 10], np.int64), np.full(10, 4, np.int32), max_k=4, max_batch=2)
    u = torch.zeros(2, dtype=torch.int32, device="cuda")
    q = torch.from_numpy(emb[:2].copy()).cuda()
    ids = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    bt = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    sp = torch.zeros(2, dtype=torch.int32, device="cuda")
    plan = fs.new_inject_plan(st, 2)
    with pytest.raises(fs.FsError) as e:                        # plan too small
        fs.fs_retrieve_plan(st, 2, u, q, 4, ids, bt, 4, sp, 8, torch.empty(64, dtype=torch.uint8, device="cuda"))
    assert e.value.status == fs.FS_E_RANGE
    with pytest.raises(fs.FsError) as e:                        # k past max_k
        fs.fs_retrieve_plan(st, 2, u, q, 5, torch.zeros((2, 5), dtype=torch.int32, device="cuda"), bt, 4, sp, 8,
                            plan)
    assert e.value.status == fs.FS_E_RANGE
    with pytest.raises(fs.FsError) as e:
        fs.fs_retrieve_plan(st, 2, u, q, 4, ids, bt, 4, sp, 0, plan)
    assert e.value.status == fs.FS_E_BLOCKTABLE
    torch.cuda.synchronize()
    assert fs.fs_poll_errors(st) == 0
    st.close()
    del keep
    # a pinned-host store has no planned path
    wl = synth.make_workload("tiny", seed=3)
    ds = build_store(wl, [0], pinned=True)
    req = request_tensors(wl)
    B, k = wl.shape.batch, wl.k
    with pytest.raises(fs.FsError) as e:
        fs.fs_retrieve_plan(ds.store, B, req["user"], req["query"], k,
                            torch.zeros((B, k), dtype=torch.int32, device="cuda"), req["block_table"],
                            wl.block_table.shape[1], req["start_pos"], wl.shape.pool_blocks,
                            torch.zeros(1 << 20, dtype=torch.uint8, device="cuda"))
    assert e.value.status == fs.FS_E_UNSUPPORTED
    ds.close()


def test_retrieve_plan_then_inject_llama_matches_inject_and_oracle():
    """The Llama-3.1-8B shape (2000 facts, k = 50, the one-wave selection) on
    four layers: three request sets, each through fs_retrieve_plan +
    fs_inject_planned and through fs_retrieve_topk + fs_inject, bit for bit;
    the first set also against the oracle."""
    wl = synth.make_workload("llama", seed=1021)
    s = wl.shape
    layers = [0, 1, 2, 3]
    B, k = s.batch, wl.k
    mb = wl.block_table.shape[1]
    say("retrieve+plan llama: building store")
    ds = build_store(wl, layers)
    sets = [request_tensors(wl, queries=r["queries"], start_pos=r["start_pos"], block_table=r["block_table"])
            for r in synth.request_sets(wl, 3, seed=wl.seed + 5)]
    nb = synth.make_caches(wl, layers, "cuda")[0][0].shape[0]
    for i, r in enumerate(sets):
        ids, scores, ntok, plan, err = _compare(ds.store, B, r["user"], r["query"], k, r["block_table"], mb,
                                                r["start_pos"], nb, where=f"llama set {i}")
        assert err == 0
        kc, vc = synth.make_caches(wl, layers, "cuda")
        fs.fs_inject_planned(ds.store, fs.FS_ALL_LAYERS, B, k, plan, fs.CacheTable(ds.store, kc, vc, nb))
        rk, rv = synth.make_caches(wl, layers, "cuda")
        fs.fs_inject(ds.store, fs.FS_ALL_LAYERS, B, r["user"], ids, k, r["block_table"], mb, r["start_pos"],
                     rk, rv, nb)
        torch.cuda.synchronize()
        assert fs.fs_poll_errors(ds.store) == 0
        for l in range(len(layers)):
            assert torch.equal(kc[l].view(torch.int16), rk[l].view(torch.int16)), f"set {i} layer {l} K"
            assert torch.equal(vc[l].view(torch.int16), rv[l].view(torch.int16)), f"set {i} layer {l} V"
        if i == 0:
            import dataclasses
            wl0 = dataclasses.replace(wl, queries=r["query"].cpu().numpy(), start_pos=r["start_pos"].cpu().numpy(),
                                      block_table=r["block_table"].cpu().numpy())
            o = check_retrieval(wl0, ids.cpu().numpy(), scores.cpu().numpy(), ntok.cpu().numpy(), [0], k)
            check_injection(wl0, ds, kc, vc, o, [0, 3])
    ds.close()
