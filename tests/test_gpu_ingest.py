"""GPU checks of store ingest (the capture half of Context-Window Encoding)
and eviction.

The encoder output is the random-weight decoder's per-layer pre-RoPE K and
raw V of each fact's window (fp64, rounded to bf16), computed on the CPU: it
stands in for the serving model's prefill.  fs_ingest_facts must store
exactly oracle.capture_rows of every window, in the next free slots and rows;
retrieval must find the new facts; fs_inject must place them like any other
fact; eviction must keep ids dense and make the removed fact unreachable."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _decoder import Decoder
from _parity import say
from kv_cache_injection_amd import fs

pytestmark = pytest.mark.gpu

L, H, D, E, BS = 2, 8, 128, 64, 16


def _dev_bits(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _host_bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture()
def setup():
    rng = np.random.default_rng(21)
    cap = [30, 12]
    live = [20, 12]
    lens = np.ones(sum(cap), np.int32)                       # spare slots: placeholders
    lens[:live[0]] = rng.integers(4, 25, live[0])
    lens[cap[0]:cap[0] + live[1]] = rng.integers(4, 25, live[1])
    used = int(lens.sum())
    T = used + 600                                           # free rows for ingest
    k_pre = [torch.randn((T, H, D), device="cuda").to(torch.bfloat16) for _ in range(L)]
    v = [torch.randn((T, H, D), device="cuda").to(torch.bfloat16) for _ in range(L)]
    emb = torch.nn.functional.normalize(torch.randn((sum(cap), E), device="cuda"), dim=1).contiguous()
    ufb = np.array([0, cap[0], sum(cap)], np.int64)
    desc = fs.make_desc(num_layers=L, num_kv_heads=H, head_dim=D, embed_dim=E, rope_theta=5e5,
                        block_size=BS, num_users=2, max_batch=2, max_k=16, num_facts=sum(cap),
                        num_tokens=T)
    st = fs.fs_create_store(desc, ufb, lens, emb, k_pre, v)
    fs.fs_ingest_init(st, live, used)
    # a conversation of 6 turns, each fact encoded with the 2 turns before it
    dec = Decoder(rng, layers=L, dm=32, hq=H, hkv=H, D=D, theta=5e5)
    turn_len = rng.integers(5, 20, 6)
    x = rng.standard_normal((int(turn_len.sum()), 32))
    wk, wv, kb, kl = [[] for _ in range(L)], [[] for _ in range(L)], [], []
    row = 0
    for j in range(6):
        a, b, keep_b, keep_l = oracle.cwe_window(turn_len, j, 2)
        _, kv = dec.prefill(x[a:b], np.arange(b - a))
        for l in range(L):
            wk[l].append(oracle.f64_to_bf16(kv[l][0]))
            wv[l].append(oracle.f64_to_bf16(kv[l][1]))
        kb.append(row + keep_b)
        kl.append(keep_l)
        row += b - a
    win_k = [np.concatenate(wk[l]) for l in range(L)]
    win_v = [np.concatenate(wv[l]) for l in range(L)]
    new_emb = rng.standard_normal((6, E)).astype(np.float32)
    new_emb /= np.linalg.norm(new_emb, axis=1, keepdims=True)
    yield dict(st=st, k_pre=k_pre, v=v, emb=emb, used=used, win_k=win_k, win_v=win_v,
               kb=np.array(kb), kl=np.array(kl), new_emb=new_emb, lens=lens, cap=cap)
    st.close()


def _retrieve_top1(st, user, q):
    ids = torch.empty((1, 1), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 1), dtype=torch.float64, device="cuda")
    fs.fs_retrieve_topk(st, 1, torch.tensor([user], dtype=torch.int32, device="cuda"),
                        torch.from_numpy(q[None].astype(np.float32)).cuda(), 1, ids, sc, None)
    assert fs.fs_poll_errors(st) == 0
    return int(ids.item()), float(sc.item())


def _inject_and_check(st, ids, k_rows, v_rows, start=7):
    """Inject one request with `ids` (user 0) and compare the cache with the
    oracle's rows for the given per-fact K/V bits (lists over ids)."""
    kbits = np.concatenate(k_rows, axis=1)       # [L, rows, H, D]
    vbits = np.concatenate(v_rows, axis=1)
    n = kbits.shape[1]
    nb = (start + n + BS - 1) // BS + 3
    table = np.random.default_rng(3).permutation(nb)[: (start + n + BS - 1) // BS].astype(np.int32)
    kc = [torch.zeros((nb, BS, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    vc = [torch.zeros_like(kc[0]) for _ in range(L)]
    fs.fs_inject(st, fs.FS_ALL_LAYERS, 1, torch.zeros(1, dtype=torch.int32, device="cuda"),
                 torch.tensor([ids], dtype=torch.int32, device="cuda"), len(ids),
                 torch.from_numpy(table[None]).cuda(), len(table),
                 torch.tensor([start], dtype=torch.int32, device="cuda"), kc, vc, nb)
    flags = fs.fs_poll_errors(st)
    if flags:
        return flags
    pos = start + np.arange(n)
    blk, slot = oracle.placement(pos, table, BS)
    for l in range(L):
        ek, ev = oracle.expected_rows(kbits[l], vbits[l], pos, 5e5)
        assert np.array_equal(_host_bits(kc[l])[blk, slot], ek), f"layer {l} K"
        assert np.array_equal(_host_bits(vc[l])[blk, slot], ev), f"layer {l} V"
    return 0


def test_ingest_then_retrieve_and_inject(setup):
    s = setup
    st = s["st"]
    say("ingest: 6 facts for user 0")
    ids = fs.fs_ingest_facts(st, [0] * 6, [_dev_bits(w) for w in s["win_k"]], [_dev_bits(w) for w in s["win_v"]],
                             s["kb"], s["kl"], torch.from_numpy(s["new_emb"]).cuda())
    assert list(ids) == list(range(20, 26))
    live, rows = fs.fs_store_live(st, 0)
    assert live == 26 and rows == s["used"] + int(s["kl"].sum())
    # the arenas hold exactly the captured rows, in order
    r = s["used"]
    for i in range(6):
        for l in range(L):
            want_k = oracle.capture_rows(s["win_k"][l], s["kb"][i], s["kl"][i])
            want_v = oracle.capture_rows(s["win_v"][l], s["kb"][i], s["kl"][i])
            assert np.array_equal(_host_bits(s["k_pre"][l][r:r + s["kl"][i]]), want_k)
            assert np.array_equal(_host_bits(s["v"][l][r:r + s["kl"][i]]), want_v)
        r += s["kl"][i]
    # the embeddings are in place: each new fact is its own best match
    for i in range(6):
        got, score = _retrieve_top1(st, 0, s["new_emb"][i])
        assert got == 20 + i and abs(score - 1.0) < 1e-6
    # injection composes them like any fact
    k_rows = [[oracle.capture_rows(s["win_k"][l], s["kb"][i], s["kl"][i]) for l in range(L)] for i in (4, 1, 5)]
    v_rows = [[oracle.capture_rows(s["win_v"][l], s["kb"][i], s["kl"][i]) for l in range(L)] for i in (4, 1, 5)]
    kb = [np.stack([k_rows[j][l] for l in range(L)]) for j in range(3)]
    vb = [np.stack([v_rows[j][l] for l in range(L)]) for j in range(3)]
    assert _inject_and_check(st, [24, 21, 25], kb, vb) == 0


def test_evict_keeps_ids_dense(setup):
    s = setup
    st = s["st"]
    fs.fs_ingest_facts(st, [0] * 6, [_dev_bits(w) for w in s["win_k"]], [_dev_bits(w) for w in s["win_v"]],
                       s["kb"], s["kl"], torch.from_numpy(s["new_emb"]).cuda())
    say("evict: fact 22")
    moved = fs.fs_evict_fact(st, 22)
    assert moved == 25
    assert fs.fs_store_live(st, 0)[0] == 25
    # the former fact 25 answers as 22; the evicted fact is gone
    got, _ = _retrieve_top1(st, 0, s["new_emb"][5])
    assert got == 22
    got, score = _retrieve_top1(st, 0, s["new_emb"][2])
    assert got != 22 and score < 1.0 - 1e-6
    # id 22 now injects the moved fact's rows; id 25 is no longer live
    kb = [np.stack([oracle.capture_rows(s["win_k"][l], s["kb"][5], s["kl"][5]) for l in range(L)])]
    vb = [np.stack([oracle.capture_rows(s["win_v"][l], s["kb"][5], s["kl"][5]) for l in range(L)])]
    assert _inject_and_check(st, [22], kb, vb) == 0
    assert _inject_and_check(st, [25], kb, vb) == fs.FS_ERR_FACT_ID
    # evicting the last live fact moves nothing
    assert fs.fs_evict_fact(st, 24) == -1
    with pytest.raises(fs.FsError):
        fs.fs_evict_fact(st, 24)                     # no longer live


def test_ingest_is_all_or_nothing(setup):
    s = setup
    st = s["st"]
    wk = [_dev_bits(w) for w in s["win_k"]]
    wv = [_dev_bits(w) for w in s["win_v"]]
    emb = torch.from_numpy(s["new_emb"]).cuda()
    before = fs.fs_store_live(st, 0), fs.fs_store_live(st, 1)
    # user 1 is full: the whole batch is refused
    with pytest.raises(fs.FsError):
        fs.fs_ingest_facts(st, [0, 0, 1, 0, 0, 0], wk, wv, s["kb"], s["kl"], emb)
    # a fact longer than the store's longest
    kl = s["kl"].copy()
    kl[0] = int(s["lens"].max()) + 1
    with pytest.raises(fs.FsError):
        fs.fs_ingest_facts(st, [0] * 6, wk, wv, s["kb"], kl, emb)
    assert (fs.fs_store_live(st, 0), fs.fs_store_live(st, 1)) == before
    # user 0 has 10 free slots: 6, then 4 more fit, then nothing
    fs.fs_ingest_facts(st, [0] * 6, wk, wv, s["kb"], s["kl"], emb)
    fs.fs_ingest_facts(st, [0] * 4, wk, wv, s["kb"][:4], s["kl"][:4], emb[:4].contiguous())
    assert fs.fs_store_live(st, 0)[0] == 30
    with pytest.raises(fs.FsError):
        fs.fs_ingest_facts(st, [0], wk, wv, s["kb"][:1], s["kl"][:1], emb[:1].contiguous())
