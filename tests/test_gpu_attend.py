"""GPU parity of fs_attend_prefill, the attention read of the injected cache,
and Theorem 3 end to end on the GPU (one layer): fs_inject of the memory and
the query tokens' own K/V, then fs_attend_prefill, equals causal attention
over the same tokens given as one prompt.

Tolerance: the kernel rounds each softmax weight w_i to bf16 before it
multiplies V (relative error at most 2^-9, plus fp32 rounding < 1e-5) and
divides by the fp32 sum of the unrounded weights, so the output differs from
the exact one by sum_i w_i d_i v_i / sum_i w_i with |d_i| <= 2^-9: at most
2^-9 * max_i |v_i| per coordinate.  The test allows 1.1 * 2^-8 * max_i |v_i|
plus 1e-5 (a factor 2 to spare)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from _parity import say
from kv_cache_injection_amd import fs

pytestmark = pytest.mark.gpu

D = 128


def _store(hkv, bs, theta, max_batch=4, facts=None, k_pre=None, v=None, max_k=4):
    """A store whose only role here is the layout (heads, block size, theta)
    and the error word, unless facts and arenas are given."""
    if facts is None:
        facts = np.array([4, 4], np.int32)
        T = int(facts.sum())
        k_pre = [torch.zeros((T, hkv, D), dtype=torch.bfloat16, device="cuda")]
        v = [torch.zeros((T, hkv, D), dtype=torch.bfloat16, device="cuda")]
    T = int(facts.sum())
    F = len(facts)
    emb = torch.nn.functional.normalize(torch.randn((F, 16), device="cuda"), dim=1).float().contiguous()
    desc = fs.make_desc(num_layers=1, num_kv_heads=hkv, head_dim=D, embed_dim=16, rope_theta=theta,
                        block_size=bs, num_users=1, max_batch=max_batch, max_k=max_k,
                        num_facts=F, num_tokens=T)
    return fs.fs_create_store(desc, np.array([0, F], np.int64), facts, emb, k_pre, v)


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _tolerance(vc_bits, table, bs, ctx_begin, q_pos, tq, group):
    """Per (token, query head): 1.1 * 2^-8 * max |v| over the attended
    positions and coordinates of its KV head, plus 1e-5."""
    hkv = vc_bits.shape[2]
    pos = np.arange(ctx_begin, q_pos + tq)
    blk, slot = oracle.placement(pos, table, bs)
    va = np.abs(oracle.bf16_to_f64(vc_bits[blk, slot]))           # [N, Hkv, D]
    tol = np.zeros((tq, hkv * group))
    for j in range(tq):
        m = va[: q_pos + j - ctx_begin + 1].max(axis=(0, 2))     # per KV head
        tol[j] = np.repeat(m, group)
    return 1.1 * 2.0**-8 * tol + 1e-5


@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "split"])
@pytest.mark.parametrize("hq, hkv, bs, tq, c0, q0", [
    (32, 8, 16, 37, 5, 200),       # Llama-3.1-8B heads, ragged query tail
    (28, 4, 16, 16, 0, 45),        # Qwen2.5-7B heads: 7 query heads per KV head
    (8, 8, 1, 1, 0, 0),            # one token attending to itself only
    (4, 1, 64, 20, 100, 300),      # one KV head, large blocks, late context start
    (16, 2, 8, 33, 0, 1000),       # 8 query heads per KV head
    (8, 2, 256, 40, 70, 600),      # blocks longer than a 64-position tile
    (8, 4, 16, 24, 3, 100),        # 2 query heads per KV head: one head per wave, two query sub-tiles
])
def test_attend_matches_oracle(hq, hkv, bs, tq, c0, q0, split):
    theta = 5e5
    rng = np.random.default_rng(hq * 7 + tq)
    B = 2
    ctx = np.array([c0, 0], np.int32)
    qpos = np.array([q0, q0 // 2 + 3], np.int32)
    need = (int(qpos.max()) + tq + bs - 1) // bs
    nb = need * B + 3
    st = _store(hkv, bs, theta)
    g = torch.Generator(device="cuda")
    g.manual_seed(hq + tq)
    kc = torch.randn((nb, bs, hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((nb, bs, hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, tq, hq, D), generator=g, device="cuda").to(torch.bfloat16)
    perm = rng.permutation(nb)
    table = np.stack([perm[:need], perm[need:2 * need]]).astype(np.int32)
    out = torch.full((B, tq, hq, D), -7.0, device="cuda")
    ws = None
    if split:
        nbytes = fs.fs_attend_workspace_size(st, B, tq, hq)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    say(f"attend hq={hq} hkv={hkv} bs={bs} tq={tq} ctx={c0} q_pos={q0} workspace={0 if ws is None else ws.numel()}")
    fs.fs_attend_prefill(st, B, q, kc, vc, torch.from_numpy(table).cuda(), need,
                         torch.from_numpy(ctx).cuda(), torch.from_numpy(qpos).cuda(),
                         1.0 / np.sqrt(D), out, ws)
    assert fs.fs_poll_errors(st) == 0
    got = out.cpu().numpy()
    kb, vb, qb = _bits(kc), _bits(vc), _bits(q)
    for b in range(B):
        ref = oracle.attend_prefill(qb[b], kb, vb, table[b], bs, int(ctx[b]), int(qpos[b]), theta,
                                    1.0 / np.sqrt(D))
        tol = _tolerance(vb, table[b], bs, int(ctx[b]), int(qpos[b]), tq, hq // hkv)
        err = np.abs(got[b] - ref).max(axis=2)
        worst = float((err / tol).max())
        say(f"  request {b}: max |err| {err.max():.3g}, worst err/tol {worst:.3f}")
        assert worst <= 1.0
    st.close()


@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "split"])
def test_attend_device_errors_write_nothing(split):
    st = _store(2, 16, 1e6)
    tq, hq, nb = 4, 4, 8
    kc = torch.zeros((nb, 16, 2, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q = torch.zeros((2, tq, hq, D), dtype=torch.bfloat16, device="cuda")
    table = torch.tensor([[0, 1], [2, 3]], dtype=torch.int32, device="cuda")
    ws = None
    if split:
        ws = torch.full((max(fs.fs_attend_workspace_size(st, 2, tq, hq), 16),), 255, dtype=torch.uint8,
                        device="cuda")                  # stale NaN-filled partials
    cases = [
        ([0, 0], [40, 0], fs.FS_ERR_BLOCK_SHORT),    # positions 40..43 need a third block
        ([5, 0], [3, 0], fs.FS_ERR_START_POS),       # context starts after the queries
        ([-1, 0], [3, 0], fs.FS_ERR_START_POS),
    ]
    for ctx, qp, bit in cases:
        out = torch.full((2, tq, hq, D), -7.0, device="cuda")
        fs.fs_attend_prefill(st, 2, q, kc, vc, table, 2, torch.tensor(ctx, dtype=torch.int32, device="cuda"),
                             torch.tensor(qp, dtype=torch.int32, device="cuda"), 0.1, out, ws)
        assert fs.fs_poll_errors(st) == bit
        o = out.cpu()
        assert torch.all(o[0] == -7.0), "rejected request wrote output"
        assert torch.all(o[1] == 0.0), "valid request not written"   # V is zero
    bad = torch.tensor([[0, 9], [2, 3]], dtype=torch.int32, device="cuda")
    out = torch.full((2, tq, hq, D), -7.0, device="cuda")
    fs.fs_attend_prefill(st, 2, q, kc, vc, bad, 2, torch.tensor([0, 0], dtype=torch.int32, device="cuda"),
                         torch.tensor([14, 0], dtype=torch.int32, device="cuda"), 0.1, out, ws)
    assert fs.fs_poll_errors(st) == fs.FS_ERR_BLOCK_ID
    assert torch.all(out.cpu()[0] == -7.0)
    st.close()


def test_store_refuses_rows_beyond_what_the_kernels_cover():
    """A cache position of 65,536 KV heads x 128 x bf16 (16 MiB) is beyond the
    16 KB token rows the inject kernels are built for and beyond the
    attention's 24-bit offset arithmetic: fs_create_store refuses it, so no
    call ever sees such a row."""
    hkv = 65536
    one = [torch.zeros((1, hkv, D), dtype=torch.bfloat16, device="cuda")]
    with pytest.raises(fs.FsError) as e:
        _store(hkv, 1, 1e4, facts=np.array([1], np.int32), k_pre=one, v=[one[0].clone()])
    assert e.value.status == fs.FS_E_UNSUPPORTED
    assert "16 KB" in str(e.value)


def test_theorem3_inject_then_attend_equals_prompt_attention():
    """One decoder layer with random weights: memory facts and the query
    tokens' own K/V go into the paged cache through fs_inject (Chunked RoPE at
    positions s..), then fs_attend_prefill reads it.  The reference is causal
    attention over the same tokens as one prompt at positions s..: RoPE
    applied to the whole sequence, written here with complex numbers."""
    rng = np.random.default_rng(31)
    hq, hkv, dm, theta, bs, s = 32, 8, 256, 5e5, 16, 13
    lens = np.array([9, 17, 5, 23, 12, 30], np.int32)
    tq = 24
    facts = np.concatenate([lens, [tq]]).astype(np.int32)          # last fact: the query tokens
    T = int(facts.sum())
    x = rng.standard_normal((T, dm))
    wq = rng.standard_normal((dm, hq * D)) / np.sqrt(dm)
    wk = rng.standard_normal((dm, hkv * D)) / np.sqrt(dm)
    wv = rng.standard_normal((dm, hkv * D)) / np.sqrt(dm)
    k_pre = oracle.f64_to_bf16((x @ wk).reshape(T, hkv, D))
    v_raw = oracle.f64_to_bf16((x @ wv).reshape(T, hkv, D))

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)

    st = _store(hkv, bs, theta, max_batch=1, facts=facts, k_pre=[dev(k_pre)], v=[dev(v_raw)],
                max_k=len(facts))
    order = [3, 0, 5, 1, 4, 2]                                     # memory in some rank order
    ids = np.array(order + [len(lens)], np.int32)
    starts = np.concatenate([[0], np.cumsum(facts)[:-1]])
    rows = np.concatenate([np.arange(starts[f], starts[f] + facts[f]) for f in ids])
    L = rows.size
    lm = L - tq
    nb = (s + L + bs - 1) // bs + 5
    table = rng.permutation(nb)[: (s + L + bs - 1) // bs].astype(np.int32)
    kc = torch.zeros((nb, bs, hkv, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    say("theorem 3: inject memory + query K/V")
    fs.fs_inject(st, 0, 1, torch.zeros(1, dtype=torch.int32, device="cuda"),
                 torch.from_numpy(ids[None]).cuda(), len(ids), torch.from_numpy(table[None]).cuda(),
                 len(table), torch.tensor([s], dtype=torch.int32, device="cuda"), [kc], [vc], nb)
    assert fs.fs_poll_errors(st) == 0
    q_pre = oracle.f64_to_bf16((x[rows[lm:]] @ wq).reshape(tq, hq, D))
    out = torch.zeros((1, tq, hq, D), device="cuda")
    say("theorem 3: query-only attention over the injected cache")
    fs.fs_attend_prefill(st, 1, dev(q_pre)[None].contiguous(), kc, vc, torch.from_numpy(table[None]).cuda(),
                         len(table), torch.tensor([s], dtype=torch.int32, device="cuda"),
                         torch.tensor([s + lm], dtype=torch.int32, device="cuda"), 1.0 / np.sqrt(D), out,
                         torch.empty(fs.fs_attend_workspace_size(st, 1, tq, hq) + 16, dtype=torch.uint8,
                                     device="cuda"))
    assert fs.fs_poll_errors(st) == 0
    # the prompt: tokens rows[0..L) at positions s..s+L-1, rotated as a whole
    pos = s + np.arange(L)
    h = D // 2
    w = theta ** (-2.0 * np.arange(h) / D)

    def rot(xb, p):
        xf = oracle.bf16_to_f64(xb)
        z = (xf[..., :h] + 1j * xf[..., h:]) * np.exp(1j * p[:, None, None] * w)
        return oracle.bf16_to_f64(oracle.f64_to_bf16(np.concatenate([z.real, z.imag], axis=-1)))

    kr = rot(k_pre[rows], pos)
    vr = oracle.bf16_to_f64(v_raw[rows])
    qr = rot(q_pre, pos[lm:])
    got = out.cpu().numpy()[0]
    group = hq // hkv
    worst = 0.0
    for hh in range(hq):
        g = hh // group
        sc = (qr[:, hh] @ kr[:, g].T) / np.sqrt(D)
        sc = np.where(pos[None, :] <= pos[lm:, None], sc, -np.inf)
        a = np.exp(sc - sc.max(axis=1, keepdims=True))
        ref = (a / a.sum(axis=1, keepdims=True)) @ vr[:, g]
        for j in range(tq):
            tol = 1.1 * 2.0**-8 * np.abs(vr[: lm + j + 1, g]).max() + 1e-5
            worst = max(worst, float(np.abs(got[j, hh] - ref[j]).max() / tol))
    say(f"theorem 3: worst err/tol {worst:.3f}")
    assert worst <= 1.0
    st.close()
