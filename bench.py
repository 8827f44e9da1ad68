"""Throughput of the KV-injection hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config llama] [--k 50]

One step = one pass of the whole hot path over one batch of requests:
fs_retrieve_plan (embedding scores, then a top-k whose block also composes
and validates the segment and writes the inject plan) followed by one
all-layer fs_inject_planned (gather -> Chunked RoPE -> paged scatter into
every layer's cache, streaming from that plan).  Inputs are resident in HBM
before the timed region; every step uses a different (query, start
position, block table) set, cycling through --sets pre-drawn sets, so the
selected facts change from step to step.

Steps are issued as a serving loop with two lanes would: step i runs its
retrieval and then its injection on stream i % 2, so step i+1's retrieval
(latency-bound, a few MB) and the start of its injection overlap step i's
injection (bandwidth-bound).  Retrievals share the store's scratch, so each
waits on an event after the previous one; the lanes inject into separate
cache pools.  two_calls times the same loop through fs_retrieve_topk and the
fused fs_inject (plan kernel + row kernel); both loops run in the warm-up.
request_latency_us.in_order runs the requests on one stream,
strictly one after the other, as a single request is served:
fs_retrieve_plan (scores, then top-k whose block also writes the inject
plan) and fs_inject_planned (the row kernel); in_order_two_calls does the
same with fs_retrieve_topk then fs_inject (plan kernel + row kernel).

Prints ONE JSON line:
  value       whole-step algorithmic HBM bytes / step time (GB/s)
  injected_payload_GBps  the K and V bytes landed in the caches / step time
  roofline    the row-streaming inject kernel (fs_inject_planned launches one
              and nothing else): its algorithmic bytes per launch over its
              average launch time (HIP events on the launch stream around the
              steps' launches issued back to back), against 8 TB/s; "cold"
              repeats it with each launch alone after a 1 GiB write that
              evicts the MALL and L2 (median, p10, p90)
  kernels_ms  average launch times of the retrieval, the fused inject (plan
              kernel + row kernel), the plan kernel alone, the row kernel
              alone (fs_plan_inject, fs_inject_planned) and the planning
              retrieval (fs_retrieve_plan), each issued back to back
  request_latency_us  one request at a time, in order: the whole step, and
              its parts from kernels_ms
  inject_cold each fused inject alone after the same 1 GiB write
  cpu_baseline  the CPU oracle on a bounded sample of the same workload, on
              every core of the process's CPU share, and beside it on one
              thread

Algorithmic bytes: inject = 8 * L * layers * heads * head_dim (K and V, bf16,
read once and written once) per request of segment length L; retrieval =
4 * N_user * embed_dim (one fp32 scan of the user's embeddings) per request.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=300)
    p.add_argument("--warmup", type=int, default=200)
    p.add_argument("--config", default="llama",
                   choices=["tiny", "llama", "qwen", "concurrent", "large"])
    p.add_argument("--k", type=int, default=None)
    p.add_argument("--layers", type=int, default=None,
                   help="resident layers (default: all; the concurrent store needs fewer)")
    p.add_argument("--sets", type=int, default=50)
    p.add_argument("--cpu-requests", type=int, default=16,
                   help="requests of the oracle's bounded CPU sample (0 = skip)")
    p.add_argument("--copy-probe", action="store_true",
                   help="also time a plain device copy of one inject's bytes (the copy ceiling at this "
                        "size; the known-size launches the HBM counters are calibrated on)")
    p.add_argument("--overlap", action="store_true",
                   help="layer-pipelined injection on a side stream under a synthetic per-layer forward "
                        "(two bf16 GEMMs per layer), for several layer-chunk plans: how much of the "
                        "injection stays exposed")
    p.add_argument("--attend", action="store_true",
                   help="time fs_attend_prefill: query tokens over one layer's injected cache")
    p.add_argument("--tq", type=int, default=128, help="query tokens per request (--attend)")
    p.add_argument("--batch", type=int, default=1, help="requests (--attend)")
    p.add_argument("--ivf", action="store_true",
                   help="approximate retrieval on a 1M-fact clustered store: build time, latency and "
                        "recall@k of the inverted-file probe against the flat scan")
    p.add_argument("--facts", type=int, default=1_000_000, help="facts of the --ivf store")
    p.add_argument("--ingest", action="store_true",
                   help="store ingest (Context-Window Encoding capture) on the Llama-8B shape: facts/s "
                        "and captured GB/s")
    p.add_argument("--pinned", action="store_true",
                   help="K/V arenas in pinned host memory: time the per-layer fetch -> inject "
                        "pipeline against a plain host-to-device copy (the host link is the bound)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "the library has no multi-GPU path: requests shard by user with no exchange, one process per GPU", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from kv_cache_injection_amd import fs, synth
    from kv_cache_injection_amd.workload import build_store, request_tensors

    torch.cuda.set_device(0)
    if args.pinned:
        return bench_pinned(args)
    if args.overlap:
        return bench_overlap(args)
    if args.attend:
        return bench_attend(args)
    if args.ivf:
        return bench_ivf(args)
    if args.ingest:
        return bench_ingest(args)
    wl = synth.make_workload(args.config, k=args.k)
    s = wl.shape
    nl = args.layers or s.num_layers
    layers = list(range(nl))
    B, k = s.batch, wl.k
    print(f"[bench] {s.name}: building store ({nl} layers, {wl.num_tokens} tokens)", file=sys.stderr, flush=True)
    ds = build_store(wl, layers)
    kc, vc = synth.make_caches(wl, layers, "cuda")
    nb = kc[0].shape[0]
    caches = fs.CacheTable(ds.store, kc, vc, nb)
    base = request_tensors(wl)
    sets = []
    for r in synth.request_sets(wl, args.sets, seed=wl.seed + 1):
        t = request_tensors(wl, queries=r["queries"], start_pos=r["start_pos"],
                            block_table=r["block_table"])
        sets.append(t)
    mb = wl.block_table.shape[1]
    user = base["user"]
    total = args.warmup + args.steps
    ids = torch.empty((total, B, k), dtype=torch.int32, device="cuda")   # one slot per step
    ntok = torch.zeros((total, B), dtype=torch.int32, device="cuda")
    plans = [fs.new_inject_plan(ds.store, B) for _ in range(total)]     # one plan per step
    e0, e1, e2, e3, e4, e5 = (torch.cuda.Event(enable_timing=True) for _ in range(6))

    # Pipelined steps on two lanes (streams at the default priority): step i
    # retrieves and injects on lane i % 2, so each inject follows its own
    # retrieval in stream order, and the other lane's retrieval and inject run
    # beside it.  Retrievals share the store's score scratch, so retrieval i
    # waits for retrieval i - 1 (an event); the two lanes write separate cache
    # pools, as two different requests would.  ids have a slot per step.
    # (Planning each step into its own plan, fs_plan_inject, and injecting
    # from it gives the same step time here: the two lanes already overlap
    # each inject's planning with the other lane's work.  Region 2 times the
    # planned kernels too.)
    kc2, vc2 = synth.make_caches(wl, layers, "cuda")
    caches2 = fs.CacheTable(ds.store, kc2, vc2, nb)
    lanes = (torch.cuda.Stream(), torch.cuda.Stream())
    ret_done = [torch.cuda.Event() for _ in range(total)]

    # arguments marshalled once per step slot; the timed loops only issue
    # the foreign calls
    def prep(stream_ret, stream_inj, cache_of=lambda i: caches):
        rc = [fs.prepare_retrieve_topk(ds.store, B, user, sets[i % len(sets)]["query"], k, ids[i],
                                       None, ntok[i], stream=stream_ret(i)) for i in range(total)]
        ic = [fs.prepare_inject(ds.store, fs.FS_ALL_LAYERS, B, user, ids[i], k,
                                sets[i % len(sets)]["block_table"], mb, sets[i % len(sets)]["start_pos"],
                                cache_of(i), stream=stream_inj(i)) for i in range(total)]
        pc = [fs.prepare_plan_inject(ds.store, B, user, ids[i], k, sets[i % len(sets)]["block_table"], mb,
                                     sets[i % len(sets)]["start_pos"], nb, plans[i], stream=stream_inj(i))
              for i in range(total)]
        jc = [fs.prepare_inject_planned(ds.store, fs.FS_ALL_LAYERS, B, k, plans[i], cache_of(i),
                                        stream=stream_inj(i)) for i in range(total)]
        # retrieval that also writes the step's plan
        rp = [fs.prepare_retrieve_plan(ds.store, B, user, sets[i % len(sets)]["query"], k, ids[i],
                                       sets[i % len(sets)]["block_table"], mb, sets[i % len(sets)]["start_pos"],
                                       nb, plans[i], num_tokens=ntok[i], stream=stream_ret(i)) for i in range(total)]
        return rc, ic, pc, jc, rp
    ret_p, inj_p, _, injp_p, rp_p = prep(lambda i: lanes[i % 2], lambda i: lanes[i % 2],
                                         lambda i: caches if i % 2 == 0 else caches2)   # two lanes
    cur = torch.cuda.current_stream()
    ret_s, inj_s, plan_s, injp_s, rp_s = prep(lambda i: cur, lambda i: cur)            # one stream, in order

    def step_pipelined(i):
        # the planning retrieval writes the step's plan, and the row kernel
        # streams from it
        lane = lanes[i % 2]
        if i > 0:
            lane.wait_event(ret_done[i - 1])
        rp_p[i]()
        ret_done[i].record(lane)
        injp_p[i]()

    def step_pipelined_two_calls(i):
        # the same lanes with fs_retrieve_topk and the fused fs_inject (plan
        # kernel + row kernel)
        lane = lanes[i % 2]
        if i > 0:
            lane.wait_event(ret_done[i - 1])
        ret_p[i]()
        ret_done[i].record(lane)
        inj_p[i]()

    def step_serial(i):
        ret_s[i]()
        inj_s[i]()

    print(f"[bench] warmup {args.warmup}, steps {args.steps}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step_pipelined_two_calls(i)
        step_pipelined(i)
    torch.cuda.synchronize()
    # timed region 1: the whole hot path for every step, each lane's
    # retrieval and inject overlapping the other lane's (no timing events)
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step_pipelined(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flags = fs.fs_poll_errors(ds.store)
    if flags:
        raise RuntimeError(f"device error bits 0x{flags:x}")
    L = ntok.cpu().numpy().astype(np.int64)[args.warmup:]          # [steps, B]
    # timed region 1c (beside value): the same two-lane loop through the
    # two-call path
    w0 = time.perf_counter()
    for i in range(args.warmup, total):
        step_pipelined_two_calls(i)
    torch.cuda.synchronize()
    w1 = time.perf_counter()
    if not np.array_equal(ntok.cpu().numpy().astype(np.int64)[args.warmup:], L):
        raise RuntimeError("the two pipelined loops selected different segments")

    # every kernel regions 1b and 2 time has run before them (the pipelined
    # warm-up ran each kind on the lanes); they run here once more on the
    # timing stream (a first launch pays one-time costs)
    for i in range(min(total, max(args.warmup, 5))):
        ret_s[i]()
        inj_s[i]()
        plan_s[i]()
        injp_s[i]()
        rp_s[i]()
        injp_s[i]()
    torch.cuda.synchronize()

    # timed region 1b: the same steps on one stream, strictly in order, as a
    # single request is served: retrieval with planning, then the row kernel
    # from that plan; then retrieval, then the fused inject
    torch.cuda.synchronize()
    u0 = time.perf_counter()
    for i in range(args.warmup, total):
        rp_s[i]()
        injp_s[i]()
    torch.cuda.synchronize()
    u1 = time.perf_counter()
    for i in range(args.warmup, total):
        step_serial(i)
    torch.cuda.synchronize()
    u2 = time.perf_counter()

    # timed region 2: per-kernel average durations for the roofline, from
    # HIP events on the launch stream: the steps' retrievals back to back
    # between two events, then their fused injects, their plans and their
    # injects from the plans, each kind back to back between two more (each
    # reads what its step's retrieval or plan wrote); the average is the
    # span over the number of launches
    e0.record()
    for i in range(args.warmup, total):
        ret_s[i]()
    e1.record()
    for i in range(args.warmup, total):
        inj_s[i]()
    e2.record()
    for i in range(args.warmup, total):
        plan_s[i]()
    e3.record()
    for i in range(args.warmup, total):
        injp_s[i]()
    e4.record()
    for i in range(args.warmup, total):
        rp_s[i]()
    e5.record()
    torch.cuda.synchronize()

    # timed region 3 (reported beside, never value): each row-kernel launch
    # (from the plan region 2 wrote) and each fused inject alone after a
    # 1 GiB write that evicts the MALL and L2, between its own HIP events
    # (an event pair adds ~2 us to one launch), for median and p10/p90
    n_cold = min(args.steps, 50)
    flush = torch.empty(1 << 28, dtype=torch.int32, device="cuda")

    def timed_cold(calls):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
        for j, (ca, cb) in enumerate(ev):
            flush.fill_(j)
            ca.record()
            calls[args.warmup + j]()
            cb.record()
        torch.cuda.synchronize()
        return np.array([ca.elapsed_time(cb) for ca, cb in ev])
    row_cold_ms = timed_cold(injp_s)
    cold_ms = timed_cold(inj_s)
    del flush

    wall = t1 - t0
    row_bytes = 2 * s.num_kv_heads * s.head_dim                      # one token, one layer, K or V
    inject_bytes = 4 * row_bytes * L.sum(axis=1) * nl                # K,V read + write
    n_user = np.diff(wl.user_fact_begin)[wl.users]
    scan_bytes = 4 * int(n_user.sum()) * s.embed_dim
    step_bytes = inject_bytes + scan_bytes
    inj_ms = np.full(args.steps, e1.elapsed_time(e2) / args.steps)
    plan_ms = e2.elapsed_time(e3) / args.steps
    planned_ms = e3.elapsed_time(e4) / args.steps
    ret_ms = np.full(args.steps, e0.elapsed_time(e1) / args.steps)
    ret_plan_ms = e4.elapsed_time(e5) / args.steps
    achieved = float(inject_bytes.sum() / (planned_ms * args.steps * 1e-3) / 1e9)
    row_cold_gbs = inject_bytes[:n_cold] / (row_cold_ms * 1e-3) / 1e9
    vpr = s.num_kv_heads * s.head_dim // 8
    lg = (vpr - 1).bit_length()
    kname = f"fs_{'row' if lg >= 6 else 'short'}_kernel<{s.head_dim}, {lg}>"
    in_order_us = (u1 - u0) / args.steps * 1e6
    in_order_two_us = (u2 - u1) / args.steps * 1e6
    value = float(step_bytes.sum() / wall / 1e9)
    ms_per_step = wall / args.steps * 1e3
    wall_two = w1 - w0
    traffic = recorded_traffic(args.config, nl)

    copy = None
    if args.copy_probe:
        # the copy ceiling at this size: a plain device copy (torch's copy
        # kernel) of as many bytes as one inject reads and writes, issued back
        # to back between two events like region 2; also the known-size
        # launches the HBM counters are calibrated on
        n16 = int(inject_bytes.mean()) // 4                          # int16 elements each way
        a = torch.empty(n16, dtype=torch.int16, device="cuda")
        bb = torch.empty_like(a)
        a.fill_(1)
        bb.copy_(a)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(args.steps):
            bb.copy_(a)
        c1.record()
        torch.cuda.synchronize()
        us = c0.elapsed_time(c1) * 1e3 / args.steps
        copy = {"bytes_per_copy": 4 * n16, "us_avg": round(us, 2),
                "GBps": round(4 * n16 / (us * 1e-6) / 1e9, 1),
                "frac": round(4 * n16 / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "note": "torch copy_ of one inject's bytes (half read, half written), back to back"}
        del a, bb

    cpu = None
    if args.cpu_requests > 0:
        cpu = cpu_baseline(wl, ds, layers, args.cpu_requests)

    out = {
        "metric": "KV-injection GB/s & requests/s at k=50, Llama-8B shape; % of HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "ms_per_step_in_order": round(in_order_us * 1e-3, 5),
        "two_calls": {"ms_per_step": round(wall_two / args.steps * 1e3, 5),
                      "value": round(float(step_bytes.sum() / wall_two / 1e9), 2),
                      "note": "the same two-lane loop through fs_retrieve_topk and the fused fs_inject "
                              "(plan kernel + row kernel)"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic",
        "requests_per_s": round(B * args.steps / wall, 1),
        "injected_payload_GBps": round(float(inject_bytes.sum() / 2 / wall / 1e9), 2),
        "hbm_frac_of_peak": round(value / HBM_PEAK_GBS, 4),
        "config": {
            "workload": f"{s.name}: {nl} layers x {s.num_kv_heads} KV heads x head_dim {s.head_dim}, "
                        f"theta {s.rope_theta:g}; {s.num_users} user(s) x {s.facts_per_user} facts "
                        f"of U[{s.len_lo},{s.len_hi}] tokens, {s.embed_dim}-d embeddings; "
                        f"{B} request(s) per step, k={k}, block_size {s.block_size}",
            "batch": B, "k": k, "layers": nl, "mean_segment_tokens": round(float(L.mean()), 1),
            "request_sets": args.sets,
        },
        "kernels_ms": {"retrieve_avg": round(float(ret_ms.mean()), 5),
                       "inject_avg": round(float(inj_ms.mean()), 5),
                       "plan_avg": round(float(plan_ms), 5),
                       "inject_from_plan_avg": round(float(planned_ms), 5),
                       "retrieve_plan_avg": round(float(ret_plan_ms), 5)},
        "request_latency_us": {
            "in_order": round(in_order_us, 2),
            "in_order_two_calls": round(in_order_two_us, 2),
            "retrieve": round(float(ret_ms.mean()) * 1e3, 2),
            "retrieve_plan": round(float(ret_plan_ms) * 1e3, 2),
            "inject": round(float(inj_ms.mean()) * 1e3, 2),
            "inject_from_plan": round(float(planned_ms) * 1e3, 2),
            "in_order_over_inject": round(in_order_us / (float(inj_ms.mean()) * 1e3), 3),
            "in_order_over_inject_from_plan": round(in_order_us / (float(planned_ms) * 1e3), 3),
            "in_order_two_calls_over_inject": round(in_order_two_us / (float(inj_ms.mean()) * 1e3), 3),
            "note": "one request at a time on one stream.  in_order: fs_retrieve_plan (scores, then a "
                    "top-k that also writes the inject plan), then fs_inject_planned (row kernel).  "
                    "in_order_two_calls: fs_retrieve_topk (scores + top-k), then fs_inject (plan kernel + "
                    "row kernel).  The other figures are back-to-back averages of one call kind"},
        "inject_cold": {
            "note": "each inject alone after a 1 GiB write that evicts the MALL and L2, own HIP events",
            "launches": n_cold,
            "ms_median": round(float(np.median(cold_ms)), 5),
            "ms_p10": round(float(np.percentile(cold_ms, 10)), 5),
            "ms_p90": round(float(np.percentile(cold_ms, 90)), 5),
            "GBps_median": round(float(np.median(inject_bytes[:n_cold] / (cold_ms * 1e-3) / 1e9)), 1)},
        "roofline": {"bound": "hbm", "kernel": kname,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": float(inject_bytes.mean()), "traffic": traffic,
                     "cold": {"launches": n_cold,
                              "ms_median": round(float(np.median(row_cold_ms)), 5),
                              "ms_p10": round(float(np.percentile(row_cold_ms, 10)), 5),
                              "ms_p90": round(float(np.percentile(row_cold_ms, 90)), 5),
                              "achieved_median": round(float(np.median(row_cold_gbs)), 1),
                              "frac_median": round(float(np.median(row_cold_gbs)) / HBM_PEAK_GBS, 4)}},
        "cpu_baseline": cpu,
    }
    if copy is not None:
        out["copy_probe"] = copy
    print(json.dumps(out), flush=True)
    ds.close()


def bench_ingest(args):
    """fs_ingest_facts on the Llama-3.1-8B shape (32 layers, 8 KV heads, head
    dim 128): 2,048 facts of U[12,48] tokens, each with a window of the 2
    turns before it (turns of U[12,48] tokens), in calls of 64 facts.  The
    window arrays stand in for the encoder's per-layer output (random bf16;
    their content does not matter to the copy).  Bytes: each kept row is read
    from the window and written to the arena, K and V, every layer:
    8 * rows * layers * H * D bytes per fact, plus its embedding read and
    written (8 * E)."""
    import numpy as np
    import torch

    from kv_cache_injection_amd import fs

    L, H, D, E, slots, max_len, per_call, w = 32, 8, 128, 768, 2048, 48, 64, 2
    T = slots * max_len
    print(f"[bench] ingest: arenas of {T} rows x {L} layers", file=sys.stderr, flush=True)
    k_pre = [torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    v = [torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    emb = torch.zeros((slots, E), device="cuda")
    desc = fs.make_desc(num_layers=L, num_kv_heads=H, head_dim=D, embed_dim=E, rope_theta=5e5,
                        block_size=16, num_users=1, max_batch=1, max_k=50, num_facts=slots, num_tokens=T)
    st = fs.fs_create_store(desc, np.array([0, slots], np.int64), np.full(slots, max_len, np.int32), emb,
                            k_pre, v)
    rng = np.random.default_rng(9)
    turns = rng.integers(12, max_len + 1, (slots // per_call, per_call, w + 1))
    wrows = int(turns.sum(axis=2).max()) * per_call
    win_k = [torch.randn((wrows, H, D), device="cuda").to(torch.bfloat16) for _ in range(L)]
    win_v = [torch.randn((wrows, H, D), device="cuda").to(torch.bfloat16) for _ in range(L)]
    new_emb = torch.nn.functional.normalize(torch.randn((per_call, E), device="cuda"), dim=1).contiguous()
    calls = []
    for c in range(slots // per_call):
        lens = turns[c]                                   # [facts, w + 1]: w context turns then the fact
        start = np.concatenate([[0], np.cumsum(lens.sum(axis=1))[:-1]])
        calls.append((start + lens[:, :w].sum(axis=1), lens[:, w].astype(np.int32)))

    def run():
        fs.fs_ingest_init(st, [0], 0)
        kept = 0
        for kb, kl in calls:
            fs.fs_ingest_facts(st, [0] * per_call, win_k, win_v, kb, kl, new_emb)
            kept += int(kl.sum())
        return kept

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = max(1, min(args.steps, 3))
    for _ in range(reps):
        kept = run()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    gb = (4.0 * kept * L * H * D * 2 + 8.0 * slots * E) / dt / 1e9      # bf16: 2 bytes
    out = {
        "metric": "store ingest (Context-Window Encoding capture): facts/s and GB/s moved",
        "value": round(slots / dt, 1), "unit": "facts/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 bytes", "data": "synthetic",
        "GBps": round(gb, 1), "rows_kept": kept, "calls": len(calls),
        "config": {"workload": f"Llama-3.1-8B KV shape ({L} layers x {H} x {D}); {slots} facts of "
                               f"U[12,{max_len}] tokens, window {w} turns, {per_call} facts per call",
                   "facts": slots, "window_turns": w},
    }
    print(json.dumps(out), flush=True)
    st.close()


def bench_ivf(args):
    """Inverted-file index on one user with --facts facts (768-d clustered unit
    embeddings around 256 topics, spread 1.0, one token each, one layer of 1 KV head:
    retrieval only).  Reports the build time, and per batch size and nprobe
    the probe latency next to the flat scan's, and recall@k: the share of
    the flat scan's top-k ids the probe returns."""
    import numpy as np
    import torch

    from kv_cache_injection_amd import fs, synth

    n, dim, topics, spread, k = args.facts, 768, 256, 1.0, args.k or 50
    nlist = 1024
    print(f"[bench] ivf: drawing {n} embeddings", file=sys.stderr, flush=True)
    emb, _ = synth.clustered_embeddings(n, dim, topics, spread, seed=4242)
    qry, _ = synth.clustered_embeddings(64, dim, topics, spread, seed=4243)
    T = n
    k_pre = [torch.zeros((T, 1, 128), dtype=torch.bfloat16, device="cuda")]
    v = [torch.zeros((T, 1, 128), dtype=torch.bfloat16, device="cuda")]
    desc = fs.make_desc(num_layers=1, num_kv_heads=1, head_dim=128, embed_dim=dim, rope_theta=1e6,
                        block_size=16, num_users=1, max_batch=64, max_k=max(k, 64),
                        num_facts=n, num_tokens=T)
    e = torch.from_numpy(emb).cuda()
    del emb
    st = fs.fs_create_store(desc, np.array([0, n], np.int64), np.ones(n, np.int32), e, k_pre, v)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ix = fs.fs_ivf_build(st, 0, nlist, 8, 128)
    build_s = time.perf_counter() - t0
    info = fs.fs_ivf_arrays(ix)
    print(f"[bench] ivf: built {nlist} lists in {build_s:.2f} s (longest {info['max_list']})",
          file=sys.stderr, flush=True)
    q = torch.from_numpy(qry).cuda()
    zeros = torch.zeros(64, dtype=torch.int32, device="cuda")

    def timed(fn, reps=30):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a0, a1 in evs:
            a0.record()
            fn()
            a1.record()
        torch.cuda.synchronize()
        return float(np.median([a0.elapsed_time(a1) for a0, a1 in evs])) * 1e3

    points = []
    for B in (1, 16):
        qb = q[:B].contiguous()
        flat_ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
        t_flat = timed(lambda: fs.fs_retrieve_topk(st, B, zeros[:B], qb, k, flat_ids, None, None))
        ref = flat_ids.cpu().numpy()
        for nprobe in (8, 16, 32, 64, 128):
            ids = torch.empty((B, k), dtype=torch.int32, device="cuda")
            t = timed(lambda: fs.fs_ivf_retrieve_topk(st, ix, B, qb, nprobe, k, ids))
            got = ids.cpu().numpy()
            rec = float(np.mean([len(set(got[b]) & set(ref[b])) / k for b in range(B)]))
            points.append({"batch": B, "nprobe": nprobe, "probe_us": round(t, 1), "flat_us": round(t_flat, 1),
                           "speedup": round(t_flat / t, 2), f"recall@{k}": round(rec, 4)})
            print(f"[bench] ivf B={B} nprobe={nprobe}: {t:.1f} us vs flat {t_flat:.1f} us, "
                  f"recall {rec:.4f}", file=sys.stderr, flush=True)
    if fs.fs_poll_errors(st):
        raise RuntimeError("device error bits set")
    # recall is averaged over the 16-query batch; the single-query points
    # carry one query's recall only
    best = max((p for p in points if p["batch"] == 16 and p[f"recall@{k}"] >= 0.9),
               key=lambda p: p["speedup"], default=points[-1])
    out = {
        "metric": f"approximate retrieval: flat-scan latency / probe latency at mean recall@{k} >= 0.9 (16 queries)",
        "value": best["speedup"], "unit": "x (flat us / probe us)", "n_gpus": 1, "steps": 30,
        "warmup": 3, "ms_per_step": round(best["probe_us"] / 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "build_s": round(build_s, 3), "nlist": nlist, "max_list": info["max_list"], "points": points,
        "config": {"workload": f"{n} facts of one user, {dim}-d unit embeddings clustered around {topics} "
                               f"topics (spread {spread}), 8 k-means iterations, k={k}",
                   "facts": n, "k": k},
    }
    print(json.dumps(out), flush=True)
    ix.close()
    st.close()


def bench_attend(args):
    """fs_attend_prefill on the Llama-3.1-8B head layout (32 query heads, 8 KV
    heads, head_dim 128): --batch requests of --tq query tokens, each after a
    context of start + injected segment (start U[0,256) + 50 facts of
    U[12,48] tokens, about 1.7k positions), one layer.  FLOPs count the two
    products per attended (token, position, head): 4 * D per pair."""
    import numpy as np
    import torch

    from kv_cache_injection_amd import fs, synth
    from kv_cache_injection_amd.workload import build_store

    wl = synth.make_workload("llama")
    s = wl.shape
    B, tq, hq = args.batch, args.tq, 32
    D = s.head_dim
    ds = build_store(wl, [0], max_batch=max(B, 1))
    rng = np.random.default_rng(wl.seed + 5)
    ctx_len = rng.integers(0, 256, B) + 1488                      # start + mean segment
    q_pos = ctx_len.astype(np.int32)
    bs = s.block_size
    need = int((q_pos.max() + tq + bs - 1) // bs)
    nb = need * B
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 6)
    kc = torch.randn((nb, bs, s.num_kv_heads, D), generator=g, device="cuda").to(torch.bfloat16)
    vc = torch.randn((nb, bs, s.num_kv_heads, D), generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn((B, tq, hq, D), generator=g, device="cuda").to(torch.bfloat16)
    table = torch.from_numpy(rng.permutation(nb)[: need * B].reshape(B, need).astype(np.int32)).cuda()
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    qp = torch.from_numpy(q_pos).cuda()
    out = torch.empty((B, tq, hq, D), device="cuda")
    scale = 1.0 / np.sqrt(D)
    ws_bytes = fs.fs_attend_workspace_size(ds.store, B, tq, hq)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")

    def call():
        fs.fs_attend_prefill(ds.store, B, q, kc, vc, table, need, ctx, qp, scale, out, ws)

    for _ in range(max(args.warmup, 5)):
        call()
    torch.cuda.synchronize()
    steps = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record()
        call()
        e1.record()
    torch.cuda.synchronize()
    if fs.fs_poll_errors(ds.store):
        raise RuntimeError("device error bits set")
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    pairs = sum(int(q_pos[b]) * tq + tq * (tq + 1) // 2 for b in range(B))   # (token, position)
    flops = 4.0 * D * hq * pairs
    kv_bytes = sum(2 * (int(q_pos[b]) + tq) * s.num_kv_heads * D * 2 for b in range(B))
    io_bytes = B * tq * hq * D * (2 + 4)
    t = float(ms.mean()) * 1e-3
    tf = flops / t / 1e12
    out_line = {
        "metric": "paged-attention prefill over the injected cache: TFLOP/s",
        "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(float(ms.mean()), 5), "ms_median": round(float(np.median(ms)), 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tf / 2500.0, 5),
                     "hbm_GBps_unique": round((kv_bytes + io_bytes) / t / 1e9, 1)},
        "config": {"workload": f"Llama-3.1-8B heads (32 q / 8 kv, D 128), {B} request(s) x {tq} query "
                               f"tokens after a context of {int(q_pos.min())}..{int(q_pos.max())} positions, "
                               f"one layer, block_size {bs}",
                   "batch": B, "tq": tq, "workspace_bytes": ws_bytes},
    }
    print(json.dumps(out_line), flush=True)
    ds.close()


def bench_overlap(args):
    """Layer-pipelined injection (device store): per step, retrieval, then
    fs_inject launches over chunks of consecutive layers on a side stream with
    one event per chunk, while the main stream runs a synthetic forward whose
    layer l waits for the event of l's chunk.  The forward is a stand-in load
    (a prefill chunk through an MLP of the model's width: two bf16 GEMMs per
    layer), not part of the library.  Plans: one launch per layer; layer 0
    alone then the rest; chunks of 1, 2, 4, ... layers; all layers before the
    forward starts; and the first and third with the batch planned once
    (fs_plan_inject) and every chunk injecting from the plan.  Reported per plan: injection alone, both overlapped, and
    the exposed time (overlapped minus forward alone); value = the best plan's."""
    import numpy as np
    import torch

    from kv_cache_injection_amd import fs, synth
    from kv_cache_injection_amd.pipeline import LayerInjector
    from kv_cache_injection_amd.workload import build_store, request_tensors

    wl = synth.make_workload(args.config, k=args.k)
    s = wl.shape
    nl = args.layers or s.num_layers
    layers = list(range(nl))
    B, k = s.batch, wl.k
    print(f"[bench] {s.name} overlap: building store ({nl} layers)", file=sys.stderr, flush=True)
    ds = build_store(wl, layers)
    kc, vc = synth.make_caches(wl, layers, "cuda")
    caches = fs.CacheTable(ds.store, kc, vc, kc[0].shape[0])
    sets = [request_tensors(wl, queries=r["queries"], start_pos=r["start_pos"], block_table=r["block_table"])
            for r in synth.request_sets(wl, max(args.sets, 1), seed=wl.seed + 1)]
    user = sets[0]["user"]
    mb = wl.block_table.shape[1]
    steps = max(1, min(args.steps, 50))
    warm = max(1, min(args.warmup, 5))
    total = warm + steps
    ids = torch.empty((total, B, k), dtype=torch.int32, device="cuda")
    ntok = torch.zeros((total, B), dtype=torch.int32, device="cuda")
    hidden, inter, tokens = 4096, 14336, 512           # Llama-3.1-8B MLP width, one prefill chunk
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.seed + 7)
    w_up = [torch.randn((hidden, inter), generator=g, device="cuda", dtype=torch.bfloat16) * 0.02
            for _ in layers]
    w_dn = [torch.randn((inter, hidden), generator=g, device="cuda", dtype=torch.bfloat16) * 0.02
            for _ in layers]
    x0 = torch.randn((tokens, hidden), generator=g, device="cuda", dtype=torch.bfloat16)
    inj = LayerInjector(ds.store, caches, nl)
    ret = [fs.prepare_retrieve_topk(ds.store, B, user, sets[i % len(sets)]["query"], k, ids[i], None,
                                    ntok[i]) for i in range(total)]
    # layer plans: consecutive chunks, one launch each
    plans = {"per_layer": [(l, l + 1) for l in layers],
             "first_then_rest": [(0, 1), (1, nl)] if nl > 1 else [(0, 1)],
             "doubling": [],
             "all_upfront": [(0, nl)]}
    b0, w = 0, 1
    while b0 < nl:
        plans["doubling"].append((b0, min(nl, b0 + w)))
        b0, w = b0 + w, 2 * w
    # the same chunkings with the batch planned once (fs_plan_inject) and
    # every chunk injecting from the plan
    for name in ("per_layer", "doubling"):
        plans[name + "_planned"] = plans[name]
    calls = {name: [inj.prepare(B, user, ids[i], k, sets[i % len(sets)]["block_table"], mb,
                                sets[i % len(sets)]["start_pos"], chunks=plan,
                                planned=name.endswith("_planned")) for i in range(total)]
             for name, plan in plans.items()}

    def forward(wait_layers: bool):
        x = x0
        for l in layers:
            if wait_layers:
                inj.wait(l)
            x = torch.matmul(torch.matmul(x, w_up[l]), w_dn[l])
        return x

    def run(mode, plan, i):
        if mode in ("both", "inject"):
            ret[i]()
            inj.launch(calls[plan][i])
        if mode in ("both", "forward"):
            forward(mode == "both")
        torch.cuda.current_stream().wait_stream(inj.stream)

    def timed(mode, plan):
        for i in range(warm):
            run(mode, plan, i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(warm, total):
            run(mode, plan, i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3

    t_fwd = timed("forward", "per_layer")
    res = {}
    for name in plans:
        t_inj = timed("inject", name)
        t_both = timed("both", name)
        exposed = max(0.0, t_both - t_fwd)
        res[name] = {"chunks": len(plans[name]), "inject_only_ms": round(t_inj, 4),
                     "overlapped_ms": round(t_both, 4), "exposed_ms": round(exposed, 4),
                     "hidden_frac": round(1.0 - exposed / t_inj, 4) if t_inj > 0 else None}
    flags = fs.fs_poll_errors(ds.store)
    if flags:
        raise RuntimeError(f"device error bits 0x{flags:x}")
    best = min(res, key=lambda n: res[n]["exposed_ms"])
    out = {
        "metric": "layer-pipelined injection under a synthetic per-layer forward: exposed injection time",
        "value": res[best]["exposed_ms"], "unit": "ms per step", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": res[best]["overlapped_ms"], "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "forward_only_ms": round(t_fwd, 4), "best_plan": best, "plans": res,
        "config": {"workload": f"{s.name}: {nl} layers, fs_inject launches over chunks of layers on a side "
                               f"stream; forward stand-in {tokens} tokens x ({hidden}->{inter}->{hidden}) "
                               f"bf16 GEMMs per layer",
                   "batch": B, "k": k, "layers": nl},
    }
    print(json.dumps(out), flush=True)
    ds.close()


def bench_pinned(args):
    """Pinned-host store: per step, retrieval, then for every layer l the
    fetch of layer l's selected rows over the host link (side stream, staging
    slot l % 2) and the injection of layer l (main stream).  The fetch of
    layer l+1 waits only for the injection of layer l-1 (which read the slot
    it refills), so the host link stays busy while layers are injected.
    Reported against a plain pinned-host -> device copy of the same bytes."""
    import numpy as np
    import torch

    from kv_cache_injection_amd import fs, synth
    from kv_cache_injection_amd.pipeline import PinnedLayerInjector
    from kv_cache_injection_amd.workload import build_store, request_tensors

    wl = synth.make_workload(args.config, k=args.k)
    s = wl.shape
    nl = args.layers or min(8, s.num_layers)
    layers = list(range(nl))
    B, k = s.batch, wl.k
    print(f"[bench] {s.name} pinned: building store ({nl} layers in pinned host memory)",
          file=sys.stderr, flush=True)
    ds = build_store(wl, layers, pinned=True, staging_layers=2)
    kc, vc = synth.make_caches(wl, layers, "cuda")
    caches = fs.CacheTable(ds.store, kc, vc, kc[0].shape[0])
    sets = [request_tensors(wl, queries=r["queries"], start_pos=r["start_pos"], block_table=r["block_table"])
            for r in synth.request_sets(wl, max(args.sets, 1), seed=wl.seed + 1)]
    user = sets[0]["user"]
    mb = wl.block_table.shape[1]
    steps = max(1, min(args.steps, 10))
    warm = max(1, min(args.warmup, 2))
    total = warm + steps
    ids = torch.empty((total, B, k), dtype=torch.int32, device="cuda")
    ntok = torch.zeros((total, B), dtype=torch.int32, device="cuda")
    main = torch.cuda.current_stream()
    pipe = PinnedLayerInjector(ds.store, caches, nl, staging_layers=2)

    def step(i, inject=True):
        r = sets[i % len(sets)]
        fs.fs_retrieve_topk(ds.store, B, user, r["query"], k, ids[i], None, ntok[i])
        pipe.launch(B, user, ids[i], k, r["block_table"], mb, r["start_pos"], inject=inject)
        pipe.wait_all(main)

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warm, total):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    flags = fs.fs_poll_errors(ds.store)
    if flags:
        raise RuntimeError(f"device error bits 0x{flags:x}")
    L = ntok.cpu().numpy().astype(np.int64)[warm:]
    link_bytes = 4 * int(L.sum()) * nl * s.num_kv_heads * s.head_dim    # K and V rows read once
    # fetch alone, same steps
    u0 = time.perf_counter()
    for i in range(warm, total):
        step(i, inject=False)
    torch.cuda.synchronize()
    u1 = time.perf_counter()
    # a plain host -> device copy of one step's bytes, pinned source
    per_step = link_bytes // steps
    h = torch.empty(per_step, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(per_step, dtype=torch.uint8, device="cuda")
    d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(steps):
        d.copy_(h, non_blocking=True)
    torch.cuda.synchronize()
    c1 = time.perf_counter()
    wall = t1 - t0
    link = link_bytes / wall / 1e9
    h2d = per_step * steps / (c1 - c0) / 1e9
    out = {
        "metric": "pinned-host KV fetch + inject: host-link GB/s per batch (k=50)",
        "value": round(link, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(wall / steps * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64", "data": "synthetic",
        "fetch_only_ms_per_step": round((u1 - u0) / steps * 1e3, 3),
        "h2d_copy_probe_GBps": round(h2d, 2), "frac_of_h2d_probe": round(link / h2d, 4),
        "requests_per_s": round(B * steps / wall, 2),
        "config": {"workload": f"{s.name} (pinned host arenas): {nl} of {s.num_layers} layers resident, "
                               f"{s.num_kv_heads} KV heads x {s.head_dim}; {B} request(s) per step, k={k}; "
                               f"staging ring of 2 layers, per-layer fetch -> inject pipeline",
                   "batch": B, "k": k, "layers": nl, "mean_segment_tokens": round(float(L.mean()), 1)},
    }
    print(json.dumps(out), flush=True)
    ds.close()


def inject_source_digest() -> str:
    """sha256 over the code of the inject kernel's sources, comments and
    whitespace removed (counters taken on other code no longer describe it;
    a comment does not change the kernel)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("inject.hip", "fs_internal.h", "fs_device.h", "fs_plan.h"):
        with open(os.path.join(ROOT, "kv_cache_injection_amd", "csrc", f)) as fh:
            text = fh.read()
        # string literals are kept whole; // and /* */ comments go
        text = re.sub(r'("(?:\\.|[^"\\])*")|//[^\n]*|/\*.*?\*/',
                      lambda m: m.group(1) or " ", text, flags=re.S)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_traffic(config: str, layers: int):
    """HBM bytes per inject launch from the committed rocprofv3 counter record
    (FETCH_SIZE and WRITE_SIZE, scaled by what the same counters read for a
    device copy of one inject's bytes), or None when the record is for
    another kernel build or workload."""
    path = os.path.join(ROOT, "profiles", "inject_llama_hbm_traffic.json")
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("config") != config or rec.get("layers") != layers:
        return None
    if rec.get("kernel_source_sha256") != inject_source_digest():
        return None
    return rec.get("traffic_bytes_per_launch")


def host_cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_share() -> tuple[int, dict]:
    """Threads for the all-cores leg: the CPUs this process may run on,
    capped by OMP_NUM_THREADS when that is set (the CPU share a job is given
    on a shared host), with the counts it came from."""
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    share = affinity
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        share = min(share, int(omp))
    return share, {"host_cpus": os.cpu_count(), "affinity_cpus": affinity,
                   "OMP_NUM_THREADS": omp or None}


def cpu_baseline(wl, ds, layers, n_req, max_host_bytes=16 << 30):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    retrieve + compose + rotate + scatter for ``n_req`` requests, over the
    resident layers whose arenas fit ``max_host_bytes`` of host memory (all of
    them for the Llama-shaped store).  Timed on every core of the process's
    CPU share (cpu_share): each request's retrieval with BLAS on that many
    threads, then its layers split over a thread pool of that size (numpy
    releases the interpreter lock inside its array operations); and beside
    it on one thread.  Same algorithmic-bytes accounting."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from kv_cache_injection_amd import synth

    s = wl.shape
    per_layer = 2 * ds.k_pre[0].numel() * 2
    nl = max(1, min(len(layers), int(max_host_bytes // per_layer)))
    use = list(range(nl))
    print(f"[bench] cpu baseline: copying {nl} layer(s) of arenas to host", file=sys.stderr, flush=True)
    kb = [synth.bf16_bits(ds.k_pre[i]) for i in use]
    vb = [synth.bf16_bits(ds.v[i]) for i in use]
    nb = s.pool_blocks
    shape = (nb, s.block_size, s.num_kv_heads, s.head_dim)
    kc = [np.full(shape, synth.SENTINEL_BITS, np.uint16) for _ in use]
    vc = [np.full(shape, synth.SENTINEL_BITS, np.uint16) for _ in use]
    sets = synth.request_sets(wl, n_req, seed=wl.seed + 1)   # the bench's first sets
    u = int(wl.users[0])
    n_user = int(wl.user_fact_begin[u + 1] - wl.user_fact_begin[u])

    def one_request(i, pool=None, chunks=None):
        r = sets[i]
        ids, _ = oracle.retrieve(wl.emb, wl.user_fact_begin, u, r["queries"][0], wl.k)
        args = (ids, wl.fact_len, wl.fact_token_begin, int(r["start_pos"][0]), r["block_table"][0],
                s.block_size, s.rope_theta)
        if pool is None:
            L = oracle.inject_request(kb, vb, kc, vc, *args, use)
        else:
            futs = [pool.submit(oracle.inject_request, [kb[j] for j in c], [vb[j] for j in c],
                                [kc[j] for j in c], [vc[j] for j in c], *args, c) for c in chunks]
            L = [f.result() for f in futs][0]
        return 8 * L * nl * s.num_kv_heads * s.head_dim + 4 * n_user * s.embed_dim

    share, counts = cpu_share()
    nt = max(1, share)
    chunks = [c for c in (use[j::nt] for j in range(nt)) if c]
    with threadpool_limits(limits=nt), ThreadPoolExecutor(len(chunks)) as pool:
        t1 = time.perf_counter()
        total_all = sum(one_request(i, pool, chunks) for i in range(n_req))
        dt_all = time.perf_counter() - t1
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        total_one = sum(one_request(i) for i in range(n_req))
        dt = time.perf_counter() - t0
    return {"value": round(total_all / dt_all / 1e9, 4), "unit": "GB/s",
            "requests_per_s": round(n_req / dt_all, 4), "cores": nt, "kind": "oracle",
            "seconds": round(dt_all, 2),
            "sample": f"{n_req} request(s) of the {s.name} workload (the first request of each "
                      f"set), {nl} layer(s), k={wl.k}: numpy fp64 oracle, retrieval with BLAS on {nt} "
                      f"threads, each request's layers split over a pool of {min(nt, nl)} threads",
            "cpu_model": host_cpu_model(), **counts,
            "one_thread": {"value": round(total_one / dt / 1e9, 4), "unit": "GB/s",
                           "requests_per_s": round(n_req / dt, 4), "cores": 1,
                           "seconds": round(dt, 2), "sample": "the same requests on one thread"}}


if __name__ == "__main__":
    main()
