"""Layer-pipelined injection: stream and event plumbing around the library.

A serving engine runs the prefill of the request's own tokens layer by layer.
Layer l's attention needs layer l's injected K/V, and nothing more, so the
injection of layer l only has to finish before the forward reaches layer l.
InferScale injects into the engine's paged cache at serving time and offloads
the store to host memory when it does not fit the GPU (gist.science summary,
"Phase En-ligne" and "Résultats").

``LayerInjector`` issues fs_inject launches on a side stream, one per chunk
of consecutive layers (one layer per chunk by default), and records one event
per chunk; the forward waits on ``wait(l)`` before it reads layer l.  ``PinnedLayerInjector`` does the same for stores whose K/V live in pinned
host memory: the fetch of layer l's rows over the host link (fs_fetch_async,
into staging slot l % staging_layers) runs on a fetch stream, the injection
of layer l waits for that fetch, and the fetch that refills a slot waits for
the injection that last read it.

Nothing here computes: every step runs in the library's kernels.  All streams
keep the default priority.
"""

from __future__ import annotations

from typing import List, Optional, Sequence

import torch

from . import fs


class LayerInjector:
    """Layer-pipelined injection of one batch on a side stream (device
    stores): one launch per chunk of consecutive layers, one event per chunk.
    One chunk per layer is the plain per-layer pipeline.  A first chunk of
    one layer followed by larger chunks keeps what the forward waits for
    before its first layer small, with fewer launches overall."""

    def __init__(self, store, caches: "fs.CacheTable", num_layers: int,
                 stream: Optional[torch.cuda.Stream] = None):
        self.store = store
        self.caches = caches
        self.num_layers = num_layers
        self.stream = stream or torch.cuda.Stream()
        # one event per launch: at most one per layer, and the plan
        self._events: List[torch.cuda.Event] = [torch.cuda.Event() for _ in range(num_layers + 1)]
        self._event_of: List[Optional[torch.cuda.Event]] = [None] * num_layers
        self._waited = {}                 # stream -> the chunk event it last waited on

    def prepare(self, batch: int, user, ids, k: int, block_table, max_blocks: int, start_pos,
                layers: Optional[Sequence[int]] = None,
                chunks: Optional[Sequence["tuple[int, int]"]] = None,
                planned: bool = False) -> List["tuple[tuple, fs.Prepared]"]:
        """Marshal the calls once (validated like fs_inject), for batches that
        reuse the same buffers.  ``chunks``: consecutive (begin, end) layer
        ranges, each one fs_inject_layers launch; default one per layer (of
        ``layers``, default all).  ``planned``: the batch is composed and
        validated once into a plan of its own (fs_plan_inject, the first
        launch), and every chunk injects from it (fs_inject_planned) instead
        of planning again."""
        if chunks is None:
            ls = range(self.num_layers) if layers is None else layers
            chunks = [(l, l + 1) for l in ls]
        out = []
        plan = None
        if planned:
            plan = fs.new_inject_plan(self.store, batch)
            out.append(((0, 0), fs.prepare_plan_inject(self.store, batch, user, ids, k, block_table, max_blocks,
                                                       start_pos, self.caches.num_blocks, plan,
                                                       stream=self.stream)))
        for b, e in chunks:
            if not 0 <= b < e <= self.num_layers:
                raise ValueError(f"layer chunk ({b}, {e}) outside [0, {self.num_layers})")
            if planned:
                call = fs.prepare_inject_planned(self.store, (b, e), batch, k, plan, self.caches,
                                                 stream=self.stream)
            else:
                lay = b if e == b + 1 else (b, e)
                call = fs.prepare_inject(self.store, lay, batch, user, ids, k, block_table,
                                         max_blocks, start_pos, self.caches, stream=self.stream)
            out.append(((b, e), call))
        return out

    def launch(self, calls, after: Optional[torch.cuda.Stream] = None):
        """Enqueue prepared calls.  ``after`` (default: the current stream) is
        the stream whose pending work produced the ids: the side stream waits
        for it first."""
        self.stream.wait_stream(after or torch.cuda.current_stream())
        self._waited.clear()
        for i, ((b, e), call) in enumerate(calls):
            call()
            ev = self._events[i]
            ev.record(self.stream)
            for l in range(b, e):
                self._event_of[l] = ev

    def wait(self, layer: int, stream: Optional[torch.cuda.Stream] = None):
        """Make ``stream`` (default: current) wait until ``layer`` is injected.
        A stream waits on each chunk's event once: the later layers of a
        chunk it has already waited for add no wait (every cross-stream wait
        costs the waiting queue a few microseconds)."""
        ev = self._event_of[layer]
        if ev is None:
            raise RuntimeError(f"layer {layer} was not launched")
        st = stream or torch.cuda.current_stream()
        if self._waited.get(st) is ev:
            return
        st.wait_event(ev)
        self._waited[st] = ev


class PinnedLayerInjector:
    """Per-layer fetch -> inject pipeline for pinned-host stores.

    fetch(l) on ``fetch_stream`` fills staging slot l % staging_layers; it
    waits for inject(l - staging_layers), the last reader of that slot.
    inject(l) on ``inject_stream`` waits for fetch(l)."""

    def __init__(self, store, caches: "fs.CacheTable", num_layers: int, staging_layers: int,
                 fetch_stream: Optional[torch.cuda.Stream] = None,
                 inject_stream: Optional[torch.cuda.Stream] = None):
        if staging_layers < 1:
            raise ValueError("staging_layers must be >= 1")
        self.store = store
        self.caches = caches
        self.num_layers = num_layers
        self.staging_layers = staging_layers
        self.fetch_stream = fetch_stream or torch.cuda.Stream()
        self.inject_stream = inject_stream or torch.cuda.Stream()
        self.fetched = [torch.cuda.Event() for _ in range(num_layers)]
        self.done = [torch.cuda.Event() for _ in range(num_layers)]

    def launch(self, batch: int, user, ids, k: int, block_table, max_blocks: int, start_pos,
               after: Optional[torch.cuda.Stream] = None, inject: bool = True):
        """Enqueue fetch and injection of every layer.  With ``inject=False``
        only the fetches run (to time the host link alone)."""
        src = after or torch.cuda.current_stream()
        self.fetch_stream.wait_stream(src)
        self.inject_stream.wait_stream(src)
        # the previous batch's injections still read the staging slots
        self.fetch_stream.wait_stream(self.inject_stream)
        S = self.staging_layers
        for l in range(self.num_layers):
            if l >= S:
                self.fetch_stream.wait_event(self.done[l - S])   # slot l % S is free again
            fs.fs_fetch_async(self.store, batch, user, ids, k, l, l + 1, stream=self.fetch_stream)
            self.fetched[l].record(self.fetch_stream)
            if inject:
                self.inject_stream.wait_event(self.fetched[l])
                fs.fs_inject(self.store, l, batch, user, ids, k, block_table, max_blocks,
                             start_pos, self.caches, stream=self.inject_stream)
                self.done[l].record(self.inject_stream)
            else:
                self.done[l].record(self.fetch_stream)

    def wait(self, layer: int, stream: Optional[torch.cuda.Stream] = None):
        (stream or torch.cuda.current_stream()).wait_event(self.done[layer])

    def wait_all(self, stream: Optional[torch.cuda.Stream] = None):
        s = stream or torch.cuda.current_stream()
        s.wait_stream(self.fetch_stream)
        s.wait_stream(self.inject_stream)
