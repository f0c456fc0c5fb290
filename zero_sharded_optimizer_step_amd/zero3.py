"""ZeRO-3 parameter gathering with prefetch, on one GPU.

"ZeRO技术解析：大模型分布式训练的革命性突破" §1.2.3 and §3.1: under stage 3
the parameters themselves are partitioned; stage3_prefetch_bucket_size
sets how much is fetched ahead and stage3_max_live_parameters bounds how
many gathered parameters are alive at once.  "大模型分片训练" (stage table):
before a layer's forward its parameters are all-gathered, and freed after;
"ZeRO 和分片优化器" (technical insight): the gathered slices a GPU does not
own are dropped.

LayerGatherer walks a model's layers in order.  Consecutive layers are
grouped into prefetch buckets by the library's bucket rule
(zero_bucket_plan); each bucket is gathered from the ranks' shards
(zero_gather_params) on a side stream, as far ahead as the live-parameter
bound allows, and the caller's stream waits for a bucket's event only when
it reaches it.  This module only schedules library calls and stream
events; it computes nothing.
"""
from __future__ import annotations

from collections import deque
from typing import Iterator, Sequence, Tuple

import torch

from . import zero_bucket_plan, zero_gather_params


class LayerGatherer:
    def __init__(self, part, shards: Sequence[torch.Tensor], layer_sizes: Sequence[int],
                 prefetch_bucket: int, max_live: int):
        if sum(layer_sizes) != part.numel:
            raise ValueError("the layers must cover the flat parameter space")
        self.part = part
        self.shards = list(shards)
        self.dtype = self.shards[0].dtype
        slots, buckets = zero_bucket_plan(list(layer_sizes), prefetch_bucket)
        self.layers = [(x.offset, x.numel) for x in slots]
        self.buckets = [(b.begin, b.end, b.first_tensor, b.n_tensors) for b in buckets]
        biggest = max((b[1] - b[0] for b in self.buckets), default=0)
        if max_live < biggest:
            raise ValueError("max_live %d is smaller than the largest bucket %d"
                             % (max_live, biggest))
        self.max_live = max_live
        self.side = torch.cuda.Stream()              # default priority

    def forward(self, stream=None) -> Iterator[Tuple[int, torch.Tensor]]:
        """Yield (layer index, its gathered parameters) in order; each view is
        ready on `stream` (default: the current stream) when yielded and may
        be used until the next bucket's first layer is requested."""
        main = stream or torch.cuda.current_stream()
        self.side.wait_stream(main)                  # the shards' last writes
        pending = deque()                            # (bucket index, buffer, event)
        live = 0
        nxt = 0

        def issue():
            nonlocal nxt, live
            lo, hi, _, _ = self.buckets[nxt]
            # Allocated on the side stream, which writes it: once the caller
            # is done (record_stream below), torch's allocator reuses the
            # memory only after the caller's stream has passed its last
            # read, so a later gather cannot overwrite a bucket still in use.
            with torch.cuda.stream(self.side):
                buf = torch.empty(hi - lo, dtype=self.dtype, device=self.shards[0].device)
            zero_gather_params(self.part, self.shards, self.dtype, lo, hi, buf, self.side)
            ev = torch.cuda.Event()
            ev.record(self.side)
            pending.append((nxt, buf, ev))
            live += hi - lo
            nxt += 1

        for k, (lo, hi, first, count) in enumerate(self.buckets):
            if not pending or pending[0][0] != k:
                issue()
            while nxt < len(self.buckets) and \
                    live + (self.buckets[nxt][1] - self.buckets[nxt][0]) <= self.max_live:
                issue()
            _, buf, ev = pending[0]
            main.wait_event(ev)
            for t in range(first, first + count):
                off, n = self.layers[t]
                yield t, buf[off - lo:off - lo + n]
            pending.popleft()
            buf.record_stream(main)                  # freed once the caller's work is done
            live -= hi - lo
