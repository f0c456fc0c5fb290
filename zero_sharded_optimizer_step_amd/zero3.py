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
it reaches it.

The gathered buckets live in one arena of max_live elements, filled in
bucket order as a ring.  A gather may only take space that no bucket the
caller still holds occupies, and before writing it the side stream waits
for the event the caller's stream recorded after its last use of whatever
bucket was there before.  So the bound holds on the device's timeline, and
the host can run ahead of the device without growing memory or blocking.
This module only schedules library calls and stream events; it computes
nothing.
"""
from __future__ import annotations

from collections import deque
from typing import Iterator, Optional, Sequence, Tuple

import torch

from . import zero_bucket_plan, zero_gather_params


def ring_place(held: Sequence[Tuple[int, int]], size: int, capacity: int) -> Optional[int]:
    """Where the next bucket of `size` elements goes in a ring arena of
    `capacity` elements whose held buckets are `held`, (start, end) pairs
    oldest first, each placed by this function in turn: right after the
    newest one, or back at 0 when the arena's end is too near; None while
    held buckets are in the way.  Never overlaps a held bucket."""
    if not held:
        return 0
    tail, head = held[0][0], held[-1][1]
    # each bucket starts where the one before it ended, except the one that
    # went back to 0: at most one, since that leaves [head, tail) free
    if all(b[0] >= a[1] for a, b in zip(held, held[1:])):
        if head + size <= capacity:              # held buckets fill [tail, head)
            return head
        return 0 if size <= tail else None
    return head if head + size <= tail else None   # they wrapped: [head, tail) is free


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
        self.arena = None                            # max_live elements, from the first walk
        self.last_stream = None                      # the caller's stream of the last walk

    def forward(self, stream=None) -> Iterator[Tuple[int, torch.Tensor]]:
        """Yield (layer index, its gathered parameters) in order; each view is
        ready on `stream` (default: the current stream) when yielded and may
        be used until the next bucket's first layer is requested."""
        main = stream or torch.cuda.current_stream()
        if self.arena is None:
            self.arena = torch.empty(self.max_live, dtype=self.dtype,
                                     device=self.shards[0].device)
            self.arena.record_stream(self.side)      # kept until the side stream is done
        self.arena.record_stream(main)               # and every caller stream that read it
        # The side stream follows all the caller has queued so far: the
        # shards' last writes and an earlier walk's last reads of the arena,
        # also when that walk ran on another stream.
        self.side.wait_stream(main)
        if self.last_stream is not None and self.last_stream != main:
            self.side.wait_stream(self.last_stream)
        self.last_stream = main
        pending = deque()       # gathered, not yet left by the caller: (bucket, start, end, event)
        released = []           # left by the caller, maybe still read on its stream: (start, end, event)
        nxt = 0

        def issue(start: int):
            nonlocal nxt, released
            lo, hi, _, _ = self.buckets[nxt]
            end = start + (hi - lo)
            # Wait for the caller's stream to be done with what was there.
            # Its events complete in order, so the newest overlapping one
            # covers every older release as well, which need no wait after.
            last = max((i for i, (a, b, _) in enumerate(released) if a < end and start < b),
                       default=-1)
            if last >= 0:
                ev = released[last][2]
                if not ev.query():
                    self.side.wait_event(ev)
                released = released[last + 1:]
            zero_gather_params(self.part, self.shards, self.dtype, lo, hi,
                               self.arena[start:end], self.side)
            ev = torch.cuda.Event()
            ev.record(self.side)
            pending.append((nxt, start, end, ev))
            nxt += 1

        for k, (lo, hi, first, count) in enumerate(self.buckets):
            if not pending:
                issue(0)                             # the bucket the caller needs now
            while nxt < len(self.buckets):           # prefetch into free space
                start = ring_place([(p[1], p[2]) for p in pending],
                                   self.buckets[nxt][1] - self.buckets[nxt][0], self.max_live)
                if start is None:
                    break
                issue(start)
            _, start, end, ev = pending[0]
            main.wait_event(ev)
            buf = self.arena[start:end]
            for t in range(first, first + count):
                off, n = self.layers[t]
                yield t, buf[off - lo:off - lo + n]
            pending.popleft()
            done = torch.cuda.Event()
            done.record(main)                        # after the caller's last use of it
            released.append((start, end, done))
