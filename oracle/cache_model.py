"""Shadow model of KV-cache slot placement (integer only).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: full-context KV heads keep every earlier token; streaming
heads hold the sequence's first positions plus a window of the newest ones (model card
"DuoAttention Laguna Adapter", "Summary" and "Why It Works"); the adapter
reorders heads so full and streaming heads are separated (same card, "Changes
In This Submission"); a static Duo KV cache is preallocated (same section).
The pages never describe slots, so the placement below is this library's own
contract, modelled here token by token in append order:

* heads of each class are numbered by ascending KV-head index (the cache-side
  image of the head reordering);
* full-context head, full layer:       slot = position;
* full-context head, sliding layer:    slot = position mod W (a ring of W);
* streaming head:                      slot = position if position < sink,
                                       else sink + (position - sink) mod recent.

Applying every appended token in order makes the last writer of a slot win,
so the final state equals "only the newest position of each slot is written".
"""
from __future__ import annotations


class ShadowCache:
    def __init__(self, *, batch: int, hkv: int, layer: str, window: int, sink: int,
                 recent: int, full_attention_heads=None):
        self.batch, self.hkv = batch, hkv
        self.layer, self.window = layer, window
        self.sink, self.recent = sink, recent
        mask = [1] * hkv if full_attention_heads is None else [int(x) for x in full_attention_heads]
        self.streaming = [m == 0 for m in mask]
        self.rank = []
        nf = ns = 0
        for s in self.streaming:
            self.rank.append(ns if s else nf)
            if s:
                ns += 1
            else:
                nf += 1
        self.n_full, self.n_stream = nf, ns
        # slots[(b, cls, rank)] = {slot: position}; cls 0 = full, 1 = streaming
        self.slots = {}

    def slot_of(self, kvh: int, pos: int) -> int:
        if self.streaming[kvh]:
            if pos < self.sink:
                return pos
            return self.sink + (pos - self.sink) % self.recent
        if self.layer == "sliding" and self.window > 0:
            return pos % self.window
        return pos

    def append(self, b: int, start: int, count: int):
        for t in range(count):
            p = start + t
            for kvh in range(self.hkv):
                cls = 1 if self.streaming[kvh] else 0
                self.slots.setdefault((b, cls, self.rank[kvh]), {})[self.slot_of(kvh, p)] = p

    def position_at(self, b: int, kvh: int, slot: int):
        """Position held in the slot, or None if never written."""
        cls = 1 if self.streaming[kvh] else 0
        return self.slots.get((b, cls, self.rank[kvh]), {}).get(slot)
