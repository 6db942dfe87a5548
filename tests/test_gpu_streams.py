"""Concurrent calls on two streams, each request with its own caches,
workspaces, inputs and outputs. The library keeps no per-call state outside
the caller's buffers (the split-K and key-range-piece arrival counters live
in each call's workspace; the device error word is only ever OR-ed), so the
two requests' calls, issued interleaved on two streams, must give the same
bits as the same calls run one after another on one stream."""
from itertools import zip_longest

import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, dev, host_bits

pytestmark = pytest.mark.gpu


class Request:
    """One decode step of a Duo layer (append the new token's K with its
    prologue; decode with the q prologue and the sink; a verify block), a
    sliding-window chunk, and a chunk over the longest sequence whose
    full-context query tiles are cut into key-range pieces."""

    def __init__(self, lib, seed, mask, lengths):
        import torch
        self.lib = lib
        layer = self.layer = lib.Layer(full_attention_heads=mask)
        hq, hkv = layer.num_q_heads, layer.num_kv_heads
        B, T = len(lengths), 4
        cap = max(lengths) + 64
        k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, lengths, hkv, 128)
        v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, lengths, hkv, 128)
        self.cache = lib.KVCache(layer, B, cap)
        for b in range(B):
            lib.kv_append(layer, self.cache, dev(k[b][None]), dev(v[b][None]),
                          torch.tensor([0], dtype=torch.int32, device="cuda"), max_end_pos=lengths[b],
                          batch=1, batch_offset=b)
        w = torch.from_numpy((1 + 0.3 * np.random.default_rng(seed).standard_normal(128)).astype(np.float32)).cuda()
        self.pro = lib.Prologue(norm_weight=w, rope=lib.Rope())
        self.sink = torch.from_numpy(wl.sink_logits(seed, hq)).cuda()
        self.kn = dev(wl.normal_tokens(seed + 1, wl.K, B, 0, 1, hkv, 128))
        self.vn = dev(wl.normal_tokens(seed + 1, wl.V, B, 0, 1, hkv, 128))
        self.q1 = dev(wl.decode_queries(seed + 1, B, hq, 128))
        self.qb = dev(wl.normal_tokens(seed + 2, wl.Q, B, 0, T, hq, 128))
        self.kb = dev(wl.normal_tokens(seed + 2, wl.K, B, 0, T, hkv, 128))
        self.vb = dev(wl.normal_tokens(seed + 2, wl.V, B, 0, T, hkv, 128))
        self.qc = dev(wl.normal_tokens(seed + 3, wl.Q, 1, 0, 256, hq, 128))
        self.kc = dev(wl.normal_tokens(seed + 3, wl.K, 1, 0, 256, hkv, 128))
        self.vc = dev(wl.normal_tokens(seed + 3, wl.V, 1, 0, 256, hkv, 128))
        self.pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        self.seq = torch.tensor([x + 1 for x in lengths], dtype=torch.int32, device="cuda")
        self.maxlen = max(lengths) + 1
        self.ws = lib.decode_workspace(layer, B, self.maxlen)
        self.wsb = lib.decode_block_workspace(layer, B, T, self.maxlen)
        self.lc = lib.Layer(kind=lib.SLIDING, window=512)
        longest = int(np.argmax(lengths))
        P = self.P = lengths[longest]
        self.qp = dev(wl.normal_tokens(seed + 4, wl.Q, 1, P, 256, hq, 128))
        self.kp = dev(wl.normal_tokens(seed + 4, wl.K, 1, P, 256, hkv, 128))
        self.vp = dev(wl.normal_tokens(seed + 4, wl.V, 1, P, 256, hkv, 128))
        self.wsp = lib.prefill_workspace(layer, 1, 256, [P])
        assert lib.prefill_plan(layer, 1, 256, P, True)[:, 5].max() > 1, "no query tile was cut"
        self.past = lib.KVCache(layer, 1, cap)
        sl = slice(longest, longest + 1)
        self.past.k_main, self.past.v_main = self.cache.k_main[sl], self.cache.v_main[sl]
        self.past.k_stream, self.past.v_stream = self.cache.k_stream[sl], self.cache.v_stream[sl]
        self.out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        self.outb = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
        self.outc = torch.empty((1, 256, hq, 128), dtype=torch.bfloat16, device="cuda")
        self.outp = torch.empty((1, 256, hq, 128), dtype=torch.bfloat16, device="cuda")

    def calls(self):
        lib, L = self.lib, self.layer
        return [
            lambda: lib.kv_append(L, self.cache, self.kn, self.vn, self.pos, max_end_pos=self.maxlen,
                                  k_prologue=self.pro),
            lambda: lib.attn_decode(L, self.cache, self.q1, self.seq, self.maxlen, self.out, self.ws,
                                    lse=self.lse, q_prologue=self.pro, sink_logits=self.sink),
            lambda: lib.attn_decode_block(L, self.cache, self.qb, self.kb, self.vb, self.seq, self.maxlen,
                                          self.outb, self.wsb, sink_logits=self.sink),
            lambda: lib.attn_prefill(self.lc, self.qc, self.kc, self.vc, self.outc),
            lambda: lib.attn_prefill(L, self.qp, self.kp, self.vp, self.outp, start_pos=self.P, past=self.past,
                                     workspace=self.wsp),
        ]

    def clear(self):
        for t in (self.out, self.lse, self.outb, self.outc, self.outp):
            t.zero_()

    def results(self):
        return [host_bits(self.out), self.lse.cpu().numpy().copy(), host_bits(self.outb), host_bits(self.outc),
                host_bits(self.outp)]


def test_two_streams_match_one_stream(lib):
    import torch
    announce("two requests interleaved on two streams")
    reqs = [Request(lib, 61, [0, 1, 0, 0, 1, 0, 0, 0], [100, 2000, 5000]),
            Request(lib, 71, [1, 0, 0, 0, 0, 0, 1, 1], [4500, 30, 800, 1500])]
    torch.cuda.synchronize()
    lib.device_errors(clear=True)
    for r in reqs:
        for c in r.calls():
            c()
    torch.cuda.synchronize()
    want = [r.results() for r in reqs]

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    names = ("decode", "lse", "block", "sliding prefill", "prefill pieces")
    for rep in range(3):
        for r in reqs:
            r.clear()
        torch.cuda.synchronize()
        for pair in zip_longest(*(r.calls() for r in reqs)):
            for s, c in zip(streams, pair):
                if c is not None:
                    with torch.cuda.stream(s):
                        c()
        torch.cuda.synchronize()
        for i, r in enumerate(reqs):
            for name, a, b in zip(names, r.results(), want[i]):
                assert np.array_equal(a, b), f"pass {rep}, request {i}: {name} differs from the one-stream result"
    assert lib.device_errors() == 0
