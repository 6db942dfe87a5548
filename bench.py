#!/usr/bin/env python3
"""Benchmark of the hybrid GQA / sliding-window / DuoAttention attention path
on one MI355X.

Headline (`value`): prefill TFLOP/s of the full-attention prefill workload
(batch 4, 48 query / 8 KV heads, head_dim 128, 8192 causal tokens, bf16 in,
fp32 accumulate). One step = one duo_attn_prefill call over the whole batch.
Algorithmic FLOP = 4 * 128 per (query row, visible key) pair; masked pairs
are not counted.

The same JSON line carries the other halves of the metric, each timed the
same way (HIP events on the stream the kernels run on, inputs resident in
HBM):
  decode      -- KV GB/s of the sliding-window decode (batch 64, window-512
                 ring) and of the DuoAttention decode (batch 16, contexts up to
                 131072, Bernoulli(0.25) full-head mask), and of block decodes
                 of 4, 6 and 8 tokens after those contexts; algorithmic bytes =
                 every visible K and V row read once per KV head; several cache
                 replicas are rotated so the 256 MB Infinity Cache cannot serve
                 them;
  chunked_prefill -- DuoAttention prefill of 131072 tokens in 8192-token
                 chunks (attend + append per chunk);
  kv_append   -- the cache manager on one 8192-token chunk;
  kv_cache    -- static-cache footprint and occupancy of the two Duo
                 workloads beside the same layer without Duo routing
                 (host-side accounting).
`roofline` describes the dominant kernel (the prefill kernel). `cpu_baseline`
times the float64 oracle on a bounded sample of the headline workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "prefill TFLOP/s (% MFMA peak) + decode KV GB/s (% HBM peak), 48Q/8KV d128"
PEAK_MFMA_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
# Ceilings measured on MI355X with in-bounds probe kernels: a loop of
# independent 16x16x32 bf16 MFMAs at two waves per SIMD, and a read stream
# shaped like the decode (per-wave 16 KB tiles, non-temporal 16-byte loads).
MEASURED_MFMA_BF16_TFLOPS = 2300.0
MEASURED_DECODE_READ_GBS = 6820.0
HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Timer:
    """HIP-event timing on torch's current stream (the stream the library
    launches on). The mean comes from one event pair around K back-to-back
    calls; a second pass of K calls with an event between consecutive calls
    gives the per-call median and minimum (events between calls slow short
    kernels slightly, so they stay out of the mean)."""

    def __init__(self, torch):
        self.torch = torch
        self.last = {}

    def run(self, fn, warmup, steps):
        torch = self.torch
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(steps):
            fn(warmup + i)
        e1.record(s)
        torch.cuda.synchronize()
        mean = e0.elapsed_time(e1) / steps  # ms per call
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(s)
        for i in range(steps):
            fn(warmup + steps + i)
            ev[i + 1].record(s)
        torch.cuda.synchronize()
        per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        self.last = {"median_ms": per[len(per) // 2], "min_ms": per[0]}
        return mean


def visible_pairs(layer, streaming: bool, start_pos: int, num_tokens: int) -> int:
    """Sum over query positions i in [start_pos, start_pos + T) of |Vis(i)|,
    from closed forms: i + 1 (causal), min(i + 1, W) (sliding window),
    min(i + 1, S + R) (streaming head)."""
    a, b = start_pos, start_pos + num_tokens - 1

    def s_min(cap):  # sum over i in [a, b] of min(i + 1, cap)
        tot = 0
        hi_lin = min(b, cap - 1)
        if hi_lin >= a:
            tot += (a + 1 + hi_lin + 1) * (hi_lin - a + 1) // 2
        flat_lo = max(a, cap)
        if b >= flat_lo:
            tot += cap * (b - flat_lo + 1)
        return tot
    if streaming:
        return s_min(layer.sink + layer.recent)
    if layer.main_ring:
        return s_min(layer.window)
    return (a + 1 + b + 1) * (b - a + 1) // 2


def prefill_flops(G, layer, batch: int, num_tokens: int, start_pos: int = 0) -> int:
    """Algorithmic FLOP of a prefill call: 4 * 128 per (query row, visible
    key) pair over all batch x Hq rows; masked pairs are not counted. Head
    classes come from the library's head-class plan."""
    g = layer.num_q_heads // layer.num_kv_heads
    classes = G.head_plan(layer)[0]
    total = sum(g * visible_pairs(layer, classes[kvh] == 1, start_pos, num_tokens)
                for kvh in range(layer.num_kv_heads))
    return 4 * 128 * batch * total


def dev_bits(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bench_prefill(torch, G, wl, timer, warmup, steps):
    w = wl.WORKLOADS[2]
    log(f"prefill workload {w.name}: generating inputs")
    q = wl.normal_tokens(w.seed, wl.Q, w.batch, 0, w.seq, w.hq, 128)
    k = wl.normal_tokens(w.seed, wl.K, w.batch, 0, w.seq, w.hkv, 128)
    v = wl.normal_tokens(w.seed, wl.V, w.batch, 0, w.seq, w.hkv, 128)
    qd, kd, vd = dev_bits(torch, q), dev_bits(torch, k), dev_bits(torch, v)
    out = torch.empty_like(qd)
    layer = G.Layer()
    flops = prefill_flops(G, layer, w.batch, w.seq)
    log("prefill: timing")
    ms = timer.run(lambda i: G.attn_prefill(layer, qd, kd, vd, out), warmup, steps)
    return w, (q, k, v), flops, ms, (layer, qd, kd, vd, out)


def bench_swa_prefill(torch, G, wl, timer, warmup, steps):
    """The 1 x 1024 sliding-window prefill (12 query / 2 KV heads, window 512):
    2.4 GFLOP in 96 workgroups, fewer than the 256 CUs, so its time is launch
    and single-workgroup latency, not throughput."""
    w = wl.WORKLOADS[1]
    q = dev_bits(torch, wl.normal_tokens(w.seed, wl.Q, w.batch, 0, w.seq, w.hq, 128))
    k = dev_bits(torch, wl.normal_tokens(w.seed, wl.K, w.batch, 0, w.seq, w.hkv, 128))
    v = dev_bits(torch, wl.normal_tokens(w.seed, wl.V, w.batch, 0, w.seq, w.hkv, 128))
    out = torch.empty_like(q)
    layer = G.Layer(num_q_heads=w.hq, num_kv_heads=w.hkv, kind=G.SLIDING, window=w.window)
    flops = prefill_flops(G, layer, w.batch, w.seq)
    ms = timer.run(lambda i: G.attn_prefill(layer, q, k, v, out), warmup, steps)
    plan = G.prefill_plan(layer, w.batch, w.seq)
    wgs = int((plan[:, 0] >= 0).sum())
    return {"workload": w.name, "algorithmic_flop": flops, "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "ms_median": timer.last["median_ms"], "ms_min": timer.last["min_ms"], "workgroups": wgs,
            "bound": f"latency: {wgs} workgroups for 256 CUs, one short wave of work; "
                     "no MFMA-peak target applies"}


def bench_prologue_epilogue(torch, G, wl, timer, warmup, steps, w, flops, base_ms, devs):
    """The optional prologue (RMSNorm + YaRN RoPE of q fused into the query
    loads; the standalone kernel; K through kv_append's prologue) and
    epilogue (sink logits + per-element output gate) on the headline prefill
    workload, beside the plain call."""
    layer, qd, kd, vd, out = devs
    B, T = w.batch, w.seq
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed)
    wq = 1 + 0.3 * torch.randn(128, device="cuda", generator=g)
    wk = 1 + 0.3 * torch.randn(128, device="cuda", generator=g)
    pq = G.Prologue(norm_weight=wq, rope=G.Rope())
    pk = G.Prologue(norm_weight=wk, rope=G.Rope())
    sink = torch.rand(w.hq, device="cuda", generator=g) * 10 - 2
    gate = torch.randn(out.shape, device="cuda", generator=g).to(torch.bfloat16)
    r = {"workload": w.name, "rope": "YaRN theta 500000 factor 64 (orig 4096, beta 64/1) + RMSNorm"}
    log("prologue/epilogue: timing")
    ms = timer.run(lambda i: G.attn_prefill(layer, qd, kd, vd, out, q_prologue=pq), warmup, steps)
    r["prefill_q_prologue"] = {"ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "over_plain": ms / base_ms}
    ms = timer.run(lambda i: G.attn_prefill(layer, qd, kd, vd, out, sink_logits=sink, gate=gate), warmup, steps)
    r["prefill_sink_gate"] = {"ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12, "over_plain": ms / base_ms}
    sp = torch.zeros(B, dtype=torch.int32, device="cuda")
    y = torch.empty_like(qd)
    for name, x, yy in (("qk_prologue_q", qd, y), ("qk_prologue_k", kd, torch.empty_like(kd))):
        ms = timer.run(lambda i: G.qk_prologue(pk, x, sp, yy), warmup, steps)
        nb = 2 * x.numel() * 2
        r[name] = {"shape": list(x.shape), "ms": ms, "bytes": nb, "GB/s": nb / (ms * 1e-3) / 1e9,
                   "frac_hbm_peak": nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    cache = G.KVCache(layer, B, T, zero=False)
    nb = 4 * kd.numel() * 2          # read K and V, write K and V
    for name, pro in (("kv_append_plain", None), ("kv_append_k_prologue", pk)):
        ms = timer.run(lambda i: G.kv_append(layer, cache, kd, vd, sp, max_end_pos=T, k_prologue=pro),
                       warmup, steps)
        r[name] = {"ms": ms, "bytes": nb, "GB/s": nb / (ms * 1e-3) / 1e9}
    return r


def bench_decode_sliding(torch, G, wl, timer, warmup, steps, replicas=8):
    w = wl.WORKLOADS[3]
    layer = G.Layer(kind=G.SLIDING, window=w.window)
    L = wl.context_lengths(w)
    log(f"decode workload {w.name}: filling {replicas} ring replicas")
    lows = np.maximum(0, L - w.window)
    ks = wl.normal_tokens_ragged(w.seed, wl.K, lows.tolist(), (L - lows).tolist(), w.hkv, 128)
    vs = wl.normal_tokens_ragged(w.seed, wl.V, lows.tolist(), (L - lows).tolist(), w.hkv, 128)
    kb = dev_bits(torch, np.stack(ks))
    vb = dev_bits(torch, np.stack(vs))
    caches = []
    sp = torch.tensor(lows, dtype=torch.int32, device="cuda")
    for r in range(replicas):
        c = G.KVCache(layer, w.batch, w.window, zero=False)
        G.kv_append(layer, c, kb, vb, sp, max_end_pos=int(L.max()))
        caches.append(c)
    q = dev_bits(torch, wl.decode_queries(w.seed, w.batch, w.hq, 128))
    out = torch.empty_like(q)
    sl = torch.tensor(L, dtype=torch.int32, device="cuda")
    maxlen = int(L.max())
    ws = G.decode_workspace(layer, w.batch, maxlen)
    nbytes = int(sum(min(int(x), w.window) for x in L)) * w.hkv * 128 * 2 * 2
    log("decode sliding: timing")
    ms = timer.run(lambda i: G.attn_decode(layer, caches[i % replicas], q, sl, maxlen, out, ws), warmup, steps)
    stats = dict(timer.last)
    pro = G.Prologue(norm_weight=torch.ones(128, device="cuda"), rope=G.Rope())
    ms_pro = timer.run(lambda i: G.attn_decode(layer, caches[i % replicas], q, sl, maxlen, out, ws, q_prologue=pro),
                       warmup, steps)
    timer.last = stats
    return w, nbytes, ms, replicas, ms_pro


def bench_decode_duo(torch, G, wl, timer, warmup, steps, replicas=2):
    w = wl.WORKLOADS[4]
    mask = wl.duo_mask(w).tolist()
    layer = G.Layer(full_attention_heads=mask)
    L = wl.context_lengths(w)
    log(f"decode workload {w.name}: mask {mask}, filling {replicas} cache replicas")
    gen = torch.Generator(device="cuda")
    chunk = 16384
    caches = [G.KVCache(layer, w.batch, w.len_hi, zero=False) for _ in range(replicas)]
    for b in range(w.batch):
        for p in range(0, int(L[b]), chunk):
            T = min(chunk, int(L[b]) - p)
            gen.manual_seed(w.seed * 1000003 + b * 1009 + p)
            kc = torch.randn((1, T, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
            vc = torch.randn((1, T, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
            sp = torch.tensor([p], dtype=torch.int32, device="cuda")
            for c in caches:
                G.kv_append(layer, c, kc, vc, sp, max_end_pos=p + T, batch=1, batch_offset=b)
    q = dev_bits(torch, wl.decode_queries(w.seed, w.batch, w.hq, 128))
    out = torch.empty_like(q)
    sl = torch.tensor(L, dtype=torch.int32, device="cuda")
    ws = G.decode_workspace(layer, w.batch, w.len_hi)
    nf = sum(1 for m in mask if m)
    ns = w.hkv - nf
    sr = w.sink + w.recent
    nbytes = int(sum(nf * int(x) + ns * min(int(x), sr) for x in L)) * 128 * 2 * 2
    log("decode duo: timing")
    ms = timer.run(lambda i: G.attn_decode(layer, caches[i % replicas], q, sl, w.len_hi, out, ws), warmup, steps)
    stats = dict(timer.last)
    # block decode (verify blocks of T tokens after the same cached contexts):
    # algorithmic bytes = the visible cached K/V rows (every full-head
    # position, the whole sink + recent cache of a streaming head) plus the
    # block's own K/V
    block = {}
    gen.manual_seed(w.seed * 7919)
    for T in (4, 6, 8):
        qb = torch.randn((w.batch, T, w.hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
        kb = torch.randn((w.batch, T, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
        vb = torch.randn((w.batch, T, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
        ob = torch.empty_like(qb)
        wsb = G.decode_block_workspace(layer, w.batch, T, w.len_hi)
        nb = nbytes + w.batch * w.hkv * T * 128 * 2 * 2
        log(f"decode block T={T}: timing")
        msb = timer.run(lambda i: G.attn_decode_block(layer, caches[i % replicas], qb, kb, vb, sl, w.len_hi, ob, wsb),
                        warmup, steps)
        block[f"T{T}"] = {"ms": msb, "kv_bytes": nb, "GB/s": nb / (msb * 1e-3) / 1e9,
                          "frac_hbm_peak": nb / (msb * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "ms_median": timer.last["median_ms"], "ms_min": timer.last["min_ms"]}
    timer.last = stats
    return w, nbytes, ms, replicas, mask, int(L.sum()), block


def bench_chunked(torch, G, wl, timer, warmup, steps):
    w = wl.WORKLOADS[5]
    mask = wl.duo_mask(w).tolist()
    layer = G.Layer(full_attention_heads=mask)
    log(f"chunked prefill workload {w.name}: mask {mask}, generating inputs on the GPU")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(w.seed)
    n_chunks = w.seq // w.chunk
    q = torch.randn((n_chunks, 1, w.chunk, w.hq, 128), generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.randn((n_chunks, 1, w.chunk, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
    v = torch.randn((n_chunks, 1, w.chunk, w.hkv, 128), generator=gen, device="cuda").to(torch.bfloat16)
    out = torch.empty((n_chunks, 1, w.chunk, w.hq, 128), dtype=torch.bfloat16, device="cuda")
    cache = G.KVCache(layer, 1, w.seq, zero=False)
    starts = [torch.tensor([c * w.chunk], dtype=torch.int32, device="cuda") for c in range(n_chunks)]
    flops = sum(prefill_flops(G, layer, 1, w.chunk, c * w.chunk) for c in range(n_chunks))
    # one prefill workspace for every chunk: the library cuts the full-context
    # query tiles of a chunk over a long past into key-range pieces
    ws = G.prefill_workspace(layer, 1, w.chunk, [c * w.chunk for c in range(n_chunks)])
    pieces = [int(G.prefill_plan(layer, 1, w.chunk, c * w.chunk, True)[:, 5].max()) for c in range(n_chunks)]

    def one_pass(_):
        for c in range(n_chunks):
            G.attn_prefill(layer, q[c], k[c], v[c], out[c], start_pos=c * w.chunk, past=cache, workspace=ws)
            G.kv_append(layer, cache, k[c], v[c], starts[c], max_end_pos=(c + 1) * w.chunk)

    # attention alone: the 16 prefill calls of a pass without their appends
    # (the cache already holds every position)
    def attend_only(_):
        for c in range(n_chunks):
            G.attn_prefill(layer, q[c], k[c], v[c], out[c], start_pos=c * w.chunk, past=cache, workspace=ws)

    # The two kinds of pass alternate, each between its own event pair, so
    # that clock drift over the run does not favour whichever is timed first
    # (the appends are 16 short kernels, about 0.3% of a pass).
    log("chunked prefill: timing passes (attend + append, attention alone, interleaved)")
    for i in range(warmup):
        one_pass(i)
        attend_only(i)
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps + 1)]
    ev[0].record(s)
    for i in range(steps):
        one_pass(i)
        ev[2 * i + 1].record(s)
        attend_only(i)
        ev[2 * i + 2].record(s)
    torch.cuda.synchronize()
    tot = sorted(ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps))
    att = sorted(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(steps))
    ms = sum(tot) / steps
    attn_ms = sum(att) / steps
    pass_stats = {"median_ms": tot[steps // 2], "min_ms": tot[0], "passes": steps,
                  "attention_only_median_ms": att[steps // 2], "attention_only_min_ms": att[0]}
    # cache manager on one chunk: read 2 x chunk rows, write 2 x chunk rows
    app_ms = timer.run(lambda i: G.kv_append(layer, cache, k[0], v[0], starts[0], max_end_pos=w.chunk), 2,
                       SHORT_CALLS)
    app_bytes = 2 * 2 * w.chunk * w.hkv * 128 * 2
    ws_bytes = 0 if ws is None else ws.numel() * 4
    return w, mask, flops, ms, attn_ms, app_ms, app_bytes, pass_stats, pieces, ws_bytes


def bench_copy(torch, timer, warmup, steps, nbytes=1 << 30):
    """A plain device copy of a known size: the reference that scales the
    FETCH_SIZE / WRITE_SIZE counters of the attention kernels to bytes."""
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = timer.run(lambda i: dst.copy_(src), warmup, steps)
    return {"bytes_read": nbytes, "bytes_written": nbytes, "ms": ms, "GB/s": 2 * nbytes / (ms * 1e-3) / 1e9}


def kv_cache_section(G, wl):
    """Static-cache footprint of the two Duo workloads beside the same layer
    without Duo routing (host-side accounting, no GPU time)."""
    out = {}
    for idx in (4, 5):
        w = wl.WORKLOADS[idx]
        mask = wl.duo_mask(w).tolist()
        layer = G.Layer(full_attention_heads=mask)
        if w.kind == "decode":
            cap, L = w.len_hi, wl.context_lengths(w)
        else:
            cap, L = w.seq, np.array([w.seq] * w.batch)
        r = G.kv_cache_report(layer, w.batch, cap, L)
        duo = r["main_bytes"] + r["stream_bytes"]
        out[w.name] = {"mask": mask, "capacity": cap, "duo_bytes": duo, "base_bytes": r["base_bytes"],
                       "duo_over_base": duo / r["base_bytes"],
                       "occupied_over_allocated": (r["main_active"] + r["stream_active"]) /
                                                  (r["main_slots"] + r["stream_slots"]),
                       "base_occupied_over_allocated": r["base_active"] / r["base_slots"]}
    return out


def kernel_source_hash() -> str:
    """Hash of the prefill kernel's sources: profile counters taken for another
    version of the kernel are not reported."""
    import hashlib
    h = hashlib.sha256()
    for f in ("prefill.hip", "duo_internal.h", "mfma_common.h", "qk_prologue.h"):
        h.update(open(os.path.join(HERE, "gqa_sliding_window_amd", "csrc", f), "rb").read())
    from gqa_sliding_window_amd import build as B
    flags = [f for f in B.common_flags() + B.SOURCE_FLAGS.get("prefill.hip", []) if not f.startswith("-I")]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


# Legs whose call takes well under a millisecond (the decodes, the verify
# blocks, the 1 x 1024 prefill, the append) time at least this many
# back-to-back calls between one event pair: the host submits the first call
# only after the start event, and over 20 calls that latency (about 30 us)
# added about 1.4 us to each 25 us decode call.
SHORT_CALLS = 200

ORACLE_ROWS = 1 << 19  # sample of the headline workload drawn for the oracle baseline


def oracle_worker(idx: int, nproc: int, target_s: float):
    """One process of the oracle baseline: the sampled rows of the (batch,
    KV head) groups g with g % nproc == idx, in random order within each
    group, until target_s seconds of oracle time have passed. Prints one JSON
    line (rows, FLOP, seconds). Inputs are regenerated from the workload's
    seeds for the batch rows this process needs."""
    import threadpoolctl
    import oracle
    import workloads as wl
    w = wl.WORKLOADS[2]
    G = w.hq // w.hkv
    rows = wl.sample_query_rows(w, w.seq, ORACLE_ROWS)
    grp = rows[:, 0] * w.hkv + rows[:, 1] // G
    mine = [g for g in range(w.batch * w.hkv) if g % nproc == idx]
    rng = np.random.default_rng(idx)
    done = flops = 0
    spent = 0.0
    with threadpoolctl.threadpool_limits(1):
        for g in mine:
            b = g // w.hkv
            counts = [w.seq if i == b else 0 for i in range(w.batch)]
            qb = np.stack([x if len(x) else np.zeros((w.seq, w.hq, 128), np.uint16) for x in
                           wl.normal_tokens_ragged(w.seed, wl.Q, [0] * w.batch, counts, w.hq, 128, threads=1)])
            kb = np.stack([x if len(x) else np.zeros((w.seq, w.hkv, 128), np.uint16) for x in
                           wl.normal_tokens_ragged(w.seed, wl.K, [0] * w.batch, counts, w.hkv, 128, threads=1)])
            vb = np.stack([x if len(x) else np.zeros((w.seq, w.hkv, 128), np.uint16) for x in
                           wl.normal_tokens_ragged(w.seed, wl.V, [0] * w.batch, counts, w.hkv, 128, threads=1)])
            sel = rows[grp == g]
            sel = sel[rng.permutation(len(sel))]
            t0 = time.perf_counter()
            for s0 in range(0, len(sel), 16):
                part = sel[s0:s0 + 16]
                oracle.prefill_rows(qb, kb, vb, 0, part, hkv=w.hkv, layer="full")
                flops += int(4 * 128 * (part[:, 2] + 1).sum())
                done += len(part)
                if spent + time.perf_counter() - t0 >= target_s:
                    break
            spent += time.perf_counter() - t0
            if spent >= target_s:
                break
    print(json.dumps({"rows": done, "flop": flops, "seconds": spent}), flush=True)


def cpu_baseline(target_s, total_flop):
    """Time the float64 oracle on the host cores: one single-threaded process
    per core of this process's CPU set (at most 16, the host share of one
    GPU), each taking the sampled rows of its own (batch, KV head) groups.
    Reports the aggregate rate and, labelled as such, its extrapolation to
    the whole headline workload."""
    import subprocess
    affinity = len(os.sched_getaffinity(0))
    nproc = max(1, min(16, affinity))
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1")
    procs = [subprocess.Popen([sys.executable, os.path.abspath(__file__), "--oracle-worker", str(i), str(nproc),
                               str(target_s)], stdout=subprocess.PIPE, env=env, cwd=HERE) for i in range(nproc)]
    res = []
    for p in procs:
        out, _ = p.communicate()
        if p.returncode != 0:
            raise RuntimeError(f"oracle worker failed with status {p.returncode}")
        res.append(json.loads(out.decode().strip().splitlines()[-1]))
    rows = sum(r["rows"] for r in res)
    flops = sum(r["flop"] for r in res)
    rate = sum(r["flop"] / r["seconds"] for r in res if r["seconds"] > 0)
    secs = max(r["seconds"] for r in res)
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": nproc, "kind": "oracle",
            "sample": f"{rows} seeded query rows of the headline workload, float64, {nproc} single-threaded "
                      f"processes split by (batch, KV head), {secs:.1f} s each",
            "host_cpus_in_affinity": affinity, "rows_per_s": rows / secs, "flop": flops,
            "extrapolated_full_workload_s": total_flop / rate,
            "extrapolation": "the headline workload's algorithmic FLOP divided by the sampled rate"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sections", default="prefill,sliding,swa,prologue,decode,chunked",
                    help="comma list of prefill, sliding and prologue (both need prefill), swa (the 1 x 1024 "
                         "sliding prefill), decode, chunked, "
                         "copy (copy = counter calibration: a plain 1 GiB device copy)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--oracle-worker", nargs=3, metavar=("IDX", "NPROC", "SECONDS"), help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.oracle_worker:
        i, n, t = args.oracle_worker
        oracle_worker(int(i), int(n), float(t))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this path runs without sharding or collectives; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_sliding_window_amd as G
    import workloads as wl
    G.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    timer = Timer(torch)
    sections = set(args.sections.split(","))
    short_steps = max(args.steps, SHORT_CALLS)
    res = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16)"}

    w2 = qkv = devs = None
    if "prefill" in sections:
        w2, qkv, flops, ms, devs = bench_prefill(torch, G, wl, timer, args.warmup, args.steps)
        tflops = flops / (ms * 1e-3) / 1e12
        res["value"] = tflops
        res["ms_per_step"] = ms
        res["ms_per_step_median"] = timer.last["median_ms"]
        res["ms_per_step_min"] = timer.last["min_ms"]
        res["config"] = {"workload": w2.name, "batch": w2.batch, "seq_len": w2.seq, "q_heads": w2.hq,
                         "kv_heads": w2.hkv, "head_dim": 128, "layer": "full causal",
                         "algorithmic_flop_per_step": flops}
        traffic = None
        if os.path.exists(TRAFFIC_FILE):
            t = json.load(open(TRAFFIC_FILE)).get("prefill_kernel")
            if t and t.get("workload") == w2.name and t.get("source_hash") == kernel_source_hash():
                traffic = t.get("bytes_per_launch")
        res["roofline"] = {"kernel": "prefill_kernel", "bound": "mfma", "achieved": tflops,
                           "peak": PEAK_MFMA_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / PEAK_MFMA_BF16_TFLOPS, "traffic": traffic,
                           "frac_of_measured_ceiling": tflops / MEASURED_MFMA_BF16_TFLOPS}
        log(f"prefill: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
    if "sliding" in sections and devs is not None:
        # the same shape on a 512-token sliding-window layer (30 of the model's
        # 40 layers are of this kind)
        layer_s = G.Layer(kind=G.SLIDING, window=512)
        fl_s = prefill_flops(G, layer_s, w2.batch, w2.seq)
        lq, qd_, kd_, vd_, od_ = devs
        ms_s = timer.run(lambda i: G.attn_prefill(layer_s, qd_, kd_, vd_, od_), args.warmup, args.steps)
        res["sliding_prefill"] = {"workload": w2.name + " on a sliding-window layer (w 512)",
                                  "algorithmic_flop": fl_s, "ms": ms_s,
                                  "TFLOP/s": fl_s / (ms_s * 1e-3) / 1e12,
                                  "ms_median": timer.last["median_ms"], "ms_min": timer.last["min_ms"]}
        log(f"sliding prefill: {ms_s:.3f} ms, {res['sliding_prefill']['TFLOP/s']:.1f} TFLOP/s")
    if "swa" in sections:
        res["swa_prefill"] = bench_swa_prefill(torch, G, wl, timer, args.warmup, short_steps)
        res["swa_prefill"]["timed_calls"] = short_steps
        log(f"swa prefill (1x1024, 12/2 heads, w 512): {res['swa_prefill']['ms'] * 1e3:.1f} us")
    if "prologue" in sections and devs is not None:
        res["prologue_epilogue"] = bench_prologue_epilogue(torch, G, wl, timer, args.warmup, args.steps, w2,
                                                           flops, ms, devs)
    devs = None

    if "decode" in sections:
        d = {}
        d["timed_calls"] = short_steps
        w3, nb3, ms3, rep3, ms3p = bench_decode_sliding(torch, G, wl, timer, args.warmup, short_steps)
        gbs3 = nb3 / (ms3 * 1e-3) / 1e9
        d["sliding_window"] = {"workload": w3.name, "kv_bytes": nb3, "ms": ms3, "GB/s": gbs3,
                               "frac_hbm_peak": gbs3 / PEAK_HBM_GBS,
                               "frac_of_measured_ceiling": gbs3 / MEASURED_DECODE_READ_GBS, "cache_replicas": rep3,
                               "ms_median": timer.last["median_ms"], "ms_min": timer.last["min_ms"],
                               "ms_with_q_prologue": ms3p}
        log(f"decode sliding: {ms3 * 1e3:.1f} us, {gbs3:.0f} GB/s")
        w4, nb4, ms4, rep4, mask4, sumL, blk4 = bench_decode_duo(torch, G, wl, timer, args.warmup, short_steps)
        gbs4 = nb4 / (ms4 * 1e-3) / 1e9
        d["duo"] = {"workload": w4.name, "mask": mask4, "sum_context": sumL, "kv_bytes": nb4, "ms": ms4,
                    "GB/s": gbs4, "frac_hbm_peak": gbs4 / PEAK_HBM_GBS,
                    "frac_of_measured_ceiling": gbs4 / MEASURED_DECODE_READ_GBS, "cache_replicas": rep4,
                    "ms_median": timer.last["median_ms"], "ms_min": timer.last["min_ms"]}
        log(f"decode duo: {ms4 * 1e3:.1f} us, {gbs4:.0f} GB/s")
        d["duo_block"] = {"workload": w4.name + " (past = the contexts; verify blocks of T tokens)", **blk4}
        res["decode"] = d

    if "chunked" in sections:
        w5, mask5, fl5, ms5, attn5, app_ms, app_bytes, st5, pieces5, ws5 = bench_chunked(
            torch, G, wl, timer, 1, max(3, args.steps // 4))
        res["chunked_prefill"] = {"workload": w5.name, "mask": mask5, "algorithmic_flop": fl5,
                                  "ms_total": ms5, "TFLOP/s": fl5 / (ms5 * 1e-3) / 1e12,
                                  "ms_total_median": st5["median_ms"], "ms_total_min": st5["min_ms"],
                                  "pieces_per_chunk": pieces5, "prefill_workspace_bytes": ws5,
                                  "attention_only_ms": attn5,
                                  "attention_only_ms_median": st5["attention_only_median_ms"],
                                  "passes_each": st5["passes"],
                                  "attention_only_TFLOP/s": fl5 / (attn5 * 1e-3) / 1e12}
        res["kv_append"] = {"workload": "one 8192-token chunk, 8 KV heads", "ms": app_ms, "timed_calls": SHORT_CALLS,
                            "GB/s": app_bytes / (app_ms * 1e-3) / 1e9}
        log(f"chunked prefill: {ms5:.2f} ms total, attention {attn5:.2f} ms")

    if "decode" in sections or "chunked" in sections:
        res["kv_cache"] = kv_cache_section(G, wl)

    if "copy" in sections:
        res["copy_reference"] = bench_copy(torch, timer, args.warmup, args.steps)
        log(f"copy reference: {res['copy_reference']['GB/s']:.0f} GB/s")

    if w2 is not None and args.cpu_seconds > 0:
        log("cpu baseline: timing the oracle")
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds, res["config"]["algorithmic_flop_per_step"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
