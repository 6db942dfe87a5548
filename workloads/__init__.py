"""Seeded synthetic inputs for the attention workloads (shared by the oracle and
the HIP path; contains none of the attention arithmetic).

Shapes follow the Laguna-XS-2.1 geometry (48 query heads, 8 KV heads, window
512; SGLang cookbook "Laguna-XS-2.1", section 1 "Model Introduction") and the
DuoAttention adapter's sink 64 / recent 256 (Hugging Face card "DuoAttention
Laguna Adapter", section "Summary"). head_dim is 128 (the pages give none).

Recipe (stated once, used everywhere):
  * each workload has a master seed; ``numpy.random.SeedSequence(seed)`` is
    split into four children: values, context lengths, Duo mask, oracle rows;
  * tensor values are N(0, 1) float32 from PCG64, generated in independent
    blocks keyed by (tensor id, batch index, block index) so any block can be
    regenerated alone and blocks can be generated in parallel threads;
  * float32 -> bfloat16 is round-to-nearest-even on the bit pattern;
  * context lengths are integers uniform in [lo, hi], inclusive at both ends;
  * the Duo mask is one Bernoulli(p) draw per KV head, never redrawn;
  * the output gate's values are N(0, 1) bf16 like Q/K/V (tensor id GATE);
    attention-sink logits are float32 uniform in [-2, 8] per query head (the
    pages give no values for either: the range runs from a sink that barely
    matters to one that outweighs a few thousand keys).
Every array handed out is ``uint16`` holding bfloat16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# tensor ids used to key value blocks (GATE: the output-gate values)
Q, K, V, GATE = 0, 1, 2, 3
BLOCK_TOKENS = 1024


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str            # "prefill" | "decode" | "chunked_prefill"
    layer: str           # "full" | "sliding"
    batch: int
    hq: int
    hkv: int
    d: int = 128
    window: int = 0      # sliding-layer window, 0 = none
    sink: int = 64
    recent: int = 256
    duo: bool = False    # per-KV-head routing mask drawn from Bernoulli(mask_p)
    mask_p: float = 0.25
    seq: int = 0         # prefill length / total tokens of the chunked prefill
    chunk: int = 0       # chunk length of the chunked prefill
    len_lo: int = 0      # decode context length range (inclusive)
    len_hi: int = 0
    oracle_rows: int = 0  # 0 = every query row

    @property
    def group(self) -> int:
        return self.hq // self.hkv


WORKLOADS = {
    1: Workload("swa_prefill_b1_h12kv2_s1024_w512", 1, "prefill", "sliding", 1, 12, 2,
                window=512, seq=1024),
    2: Workload("full_prefill_b4_h48kv8_s8192", 2, "prefill", "full", 4, 48, 8,
                seq=8192, oracle_rows=4096),
    3: Workload("swa_decode_b64_h48kv8_w512_len512-32768", 3, "decode", "sliding", 64, 48, 8,
                window=512, len_lo=512, len_hi=32768),
    4: Workload("duo_decode_b16_h48kv8_len32768-131072", 4, "decode", "full", 16, 48, 8,
                duo=True, len_lo=32768, len_hi=131072),
    5: Workload("duo_chunked_prefill_b1_h48kv8_s131072_c8192", 5, "chunked_prefill", "full", 1, 48, 8,
                duo=True, seq=131072, chunk=8192, oracle_rows=4096),
}


def _children(seed: int):
    return np.random.SeedSequence(seed).spawn(4)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_rng(seed: int, tensor: int, b: int, blk: int) -> np.random.Generator:
    vals = _children(seed)[0]
    ss = np.random.SeedSequence(vals.entropy, spawn_key=vals.spawn_key + (tensor, b, blk))
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_tokens(seed: int, tensor: int, batch: int, pos0: int, ntok: int, heads: int, d: int,
                  threads: int | None = None) -> np.ndarray:
    """bf16 bits of shape [batch, ntok, heads, d] for token positions
    [pos0, pos0 + ntok). Position p of batch row b always gets the same value,
    whichever window of positions is asked for."""
    out = np.empty((batch, ntok, heads, d), dtype=np.uint16)
    if ntok == 0 or batch == 0:
        return out
    b0, b1 = pos0 // BLOCK_TOKENS, (pos0 + ntok - 1) // BLOCK_TOKENS
    jobs = [(b, blk) for b in range(batch) for blk in range(b0, b1 + 1)]

    def run(job):
        b, blk = job
        g = _block_rng(seed, tensor, b, blk)
        vals = g.standard_normal((BLOCK_TOKENS, heads, d), dtype=np.float32)
        lo = max(pos0, blk * BLOCK_TOKENS)
        hi = min(pos0 + ntok, (blk + 1) * BLOCK_TOKENS)
        out[b, lo - pos0:hi - pos0] = f32_to_bf16_bits(vals[lo - blk * BLOCK_TOKENS:hi - blk * BLOCK_TOKENS])

    nt = threads or _threads()
    if nt == 1 or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, jobs))
    return out


def normal_tokens_ragged(seed: int, tensor: int, starts, counts, heads: int, d: int,
                         threads: int | None = None) -> list:
    """Per batch row b: bf16 bits [counts[b], heads, d] for positions
    [starts[b], starts[b] + counts[b]); identical values to normal_tokens."""
    res = [np.empty((c, heads, d), dtype=np.uint16) for c in counts]
    jobs = [(b, blk) for b, (s, c) in enumerate(zip(starts, counts)) if c > 0
            for blk in range(s // BLOCK_TOKENS, (s + c - 1) // BLOCK_TOKENS + 1)]

    def run(job):
        b, blk = job
        s, c = starts[b], counts[b]
        g = _block_rng(seed, tensor, b, blk)
        vals = g.standard_normal((BLOCK_TOKENS, heads, d), dtype=np.float32)
        lo, hi = max(s, blk * BLOCK_TOKENS), min(s + c, (blk + 1) * BLOCK_TOKENS)
        res[b][lo - s:hi - s] = f32_to_bf16_bits(vals[lo - blk * BLOCK_TOKENS:hi - blk * BLOCK_TOKENS])

    nt = threads or _threads()
    if nt == 1 or len(jobs) <= 1:
        for j in jobs:
            run(j)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(run, jobs))
    return res


def decode_queries(seed: int, batch: int, hq: int, d: int) -> np.ndarray:
    """bf16 bits [batch, hq, d]: the one query token of each sequence."""
    return normal_tokens(seed, Q, batch, 0, 1, hq, d)[:, 0]


def context_lengths(w: Workload) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(_children(w.seed)[1]))
    return g.integers(w.len_lo, w.len_hi, size=w.batch, endpoint=True).astype(np.int64)


def duo_mask(w: Workload) -> np.ndarray:
    """uint8[hkv]: 1 = full-context KV head, 0 = streaming head."""
    g = np.random.Generator(np.random.PCG64(_children(w.seed)[2]))
    return (g.random(w.hkv) < w.mask_p).astype(np.uint8)


def rows_rng(w: Workload) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_children(w.seed)[3]))


def sample_query_rows(w: Workload, n_tokens: int, count: int, must=(), chunk: int = 0):
    """Seeded (b, h, i) query rows: ``count`` rows, always including positions
    in ``must`` (clipped to the range) and, when ``chunk`` > 0, the first and
    last row of every chunk. Returns an int64 array [n, 3], sorted."""
    g = rows_rng(w)
    forced = {p for p in must if 0 <= p < n_tokens}
    if chunk:
        for c0 in range(0, n_tokens, chunk):
            forced.add(c0)
            forced.add(min(n_tokens, c0 + chunk) - 1)
    rows = set()
    forced = sorted(forced)
    for idx, p in enumerate(forced):
        rows.add((int(g.integers(w.batch)), int(g.integers(w.hq)), p))
    while len(rows) < count:
        rows.add((int(g.integers(w.batch)), int(g.integers(w.hq)), int(g.integers(n_tokens))))
    return np.array(sorted(rows), dtype=np.int64).reshape(-1, 3)


def sink_logits(seed: int, hq: int) -> np.ndarray:
    """float32 [hq]: one attention-sink logit per query head."""
    ss = np.random.SeedSequence(seed, spawn_key=(GATE, 1))
    return np.random.Generator(np.random.PCG64(ss)).uniform(-2.0, 8.0, size=hq).astype(np.float32)
