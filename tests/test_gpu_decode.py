"""duo_attn_decode (split-K partials + merge) against the float64 oracle.

Caches are filled by duo_kv_append from seeded K/V; the oracle reads the same
K/V by absolute position (never from the GPU caches)."""
import zlib

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, bits_to_f64, check_close, dev, host_bits

pytestmark = pytest.mark.gpu


class Seqs:
    """Seeded K/V per sequence for positions [lo_b, L_b)."""

    def __init__(self, seed, lengths, lows, hkv):
        self.seed, self.L, self.lo, self.hkv = seed, list(lengths), list(lows), hkv
        cnt = [L - lo for L, lo in zip(self.L, self.lo)]
        self.k = wl.normal_tokens_ragged(seed, wl.K, self.lo, cnt, hkv, 128)
        self.v = wl.normal_tokens_ragged(seed, wl.V, self.lo, cnt, hkv, 128)

    def kv_of(self, b, kvh, pos):
        idx = np.asarray(pos) - self.lo[b]
        assert (idx >= 0).all(), "oracle asked for a position that was never generated"
        return self.k[b][idx, kvh], self.v[b][idx, kvh]


def fill_cache(lib, layer, cache, seqs, chunk=1 << 20):
    import torch
    for b in range(len(seqs.L)):
        lo, L = seqs.lo[b], seqs.L[b]
        for p in range(lo, L, chunk):
            T = min(chunk, L - p)
            kd = dev(seqs.k[b][p - lo:p - lo + T][None])
            vd = dev(seqs.v[b][p - lo:p - lo + T][None])
            sp = torch.tensor([p], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, kd, vd, sp, max_end_pos=p + T, batch=1, batch_offset=b)
    torch.cuda.synchronize()


def run_decode(lib, layer, cache, q, lengths, max_len, ws=None):
    import torch
    B, hq, _ = q.shape
    ws = lib.decode_workspace(layer, B, max_len) if ws is None else ws
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    lib.attn_decode(layer, cache, dev(q), sl, max_len, out, ws, lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), lse.cpu().numpy()


def check_decode(layer, q, seqs, out, lse, what, **tol):
    B, hq, _ = q.shape
    rows = [(b, h) for b in range(B) for h in range(hq) if seqs.L[b] > 0]
    o_ref, l_ref = oracle.decode_rows(q, seqs.kv_of, np.asarray(seqs.L), rows,
                                      hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                                      window=layer.window, sink=layer.sink, recent=layer.recent,
                                      full_attention_heads=layer.full_attention_heads)
    r = np.asarray(rows)
    check_close(bits_to_f64(out[r[:, 0], r[:, 1]]), o_ref, what, **tol)
    err = np.abs(lse[r[:, 0], r[:, 1]] - l_ref).max()
    assert err < 1e-3, f"{what}: lse error {err}"


def lows_for(layer, lengths):
    """First position a decode can see: the window/ring start for sliding layers
    (the workload fills only the last W positions), else 0."""
    if layer.main_ring and layer.full_attention_heads is None:
        return [max(0, L - layer.window) for L in lengths]
    return [0] * len(lengths)


def test_sliding_decode_workload(lib):
    """Batch 64, 48/8 heads, window 512 ring, context lengths U[512, 32768]:
    every row against the oracle."""
    w = wl.WORKLOADS[3]
    announce(f"decode parity {w.name}")
    layer = lib.Layer(kind=1, window=w.window)
    L = wl.context_lengths(w).tolist()
    seqs = Seqs(w.seed, L, lows_for(layer, L), w.hkv)
    cache = lib.KVCache(layer, w.batch, w.window)
    fill_cache(lib, layer, cache, seqs)
    q = wl.decode_queries(w.seed, w.batch, w.hq, 128)
    out, lse = run_decode(lib, layer, cache, q, L, max(L))
    check_decode(layer, q, seqs, out, lse, w.name)


def test_duo_decode_workload(lib):
    """Batch 16, 48/8 heads, contexts U[32768, 131072], Bernoulli(0.25) Duo
    mask: every row against the oracle."""
    w = wl.WORKLOADS[4]
    announce(f"decode parity {w.name}")
    mask = wl.duo_mask(w).tolist()
    layer = lib.Layer(full_attention_heads=mask)
    L = wl.context_lengths(w).tolist()
    seqs = Seqs(w.seed, L, [0] * w.batch, w.hkv)
    cache = lib.KVCache(layer, w.batch, w.len_hi, zero=False)
    fill_cache(lib, layer, cache, seqs, chunk=32768)
    q = wl.decode_queries(w.seed, w.batch, w.hq, 128)
    ws = lib.decode_workspace(layer, w.batch, w.len_hi)
    out, lse = run_decode(lib, layer, cache, q, L, w.len_hi, ws)
    check_decode(layer, q, seqs, out, lse, w.name)
    # split-K arrival counters are back at zero: a second call on the same
    # workspace gives the same bits
    out2, lse2 = run_decode(lib, layer, cache, q, L, w.len_hi, ws)
    np.testing.assert_array_equal(out2, out)


SMALL = {
    # lengths straddling sink, sink+recent, window; single-token sequences
    "duo_short": (dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 1, 0]), [1, 2, 63, 64, 65, 319, 320, 321, 700, 3000]),
    "sliding_short": (dict(kind=1, window=512), [1, 5, 511, 512, 513, 1200]),
    "full_ragged": (dict(num_q_heads=12, num_kv_heads=2), [1, 100, 4097, 9000]),
    "all_streaming": (dict(full_attention_heads=[0, 0], num_q_heads=12, num_kv_heads=2, sink=3, recent=5),
                      [1, 4, 8, 9, 100]),
    "group16": (dict(num_q_heads=16, num_kv_heads=1), [1, 300, 1000]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_small(lib, name):
    kw, L = SMALL[name]
    announce(f"decode parity {name}")
    layer = lib.Layer(**kw)
    seqs = Seqs(zlib.crc32(name.encode()) % 1000, L, lows_for(layer, L), layer.num_kv_heads)
    big = max(L) * 8 + 1000
    cache = lib.KVCache(layer, len(L), big)
    fill_cache(lib, layer, cache, seqs, chunk=257)
    q = wl.decode_queries(zlib.crc32(name.encode()) % 1000 + 1, len(L), layer.num_q_heads, 128)
    out, lse = run_decode(lib, layer, cache, q, L, max(L))
    check_decode(layer, q, seqs, out, lse, name)
    # a larger max_seq_len hint changes the split plan, not the result; the
    # second call on the same workspace checks the counters were reset
    ws = lib.decode_workspace(layer, len(L), big)
    for _ in range(2):
        out2, lse2 = run_decode(lib, layer, cache, q, L, big, ws)
        d = np.abs(bits_to_f64(out2) - bits_to_f64(out)).max()
        assert d <= 1.6e-2, d


def test_zero_length_rows(lib):
    announce("decode zero-length rows")
    layer = lib.Layer(num_q_heads=12, num_kv_heads=2)
    L = [0, 10, 0]
    seqs = Seqs(5, L, [0, 0, 0], 2)
    cache = lib.KVCache(layer, 3, 16)
    fill_cache(lib, layer, cache, seqs)
    q = wl.decode_queries(6, 3, 12, 128)
    out, lse = run_decode(lib, layer, cache, q, L, 16)
    assert (out[0] == 0).all() and (out[2] == 0).all()
    assert np.isneginf(lse[0]).all() and np.isneginf(lse[2]).all()
    check_decode(layer, q, seqs, out, lse, "zero_length_neighbour")


def test_decode_equals_prefill_last_row(lib):
    import torch
    announce("decode == prefill last row")
    layer = lib.Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 1])
    N = 1500
    q = wl.normal_tokens(41, wl.Q, 1, 0, N, 48, 128)
    k = wl.normal_tokens(41, wl.K, 1, 0, N, 8, 128)
    v = wl.normal_tokens(41, wl.V, 1, 0, N, 8, 128)
    out = torch.empty((1, N, 48, 128), dtype=torch.bfloat16, device="cuda")
    lib.attn_prefill(layer, dev(q), dev(k), dev(v), out)
    cache = lib.KVCache(layer, 1, N)
    lib.kv_append(layer, cache, dev(k), dev(v), torch.zeros(1, dtype=torch.int32, device="cuda"), max_end_pos=N)
    od, _ = run_decode(lib, layer, cache, q[:, N - 1], [N], N)
    torch.cuda.synchronize()
    pre = bits_to_f64(host_bits(out)[0, N - 1])
    d = np.abs(bits_to_f64(od[0]) - pre).max()
    assert d <= 1.6e-2, d


def test_cache_offsets_past_2pow31_elements(lib):
    """A full-layer cache of 16 x 8 x 131136 x 128 elements per K and per V,
    more than 2^31. The last sequence fills 131072 positions, so the rows of
    its last KV head from slot ~123000 on lie past element 2^31 (and every
    row of sequences 8-15 past byte 2^31). Append and decode index the cache
    with 64-bit offsets: every row of the long sequence and of the short
    ones against the oracle."""
    announce("cache with offsets past 2^31 elements: B16 cap 131136, 48/8")
    layer = lib.Layer()
    B, cap = 16, 131072 + 64
    assert B * layer.num_kv_heads * cap * 128 > 2 ** 31
    lengths = [100] + [1 + 7 * b for b in range(1, 15)] + [131072]
    seqs = Seqs(2031, lengths, [0] * B, layer.num_kv_heads)
    cache = lib.KVCache(layer, B, cap)
    fill_cache(lib, layer, cache, seqs)
    q = wl.decode_queries(2031, B, layer.num_q_heads, 128)
    out, lse = run_decode(lib, layer, cache, q, lengths, max(lengths))
    check_decode(layer, q, seqs, out, lse, "decode over a cache past 2^31 elements")
