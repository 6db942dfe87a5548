"""The three attention entry points on seeded random layer shapes against the
float64 oracle: layer kind and window, KV heads and group size, Duo masks
(all-full, all-streaming, mixed), sink and recent sizes, batch and ragged
lengths, at the usual bar (max-abs 2e-2, mean-abs 2e-3, lse 1e-3).

* duo_attn_prefill, one-shot and chunked (attend then append) with ragged
  chunk sizes: a seeded sample of rows, always with each sequence's first and
  last row.
* duo_attn_decode: every row, context lengths drawn around the sink, the
  sink + recent band and the window as well as uniformly.
* duo_attn_decode_block: every row of blocks of 1..64 tokens."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce
from test_gpu_decode import Seqs, check_decode, fill_cache, lows_for, run_decode
from test_gpu_decode_block import check_block, run_block
from test_gpu_prefill import compare_rows, run_chunked

pytestmark = pytest.mark.gpu

N_CASES = 12


def _layer(rng, groups=(1, 2, 3, 4, 6)):
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice(groups))
    kw = dict(num_q_heads=hkv * group, num_kv_heads=hkv)
    if rng.random() < 0.5:
        kw.update(kind=1, window=int(rng.choice([64, 200, 512])))
    mask_kind = rng.choice(["none", "mixed", "all_full", "all_stream"])
    if mask_kind != "none":
        mask = {"mixed": rng.integers(0, 2, hkv), "all_full": np.ones(hkv, int),
                "all_stream": np.zeros(hkv, int)}[mask_kind]
        kw.update(full_attention_heads=[int(x) for x in mask], sink=int(rng.choice([0, 4, 64])),
                  recent=int(rng.choice([16, 100, 256])))
    return kw


def _lengths(rng, kw, n, lo=1, hi=3000):
    """Lengths drawn uniformly or next to the layer's sink, sink + recent band
    and window edges."""
    edges = [kw.get("sink", 64), kw.get("sink", 64) + kw.get("recent", 256), kw.get("window", 0)]
    out = []
    for _ in range(n):
        if rng.random() < 0.5:
            out.append(int(rng.integers(lo, hi)))
        else:
            e = int(rng.choice(edges))
            out.append(max(lo, e + int(rng.integers(-1, 2))))
    return out


def _case(i):
    rng = np.random.default_rng(7100 + i)
    kw = _layer(rng)
    B = int(rng.choice([1, 2]))
    N = int(rng.integers(1, 900))
    chunk = int(rng.choice([N, 64, 333, 512]))
    chunk = max(1, min(chunk, N))
    return kw, B, N, chunk, 7200 + i


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_prefill(lib, i):
    kw, B, N, chunk, seed = _case(i)
    announce(f"random shape {i}: {kw} B={B} N={N} chunk={chunk}")
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    q = wl.normal_tokens(seed, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, N, hkv, 128)
    out, lse = run_chunked(lib, layer, q, k, v, chunk)
    rng = np.random.default_rng(seed)
    rows = {(b, h, t) for b in range(B) for h in range(hq) for t in (0, N - 1)}
    n_all = B * hq * N
    for x in rng.choice(n_all, size=min(300, n_all), replace=False):
        b, rem = divmod(int(x), hq * N)
        h, t = divmod(rem, N)
        rows.add((b, h, t))
    compare_rows(layer, q, k, v, out, lse, sorted(rows), f"random shape {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_decode(lib, i):
    rng = np.random.default_rng(7300 + i)
    kw = _layer(rng, groups=(1, 2, 3, 6, 8, 16))
    B = int(rng.integers(1, 7))
    L = _lengths(rng, kw, B)
    announce(f"random decode {i}: {kw} lengths={L}")
    layer = lib.Layer(**kw)
    seqs = Seqs(7400 + i, L, lows_for(layer, L), layer.num_kv_heads)
    # a max_seq_len hint above the longest row changes the split plan only
    max_len = max(L) + int(rng.integers(0, 2000))
    cache = lib.KVCache(layer, B, max_len)
    fill_cache(lib, layer, cache, seqs, chunk=int(rng.choice([97, 512, 4096])))
    q = wl.decode_queries(7500 + i, B, layer.num_q_heads, 128)
    out, lse = run_decode(lib, layer, cache, q, L, max_len)
    check_decode(layer, q, seqs, out, lse, f"random decode {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_decode_block(lib, i):
    rng = np.random.default_rng(7600 + i)
    kw = _layer(rng, groups=(1, 2, 3, 6, 8, 16))
    B = int(rng.integers(1, 5))
    past = _lengths(rng, kw, B, lo=0)
    T = int(rng.choice([1, 2, 3, 4, 5, 8, 13, 16, 33, 64]))
    announce(f"random decode block {i}: {kw} past={past} T={T}")
    layer = lib.Layer(**kw)
    q, k, v, out, lse, _ = run_block(lib, layer, past, T, 7700 + i)
    check_block(layer, past, T, q, k, v, out, lse, f"random decode block {i}")
