"""duo_attn_prefill (one-shot and chunked, attend then append) on seeded random
layer shapes against the float64 oracle: layer kind and window, KV heads and
group size (both workgroup forms), Duo masks (all-full, all-streaming, mixed),
sink and recent sizes, batch, ragged lengths and chunk sizes. Each case checks
a seeded sample of rows (always including each sequence's first and last
row) at the usual bar (max-abs 2e-2, mean-abs 2e-3, lse 1e-3)."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce
from test_gpu_prefill import compare_rows, run_chunked

pytestmark = pytest.mark.gpu

N_CASES = 12


def _case(i):
    rng = np.random.default_rng(7100 + i)
    hkv = int(rng.choice([1, 2, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 6]))
    kw = dict(num_q_heads=hkv * group, num_kv_heads=hkv)
    if rng.random() < 0.5:
        kw.update(kind=1, window=int(rng.choice([64, 200, 512])))
    mask_kind = rng.choice(["none", "mixed", "all_full", "all_stream"])
    if mask_kind != "none":
        mask = {"mixed": rng.integers(0, 2, hkv), "all_full": np.ones(hkv, int),
                "all_stream": np.zeros(hkv, int)}[mask_kind]
        kw.update(full_attention_heads=[int(x) for x in mask], sink=int(rng.choice([0, 4, 64])),
                  recent=int(rng.choice([16, 100, 256])))
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
