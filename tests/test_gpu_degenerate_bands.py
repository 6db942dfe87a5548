"""Degenerate bands: a sliding window of 1 or 2 positions, a streaming head
that keeps only the current token (sink 0, recent 1), or the sink and the
current token (recent 1). A row that sees one key gives it softmax weight
exactly 1, so its output is that key's V row exactly. Every case is also
compared with the float64 oracle, row by row, for the prefill (one-shot and
chunked over a past cache), the decode and the verify block."""
import zlib

import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, bits_to_f64
from test_gpu_decode import Seqs, check_decode, fill_cache, lows_for, run_decode
from test_gpu_decode_block import check_block, run_block
from test_gpu_prefill import all_rows, compare_rows, run_chunked

pytestmark = pytest.mark.gpu

CASES = {
    "window_1": dict(kind=1, window=1, num_q_heads=12, num_kv_heads=2),
    "window_2": dict(kind=1, window=2, num_q_heads=12, num_kv_heads=2),
    "stream_self_only": dict(num_q_heads=12, num_kv_heads=2, full_attention_heads=[0, 0], sink=0, recent=1),
    "stream_sink_and_self": dict(num_q_heads=12, num_kv_heads=2, full_attention_heads=[0, 1], sink=64, recent=1),
    "sliding_duo_w1_r1": dict(kind=1, window=1, num_q_heads=12, num_kv_heads=2, full_attention_heads=[1, 0],
                              sink=0, recent=1),
}
# KV heads whose rows see only their own key
SELF_ONLY = {"window_1": [0, 1], "stream_self_only": [0, 1], "sliding_duo_w1_r1": [0, 1]}


def _seed(name):
    return zlib.crc32(name.encode()) % 10000


@pytest.mark.parametrize("chunk", [300, 128])
@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_prefill(lib, name, chunk):
    announce(f"degenerate prefill {name} chunk {chunk}")
    layer = lib.Layer(**CASES[name])
    B, N, hq, hkv = 2, 300, layer.num_q_heads, layer.num_kv_heads
    seed = _seed(name)
    q = wl.normal_tokens(seed, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, N, hkv, 128)
    out, lse = run_chunked(lib, layer, q, k, v, chunk)
    # compared as values: the accumulator starts at +0, so a -0 in V (the
    # float32 normal sampler can return an exact zero) comes out as +0
    for kvh in SELF_ONLY.get(name, []):
        G = hq // hkv
        for h in range(kvh * G, (kvh + 1) * G):
            np.testing.assert_array_equal(bits_to_f64(out[:, :, h]), bits_to_f64(v[:, :, kvh]),
                                          err_msg=f"{name} head {h}")
    compare_rows(layer, q, k, v, out, lse, all_rows(B, N, hq), f"degenerate {name}")


@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_decode(lib, name):
    announce(f"degenerate decode {name}")
    layer = lib.Layer(**CASES[name])
    L = [1, 2, 3, 64, 65, 300]
    seqs = Seqs(_seed(name) + 1, L, lows_for(layer, L), layer.num_kv_heads)
    cache = lib.KVCache(layer, len(L), max(L))
    fill_cache(lib, layer, cache, seqs, chunk=97)
    q = wl.decode_queries(_seed(name) + 2, len(L), layer.num_q_heads, 128)
    out, lse = run_decode(lib, layer, cache, q, L, max(L))
    check_decode(layer, q, seqs, out, lse, f"degenerate decode {name}")


@pytest.mark.parametrize("name", list(CASES))
def test_degenerate_decode_block(lib, name):
    announce(f"degenerate decode block {name}")
    layer = lib.Layer(**CASES[name])
    past, T = [0, 1, 5, 300], 4
    q, k, v, out, lse, _ = run_block(lib, layer, past, T, _seed(name) + 3)
    check_block(layer, past, T, q, k, v, out, lse, f"degenerate decode block {name}")
