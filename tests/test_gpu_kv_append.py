"""duo_kv_append against the shadow cache model: every slot holds the bf16
bits of exactly the position the model assigns, bit for bit, and unwritten
slots keep their canary."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, dev, host_bits

pytestmark = pytest.mark.gpu

CANARY = 0x7F7F


def run_case(lib, layer, batch, appends, capacity, seed=0):
    """appends: list of (start_positions[B], T)."""
    import torch
    G = lib
    hkv = layer.num_kv_heads
    cache = G.KVCache(layer, batch, capacity)
    for t in (cache.k_main, cache.v_main, cache.k_stream, cache.v_stream):
        if t is not None:
            t.view(torch.int16).fill_(CANARY)
    shadow = oracle.ShadowCache(batch=batch, hkv=hkv, layer="sliding" if layer.main_ring else "full",
                                window=layer.window, sink=layer.sink, recent=layer.recent,
                                full_attention_heads=layer.full_attention_heads)
    kvals = {}
    vvals = {}
    for n, (starts, T) in enumerate(appends):
        kb = np.empty((batch, T, hkv, 128), np.uint16)
        vb = np.empty((batch, T, hkv, 128), np.uint16)
        for b, s in enumerate(starts):
            kb[b] = wl.normal_tokens_ragged(seed + b, wl.K, [s], [T], hkv, 128)[0]
            vb[b] = wl.normal_tokens_ragged(seed + b, wl.V, [s], [T], hkv, 128)[0]
            for t in range(T):
                kvals[(b, s + t)] = kb[b, t]
                vvals[(b, s + t)] = vb[b, t]
            shadow.append(b, s, T)
        sp = torch.tensor(starts, dtype=torch.int32, device="cuda")
        G.kv_append(layer, cache, dev(kb), dev(vb), sp, max_end_pos=max(starts) + T)
    torch.cuda.synchronize()
    cls_of = shadow.streaming
    checked = 0
    for name, kt, vt, want_stream in (("main", cache.k_main, cache.v_main, False),
                                      ("stream", cache.k_stream, cache.v_stream, True)):
        if kt is None:
            continue
        kh, vh = host_bits(kt), host_bits(vt)
        heads = [h for h in range(hkv) if cls_of[h] == want_stream]
        for b in range(batch):
            for rank, kvh in enumerate(heads):
                for slot in range(kh.shape[2]):
                    pos = shadow.position_at(b, kvh, slot)
                    if pos is None:
                        assert (kh[b, rank, slot] == CANARY).all(), (name, b, kvh, slot)
                        assert (vh[b, rank, slot] == CANARY).all(), (name, b, kvh, slot)
                    else:
                        np.testing.assert_array_equal(kh[b, rank, slot], kvals[(b, pos)][kvh])
                        np.testing.assert_array_equal(vh[b, rank, slot], vvals[(b, pos)][kvh])
                        checked += 1
    assert checked > 0


CASES = {
    # streaming heads: L < S, S <= L < S+R, L >= S+R, chunks straddling S and S+R, T > R in one call
    "duo_small_chunks": (dict(full_attention_heads=[1, 0, 0, 1], num_q_heads=8, num_kv_heads=4),
                         2, [([0, 0], 30), ([30, 30], 50), ([80, 80], 250), ([330, 330], 7)], 400),
    "duo_one_call_longer_than_ring": (dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 0, 0]),
                                      1, [([0], 1000)], 1024),
    "duo_ragged_starts": (dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 0, 1]),
                          3, [([0, 10, 300], 20), ([20, 30, 320], 300), ([320, 330, 620], 1)], 1024),
    "sliding_ring": (dict(kind=1, window=512), 2, [([0, 100], 300), ([300, 400], 700), ([1000, 1100], 1)], 512),
    "full_layer": (dict(), 2, [([0, 0], 100), ([100, 100], 28)], 256),
    "all_streaming_tiny_ring": (dict(full_attention_heads=[0, 0], num_q_heads=12, num_kv_heads=2, sink=2, recent=3),
                                1, [([0], 1), ([1], 1), ([2], 4), ([6], 9)], 16),
}


@pytest.mark.parametrize("name", list(CASES))
def test_kv_append_bitexact(lib, name):
    layer_kw, batch, appends, cap = CASES[name]
    announce(f"kv_append {name}")
    layer = lib.Layer(**layer_kw)
    run_case(lib, layer, batch, appends, cap)
