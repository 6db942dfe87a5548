"""Pins for the shadow cache model: slot placement must hold exactly the
positions the visibility rule needs (two independent formulations: slot
arithmetic vs. the visible-set definition)."""
import numpy as np
import pytest

import oracle
from oracle import attention as oa


@pytest.mark.parametrize("S,R", [(64, 256), (2, 3), (1, 1), (5, 2)])
def test_streaming_ring_holds_exactly_the_visible_set(S, R):
    for L in list(range(1, 3 * (S + R) + 5)):
        c = oracle.ShadowCache(batch=1, hkv=2, layer="full", window=0, sink=S, recent=R,
                               full_attention_heads=[1, 0])
        c.append(0, 0, L)
        held = sorted(p for p in (c.position_at(0, 1, s) for s in range(S + R)) if p is not None)
        assert held == oa.visible_positions(L - 1, "full", 0, True, S, R).tolist()
        full_held = [c.position_at(0, 0, s) for s in range(L)]
        assert full_held == list(range(L))


@pytest.mark.parametrize("W", [512, 4, 1, 7])
def test_sliding_ring_holds_exactly_the_window(W):
    for L in range(1, 3 * W + 3):
        c = oracle.ShadowCache(batch=1, hkv=1, layer="sliding", window=W, sink=64, recent=256)
        c.append(0, 0, L)
        held = sorted(p for p in (c.position_at(0, 0, s) for s in range(W)) if p is not None)
        assert held == oa.visible_positions(L - 1, "sliding", W, False, 64, 256).tolist()


def test_chunked_appends_equal_one_shot():
    rng = np.random.default_rng(0)
    S, R = 4, 6
    for trial in range(50):
        total = int(rng.integers(1, 60))
        one = oracle.ShadowCache(batch=1, hkv=3, layer="full", window=0, sink=S, recent=R,
                                 full_attention_heads=[0, 1, 0])
        one.append(0, 0, total)
        ch = oracle.ShadowCache(batch=1, hkv=3, layer="full", window=0, sink=S, recent=R,
                                full_attention_heads=[0, 1, 0])
        p = 0
        while p < total:
            n = int(rng.integers(1, 15))
            n = min(n, total - p)
            ch.append(0, p, n)
            p += n
        assert one.slots == ch.slots


def test_head_ranks_are_ascending_per_class():
    c = oracle.ShadowCache(batch=1, hkv=8, layer="full", window=0, sink=64, recent=256,
                           full_attention_heads=[0, 1, 1, 0, 0, 1, 0, 0])
    assert c.rank == [0, 0, 1, 1, 2, 2, 3, 4]
    assert (c.n_full, c.n_stream) == (3, 5)


# ---------------------------------------------------------------- cache report
def _report_case(layer_kw, B, cap, lens):
    import gqa_sliding_window_amd as g
    L = g.Layer(**layer_kw)
    return L, g.kv_cache_report(L, B, cap, lens)


def test_cache_report_closed_forms(lib):
    """Duo decode workload shape: batch 16, one full head of 8, 131072-slot
    full cache; streaming heads hold sink 64 + recent 256 (model card,
    "Summary"); the base layer keeps every head's whole context."""
    lens = [32768 + 6000 * i for i in range(16)]
    L, r = _report_case(dict(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0]), 16, 131072, lens)
    slot = 2 * 128 * 2
    assert r["main_slots"] == 16 * 1 * 131072 and r["stream_slots"] == 16 * 7 * 320
    assert r["main_bytes"] == 16 * 131072 * slot == 1073741824
    assert r["stream_bytes"] == 16 * 7 * 320 * slot == 18350080
    assert r["base_bytes"] == 16 * 8 * 131072 * slot == 8589934592
    assert r["main_active"] == sum(lens) and r["stream_active"] == 16 * 7 * 320
    assert r["base_active"] == 8 * sum(lens)
    # sliding layer: every head is a window ring; Duo streaming heads are smaller still
    L, r = _report_case(dict(kind=1, window=512, full_attention_heads=[1, 1, 0, 0, 0, 0, 0, 0]), 2, 0, [100, 5000])
    assert r["main_slots"] == 2 * 2 * 512 and r["stream_slots"] == 2 * 6 * 320
    assert r["main_active"] == 2 * (100 + 512) and r["stream_active"] == 6 * (100 + 320)
    assert r["base_slots"] == 2 * 8 * 512 and r["base_active"] == 8 * (100 + 512)


@pytest.mark.parametrize("mask,kind,window,cap", [
    ([1, 0, 0, 1], 0, 0, 900), ([0, 0, 0, 0], 0, 0, 50), ([1, 0, 1, 0], 1, 40, 0)])
def test_cache_report_occupancy_matches_shadow_model(lib, mask, kind, window, cap):
    """Occupied slots equal the slots the token-by-token shadow model has
    written after appending positions [0, len) of every sequence."""
    lens = [0, 1, 63, 64, 65, 300, 321, 700]
    B = len(lens)
    L, r = _report_case(dict(num_q_heads=8, num_kv_heads=4, kind=kind, window=window, sink=5,
                             recent=17, full_attention_heads=mask), B, cap, lens)
    sc = oracle.ShadowCache(batch=B, hkv=4, layer="sliding" if kind == 1 else "full", window=window, sink=5,
                     recent=17, full_attention_heads=mask)
    for b, n in enumerate(lens):
        sc.append(b, 0, n)
    occ = {0: 0, 1: 0}
    for (b, cls, rank), slots in sc.slots.items():
        occ[cls] += len(slots)
    assert (r["main_active"], r["stream_active"]) == (occ[0], occ[1])
