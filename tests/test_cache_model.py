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
