"""The seeded input generator: determinism, window independence, recipe."""
import numpy as np

import workloads as wl


def test_positions_get_the_same_values_whatever_window():
    a = wl.normal_tokens(5, wl.K, 2, 0, 3000, 2, 8)
    b = wl.normal_tokens(5, wl.K, 2, 1000, 1500, 2, 8)
    np.testing.assert_array_equal(a[:, 1000:2500], b)
    c = wl.normal_tokens_ragged(5, wl.K, [1000, 17], [1500, 2000], 2, 8)
    np.testing.assert_array_equal(c[0], a[0, 1000:2500])
    np.testing.assert_array_equal(c[1], a[1, 17:2017])


def test_threaded_generation_is_deterministic():
    a = wl.normal_tokens(9, wl.V, 3, 0, 5000, 4, 16, threads=1)
    b = wl.normal_tokens(9, wl.V, 3, 0, 5000, 4, 16, threads=8)
    np.testing.assert_array_equal(a, b)


def test_tensors_and_seeds_are_independent():
    a = wl.normal_tokens(1, wl.Q, 1, 0, 64, 2, 8)
    assert not np.array_equal(a, wl.normal_tokens(1, wl.K, 1, 0, 64, 2, 8))
    assert not np.array_equal(a, wl.normal_tokens(2, wl.Q, 1, 0, 64, 2, 8))


def test_values_look_standard_normal():
    x = wl.bf16_bits_to_f32(wl.normal_tokens(3, wl.Q, 1, 0, 4096, 8, 128)).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_lengths_mask_rows():
    w3 = wl.WORKLOADS[3]
    L = wl.context_lengths(w3)
    assert L.shape == (64,) and L.min() >= 512 and L.max() <= 32768
    np.testing.assert_array_equal(L, wl.context_lengths(w3))
    m = wl.duo_mask(wl.WORKLOADS[4])
    assert m.shape == (8,) and set(np.unique(m)) <= {0, 1}
    w5 = wl.WORKLOADS[5]
    rows = wl.sample_query_rows(w5, w5.seq, 4096, must=(0, 63, 64, 255, 256, 319, 320, 511, 512, 8191),
                                chunk=w5.chunk)
    assert len(rows) == 4096 and len({tuple(r) for r in rows}) == 4096
    pos = set(rows[:, 2].tolist())
    for c0 in range(0, w5.seq, w5.chunk):
        assert c0 in pos and c0 + w5.chunk - 1 in pos
