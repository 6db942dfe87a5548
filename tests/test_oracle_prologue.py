"""Pins of the prologue oracle (RMSNorm of q/k, then RoPE with YaRN) against
things other than itself: library routines (torch's rms_norm, scipy's matrix
exponential of the rotation generator), the page's parameters with indices
derived by hand (tests/golden/laguna_rope.json), turn counts computed
directly, and invariants of rotations."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import prologue as op
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "laguna_rope.json")


def _rope_cfg():
    with open(GOLDEN) as f:
        g = json.load(f)
    return g, dict(theta=g["rope_theta"], factor=g["factor"], original_max_pos=g["original_max_position_embeddings"],
                   beta_fast=g["beta_fast"], beta_slow=g["beta_slow"])


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def test_rms_norm_matches_torch():
    import torch
    x = _rand(1, 5, 3, 128) * 3.0
    w = _rand(2, 128)
    for eps in (1e-6, 1e-2):
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(w), eps).numpy()
        assert np.allclose(op.rms_norm(x, w, eps), ref, rtol=1e-12, atol=1e-12)


def test_rms_norm_closed_forms():
    # unit weight: each head's output has mean square ms / (ms + eps)
    x = _rand(3, 4, 128)
    y = op.rms_norm(x, np.ones(128), 1e-3)
    ms = np.mean(x * x, axis=-1)
    assert np.allclose(np.mean(y * y, axis=-1), ms / (ms + 1e-3), rtol=1e-12)
    # per head, not across heads: scaling one head leaves the others alone
    x2 = x.copy()
    x2[1] *= 50.0
    y2 = op.rms_norm(x2, np.ones(128), 0.0)
    assert np.allclose(y2[0], op.rms_norm(x, np.ones(128), 0.0)[0])
    assert np.allclose(y2[1], op.rms_norm(x, np.ones(128), 0.0)[1])
    # constant row c: output = w * c / sqrt(c^2 + eps)
    c = np.full(128, -2.0)
    w = np.arange(128.0)
    assert np.allclose(op.rms_norm(c, w, 0.5), w * -2.0 / math.sqrt(4.5))


def test_plain_rope_frequencies_closed_form():
    f = op.rope_frequencies(10000.0)
    assert f[0] == 1.0
    assert np.allclose(f[1:] / f[:-1], 10000.0 ** (-2.0 / 128), rtol=1e-12)
    assert np.allclose(f[-1], 10000.0 ** (-126.0 / 128), rtol=1e-12)
    # factor <= 1 leaves YaRN off
    assert np.array_equal(op.rope_frequencies(500000.0, 1.0), op.rope_frequencies(500000.0))


def test_yarn_correction_indices_from_turn_counts():
    """The hand-derived indices of the page's parameters, and the turn count
    of each base frequency over the original context computed directly."""
    g, cfg = _rope_cfg()
    lo = op.yarn_correction_index(cfg["beta_fast"], cfg["theta"], cfg["original_max_pos"])
    hi = op.yarn_correction_index(cfg["beta_slow"], cfg["theta"], cfg["original_max_pos"])
    assert math.floor(lo) == g["low"] and math.ceil(hi) == g["high"]
    i = np.arange(64)
    turns = cfg["original_max_pos"] * cfg["theta"] ** (-2.0 * i / 128) / (2 * math.pi)
    assert turns[g["low"]] > cfg["beta_fast"] > turns[g["low"] + 1]
    assert turns[g["high"] - 1] > cfg["beta_slow"] > turns[g["high"]]


def test_yarn_frequencies_of_the_page_parameters():
    g, cfg = _rope_cfg()
    f = op.rope_frequencies(**cfg)
    base = op.rope_frequencies(cfg["theta"])
    lo, hi, s = g["low"], g["high"], cfg["factor"]
    # many turns in the original context: kept; fewer than one: divided by s
    assert np.array_equal(f[:lo + 1], base[:lo + 1])
    assert np.allclose(f[hi:], base[hi:] / s, rtol=1e-12)
    # in between: linear in the pair index from "kept" to "divided by s"
    for i in range(lo + 1, hi):
        r = (i - lo) / (hi - lo)
        assert np.isclose(f[i] / base[i], (1 - r) + r / s, rtol=1e-12)
    assert np.all(np.diff(f) < 0)


def test_rope_matches_matrix_exponential_of_the_generator():
    """R(pos) = expm(pos * J) with J the block generator that turns channel
    i towards channel i + 64 at angular speed f_i."""
    _, cfg = _rope_cfg()
    f = op.rope_frequencies(**cfg)
    J = np.zeros((128, 128))
    for i in range(64):
        J[i + 64, i] = f[i]
        J[i, i + 64] = -f[i]
    x = _rand(5, 6, 128)
    pos = np.array([0, 1, 7, 300, 4097, 131071])
    got = op.rope_rotate(x, pos, f)
    for n, p in enumerate(pos):
        R = scipy.linalg.expm(p * J)
        assert np.allclose(got[n], R @ x[n], rtol=0, atol=1e-9), p


def test_rope_invariants():
    f = op.rope_frequencies(500000.0, 64.0, 4096, 64.0, 1.0)
    q, k = _rand(7, 1, 4, 128), _rand(8, 1, 4, 128)
    # position 0 is the identity; rotations keep norms; attention_factor scales
    assert np.allclose(op.rope_rotate(q, [0], f), q)
    assert np.allclose(np.linalg.norm(op.rope_rotate(q, [12345], f), axis=-1), np.linalg.norm(q, axis=-1))
    assert np.allclose(op.rope_rotate(q, [99], f, 0.5), 0.5 * op.rope_rotate(q, [99], f))
    # scores depend on the relative position only
    def score(m, n):
        return np.sum(op.rope_rotate(q, [m], f) * op.rope_rotate(k, [n], f), axis=-1)
    assert np.allclose(score(10, 3), score(1010, 1003))
    assert np.allclose(score(70000, 69990), score(10, 0))
    assert not np.allclose(score(10, 3), score(3, 10))
    # composition: rotating by a then b = rotating by a + b
    assert np.allclose(op.rope_rotate(op.rope_rotate(q, [40], f), [2], f), op.rope_rotate(q, [42], f))


def test_qk_prologue_composition():
    bits = wl.normal_tokens(5, wl.Q, 1, 0, 9, 3, 128)[0]          # [9, 3, 128]
    x = wl.bf16_bits_to_f32(bits).astype(np.float64)
    w = _rand(9, 128)
    pos = np.arange(100, 109)
    rope = dict(theta=500000.0, factor=64.0, original_max_pos=4096, beta_fast=64.0, beta_slow=1.0)
    assert np.array_equal(op.qk_prologue(bits, pos), x)
    assert np.allclose(op.qk_prologue(bits, pos, w, 1e-6), op.rms_norm(x, w, 1e-6))
    want = op.rope_rotate(op.rms_norm(x, w, 1e-6), pos, op.rope_frequencies(**rope))
    assert np.allclose(op.qk_prologue(bits, pos, w, 1e-6, rope), want)
    # rows at different positions rotate differently; heads of one row alike
    y = op.qk_prologue(np.broadcast_to(bits[:1], bits.shape), pos, None, 0.0, rope)
    assert not np.allclose(y[0], y[1])
    z = op.qk_prologue(np.broadcast_to(bits[0, :1], (9, 3, 128)), pos, None, 0.0, rope)
    assert np.allclose(z[:, 0], z[:, 1])


def test_round_bf16_matches_the_bit_level_rounding():
    """On float32 values (no double rounding possible) it equals the
    generator's round-to-nearest-even on the bit pattern; exact ties go to
    the even neighbour; bf16 values are fixed points."""
    x32 = (np.random.default_rng(3).standard_normal(20000) * np.exp(np.linspace(-20, 20, 20000))).astype(np.float32)
    want = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(x32)).astype(np.float64)
    assert np.array_equal(op.round_bf16(x32.astype(np.float64)), want)
    one = 1.0
    assert op.round_bf16(one + 2.0 ** -8) == one                    # tie, 1.0 is even
    assert op.round_bf16(one + 3 * 2.0 ** -8) == one + 2.0 ** -6    # tie, goes up to even
    assert op.round_bf16(-(one + 2.0 ** -8 + 2.0 ** -30)) == -(one + 2.0 ** -7)
    assert np.array_equal(op.round_bf16(want), want)
    assert op.round_bf16(0.0) == 0.0


@pytest.mark.parametrize("mistake", ["interleaved_pairs", "reversed_turn", "ramp_reversed", "norm_over_heads",
                                     "sum_not_mean"])
def test_planted_prologue_mistakes_are_caught(monkeypatch, mistake):
    """Each plausible mistake in the prologue oracle fails at least one pin."""
    orig_rotate, orig_freqs = op.rope_rotate, op.rope_frequencies

    if mistake == "interleaved_pairs":
        def bad(x, positions, freqs, attention_factor=1.0):
            x = np.asarray(x, np.float64)
            perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
            y = orig_rotate(x[..., perm], positions, freqs, attention_factor)
            out = np.empty_like(y)
            out[..., perm] = y
            return out
        monkeypatch.setattr(op, "rope_rotate", bad)
        pins = [test_rope_matches_matrix_exponential_of_the_generator]
    elif mistake == "reversed_turn":
        monkeypatch.setattr(op, "rope_rotate", lambda x, p, f, af=1.0: orig_rotate(x, -np.asarray(p), f, af))
        pins = [test_rope_matches_matrix_exponential_of_the_generator]
    elif mistake == "ramp_reversed":
        def bad(theta, factor=1.0, original_max_pos=4096, beta_fast=64.0, beta_slow=1.0, dim=128):
            good = orig_freqs(theta, factor, original_max_pos, beta_fast, beta_slow, dim)
            base = orig_freqs(theta)
            return base * base / good      # slow pairs multiplied by the factor instead of divided
        monkeypatch.setattr(op, "rope_frequencies", bad)
        pins = [test_yarn_frequencies_of_the_page_parameters]
    elif mistake == "norm_over_heads":
        def bad(x, weight, eps):
            x = np.asarray(x, np.float64)
            ms = np.mean(x * x, axis=tuple(range(1, x.ndim)) if x.ndim > 1 else -1, keepdims=True)
            return x / np.sqrt(ms + eps) * weight
        monkeypatch.setattr(op, "rms_norm", bad)
        pins = [test_rms_norm_matches_torch, test_rms_norm_closed_forms]
    else:
        def bad(x, weight, eps):
            x = np.asarray(x, np.float64)
            return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * weight
        monkeypatch.setattr(op, "rms_norm", bad)
        pins = [test_rms_norm_matches_torch, test_rms_norm_closed_forms]

    def fails(fn):
        try:
            fn()
        except AssertionError:
            return True
        return False
    assert any(fails(p) for p in pins), mistake
