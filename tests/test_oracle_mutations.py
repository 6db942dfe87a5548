"""Plant plausible mistakes in the oracle (on the CPU, by monkeypatching) and
check that the pins catch each one."""
import numpy as np
import pytest

from oracle import attention as oa
import test_oracle_pins as pins


def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_wrong_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "kv_head_of", lambda h, hq, hkv: h % hkv)
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("causal"))


def test_window_off_by_one_is_caught(monkeypatch):
    orig = oa.visible_positions

    def bad(i, layer, window, streaming, sink, recent):
        if layer == "sliding" and window > 0 and not streaming:
            return np.arange(max(0, i - window), i + 1)
        return orig(i, layer, window, streaming, sink, recent)
    monkeypatch.setattr(oa, "visible_positions", bad)
    assert _fails(lambda: pins.test_visible_counts_closed_form(700))
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("sliding"))


def test_recent_excluding_current_token_is_caught(monkeypatch):
    orig = oa.visible_positions

    def bad(i, layer, window, streaming, sink, recent):
        if streaming:
            return np.union1d(np.arange(0, min(sink, i + 1)), np.arange(max(0, i - recent), i + 1))
        return orig(i, layer, window, streaming, sink, recent)
    monkeypatch.setattr(oa, "visible_positions", bad)
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("duo"))


def test_wrong_scale_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "_layer_scale", lambda d, s: 1.0 / d)
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("causal"))


def test_dropped_max_subtraction_sign_is_caught(monkeypatch):
    def bad_attend(q, k, v, scale, sink_logit=None):
        s = scale * (k @ q)
        m = s.max()
        w = np.exp(s + m)          # wrong sign: cancels in the output, not in lse
        z = w.sum()
        return (w @ v) / z, m + np.log(z)
    monkeypatch.setattr(oa, "attend", bad_attend)
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("causal"))


def test_transposed_value_use_is_caught(monkeypatch):
    def bad_attend(q, k, v, scale, sink_logit=None):
        s = scale * (k @ q)
        w = np.exp(s - s.max())
        return (w @ k) / w.sum(), s.max() + np.log(w.sum())   # keys used as values
    monkeypatch.setattr(oa, "attend", bad_attend)
    assert _fails(lambda: pins.test_oracle_matches_torch_sdpa("sliding"))


def test_sink_left_out_of_the_normaliser_is_caught(monkeypatch):
    orig = oa.attend

    def bad_attend(q, k, v, scale, sink_logit=None):
        out, lse = orig(q, k, v, scale)          # the sink logit is ignored
        return out, lse
    monkeypatch.setattr(oa, "attend", bad_attend)
    assert _fails(pins.test_sink_closed_form_zero_keys_one_hot_values)
    assert _fails(pins.test_sink_equals_library_softmax_with_an_extra_zero_value_key)


def test_gate_with_the_wrong_sign_is_caught(monkeypatch):
    monkeypatch.setattr(oa, "output_gate", lambda out, gate: out / (1.0 + np.exp(np.asarray(gate, float))))
    assert _fails(pins.test_output_gate_values)
