"""Pins for the float64 oracle: checks against things other than itself.

* closed forms for the visible-set sizes and boundaries;
* a library routine (torch scaled_dot_product_attention in float64 on the CPU,
  with masks built by torch.tril/triu, and GQA expanded by repeat_interleave);
* invariants (constant V, zero K, first row, sink+recent >= n, window >= n,
  key permutation, MHA reduction);
* a hand-derived two-key example;
* brute force with pure-Python scalar loops on tiny inputs;
* the bf16 conversions against torch's bfloat16 casts.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oa
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _bits(x: np.ndarray) -> np.ndarray:
    return workloads.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 255, 256, 257, 319, 320, 321, 511, 512, 513, 700])
def test_visible_counts_closed_form(n):
    S, R, W = 64, 256, 512
    for i in range(n):
        full = oa.visible_positions(i, "full", 0, False, S, R)
        assert len(full) == i + 1 and full[0] == 0 and full[-1] == i
        sw = oa.visible_positions(i, "sliding", W, False, S, R)
        assert len(sw) == min(i + 1, W)
        assert sw[0] == max(0, i - W + 1) and sw[-1] == i
        st = oa.visible_positions(i, "full", 0, True, S, R)
        assert len(st) == min(i + 1, S + R)
        assert st[-1] == i and len(np.unique(st)) == len(st)
        if i >= S + R:
            # exactly sink [0, S) and recent [i-R+1, i]
            assert st[S - 1] == S - 1 and st[S] == i - R + 1
            assert S not in st and (i - R) not in st


@pytest.mark.parametrize("S,R,W", [(2, 3, 4), (1, 1, 1), (3, 5, 2), (64, 256, 512)])
def test_visible_small_params(S, R, W):
    for i in range(40):
        st = set(oa.visible_positions(i, "full", 0, True, S, R).tolist())
        expect = {j for j in range(i + 1) if j < S or j > i - R}
        assert st == expect
        sw = set(oa.visible_positions(i, "sliding", W, False, S, R).tolist())
        assert sw == {j for j in range(i + 1) if i - j < W}


def test_window_nonpositive_means_full():
    for w in (0, -1):
        for i in (0, 5, 600):
            assert len(oa.visible_positions(i, "sliding", w, False, 64, 256)) == i + 1


def test_streaming_overrides_sliding_layer():
    v = oa.visible_positions(1000, "sliding", 512, True, 64, 256)
    assert len(v) == 320 and v[0] == 0 and v[64] == 1000 - 255


# ------------------------------------------------------------- library routine
def _torch_reference(qb, kb, vb, hkv, mask_fn):
    """SDPA in float64 on CPU; kb/vb bits [B, n, Hkv, D] (positions 0..n-1);
    mask_fn(n, kvh) -> bool [n, n] built with torch ops."""
    B, n, hq, d = qb.shape
    g = hq // hkv
    to = lambda a: torch.from_numpy(oa.bf16_bits_to_f64(a))
    q = to(qb).permute(0, 2, 1, 3)                       # B, Hq, n, D
    k = to(kb).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    v = to(vb).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
    masks = torch.stack([mask_fn(n, h // g) for h in range(hq)])  # Hq, n, n
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=masks[None])
    s = (q @ k.transpose(-1, -2)) / math.sqrt(d)
    s = s.masked_fill(~masks[None], float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()  # [B, n, Hq, D], [B, Hq, n]


def _all_rows(B, n, hq):
    return [(b, h, t) for b in range(B) for h in range(hq) for t in range(n)]


@pytest.mark.parametrize("case", ["causal", "sliding", "duo", "duo_sliding"])
def test_oracle_matches_torch_sdpa(case):
    rng = np.random.default_rng(7)
    B, n, hq, hkv, d = 2, 37, 6, 2, 16
    S, R, W = 3, 5, 7
    qb = _bits(rng.standard_normal((B, n, hq, d)))
    kb = _bits(rng.standard_normal((B, n, hkv, d)))
    vb = _bits(rng.standard_normal((B, n, hkv, d)))
    full_heads = None
    layer, window = "full", 0
    if case in ("duo", "duo_sliding"):
        full_heads = np.array([1, 0], dtype=np.uint8)
    if case in ("sliding", "duo_sliding"):
        layer, window = "sliding", W

    def mask_fn(nn, kvh):
        causal = torch.ones(nn, nn, dtype=torch.bool).tril()
        if full_heads is not None and full_heads[kvh] == 0:
            sink_cols = torch.zeros(nn, nn, dtype=torch.bool)
            sink_cols[:, :S] = True
            band = torch.ones(nn, nn, dtype=torch.bool).triu(-(R - 1))
            return causal & (sink_cols | band)
        if window > 0:
            return causal & torch.ones(nn, nn, dtype=torch.bool).triu(-(window - 1))
        return causal

    ref_o, ref_lse = _torch_reference(qb, kb, vb, hkv, mask_fn)
    rows = _all_rows(B, n, hq)
    o, lse = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=hkv, layer=layer, window=window,
                                 sink=S, recent=R, full_attention_heads=full_heads)
    r = np.asarray(rows)
    np.testing.assert_allclose(o, ref_o[r[:, 0], r[:, 2], r[:, 1]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[r[:, 0], r[:, 1], r[:, 2]], rtol=0, atol=1e-12)


def test_oracle_chunk_offset_matches_sdpa():
    """Rows of a later chunk (start_pos > 0) equal the same rows of a one-shot run."""
    rng = np.random.default_rng(3)
    B, n, hq, hkv, d = 1, 30, 4, 2, 8
    qb = _bits(rng.standard_normal((B, n, hq, d)))
    kb = _bits(rng.standard_normal((B, n, hkv, d)))
    vb = _bits(rng.standard_normal((B, n, hkv, d)))
    ref_o, _ = _torch_reference(qb, kb, vb, hkv, lambda nn, kvh: torch.ones(nn, nn, dtype=torch.bool).tril())
    P = 17
    rows = _all_rows(B, n - P, hq)
    o, _ = oracle.prefill_rows(qb[:, P:], kb, vb, P, rows, hkv=hkv, layer="full")
    r = np.asarray(rows)
    np.testing.assert_allclose(o, ref_o[r[:, 0], r[:, 2] + P, r[:, 1]], atol=1e-12, rtol=0)


def test_decode_rows_match_prefill_last_row():
    rng = np.random.default_rng(11)
    B, n, hq, hkv, d = 3, 50, 4, 2, 8
    qb = _bits(rng.standard_normal((B, n, hq, d)))
    kb = _bits(rng.standard_normal((B, n, hkv, d)))
    vb = _bits(rng.standard_normal((B, n, hkv, d)))
    lengths = np.array([50, 33, 1])
    mask = np.array([0, 1], dtype=np.uint8)
    kw = dict(hkv=hkv, layer="full", sink=4, recent=6, full_attention_heads=mask)
    rows = [(b, h) for b in range(B) for h in range(hq)]
    qd = np.stack([qb[b, lengths[b] - 1] for b in range(B)])
    o, lse = oracle.decode_rows(qd, lambda b, kvh, pos: (kb[b, pos, kvh], vb[b, pos, kvh]),
                                lengths, rows, **kw)
    for n_, (b, h) in enumerate(rows):
        L = lengths[b]
        po, plse = oracle.prefill_rows(qb[:, :L], kb, vb, 0, [(b, h, L - 1)], **kw)
        np.testing.assert_allclose(o[n_], po[0], atol=1e-13, rtol=0)
        assert abs(lse[n_] - plse[0]) < 1e-12


# ------------------------------------------------------------------ invariants
def _rand_case(seed, B=1, n=40, hq=4, hkv=2, d=8):
    rng = np.random.default_rng(seed)
    return (_bits(rng.standard_normal((B, n, hq, d))), _bits(rng.standard_normal((B, n, hkv, d))),
            _bits(rng.standard_normal((B, n, hkv, d))))


@pytest.mark.parametrize("case", [("full", 0, None), ("sliding", 5, None), ("full", 0, [0, 1])])
def test_constant_v_gives_constant_output(case):
    layer, w, mask = case
    qb, kb, vb = _rand_case(1)
    vb[:] = _bits(np.full(1, 0.75))[0]
    rows = _all_rows(1, 40, 4)
    o, _ = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer=layer, window=w, sink=3, recent=4,
                               full_attention_heads=mask)
    np.testing.assert_allclose(o, 0.75, atol=1e-15, rtol=0)


@pytest.mark.parametrize("case", [("full", 0, None), ("sliding", 5, None), ("full", 0, [0, 1])])
def test_zero_k_gives_mean_of_visible_v(case):
    layer, w, mask = case
    qb, kb, vb = _rand_case(2)
    kb[:] = 0
    rows = _all_rows(1, 40, 4)
    o, lse = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer=layer, window=w, sink=3, recent=4,
                                 full_attention_heads=mask)
    vf = oa.bf16_bits_to_f64(vb)
    for n_, (b, h, t) in enumerate(rows):
        kvh = h // 2
        streaming = mask is not None and mask[kvh] == 0
        if streaming:
            vis = [j for j in range(t + 1) if j < 3 or j > t - 4]
        elif w > 0:
            vis = list(range(max(0, t - w + 1), t + 1))
        else:
            vis = list(range(t + 1))
        np.testing.assert_allclose(o[n_], vf[b, vis, kvh].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[n_] - math.log(len(vis))) < 1e-14


def test_first_row_is_first_value():
    qb, kb, vb = _rand_case(3)
    o, lse = oracle.prefill_rows(qb, kb, vb, 0, [(0, h, 0) for h in range(4)], hkv=2, layer="full")
    vf = oa.bf16_bits_to_f64(vb)
    for h in range(4):
        np.testing.assert_array_equal(o[h], vf[0, 0, h // 2])


def test_large_sink_recent_equals_causal_and_large_window_equals_causal():
    qb, kb, vb = _rand_case(4)
    rows = _all_rows(1, 40, 4)
    ref, rl = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer="full")
    st, sl = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer="full", sink=10, recent=30,
                                 full_attention_heads=[0, 0])
    sw, swl = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer="sliding", window=40)
    np.testing.assert_array_equal(st, ref)
    np.testing.assert_array_equal(sw, ref)
    # and when sink + recent < n the streaming result must differ somewhere
    st2, _ = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer="full", sink=10, recent=29,
                                 full_attention_heads=[0, 0])
    assert np.abs(st2 - ref).max() > 1e-6


def test_key_permutation_invariance():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(16)
    k = rng.standard_normal((30, 16))
    v = rng.standard_normal((30, 16))
    perm = rng.permutation(30)
    o1, l1 = oa.attend(q, k, v, 0.25)
    o2, l2 = oa.attend(q, k[perm], v[perm], 0.25)
    np.testing.assert_allclose(o1, o2, atol=1e-14, rtol=0)
    assert abs(l1 - l2) < 1e-13


def test_mha_reduction():
    """GQA with G = 2 equals MHA over KV heads duplicated per query head."""
    qb, kb, vb = _rand_case(6)
    rows = _all_rows(1, 40, 4)
    o_gqa, _ = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=2, layer="sliding", window=9)
    kb2, vb2 = np.repeat(kb, 2, axis=2), np.repeat(vb, 2, axis=2)
    o_mha, _ = oracle.prefill_rows(qb, kb2, vb2, 0, rows, hkv=4, layer="sliding", window=9)
    np.testing.assert_array_equal(o_gqa, o_mha)


def test_head_map_is_contiguous_groups():
    assert [oa.kv_head_of(h, 48, 8) for h in range(48)] == [h // 6 for h in range(48)]
    assert oa.kv_head_of(5, 48, 8) == 0 and oa.kv_head_of(6, 48, 8) == 1


# ------------------------------------------------------------- hand-derived
def test_two_key_worked_example():
    """Logits 0 and ln 3 give weights 1/4 and 3/4, lse = ln 4."""
    d = 2
    scale = 1 / math.sqrt(d)
    q = np.array([math.log(3) * math.sqrt(d), 0.0])
    k = np.array([[0.0, 0.0], [1.0, 0.0]])
    v = np.array([[4.0, -8.0], [0.0, 8.0]])
    o, lse = oa.attend(q, k, v, scale)
    np.testing.assert_allclose(o, [1.0, 4.0], atol=1e-14)
    assert abs(lse - math.log(4)) < 1e-14


# ---------------------------------------------------------------- brute force
def test_brute_force_pure_python():
    rng = np.random.default_rng(9)
    n, hq, hkv, d, S, R, W = 12, 4, 2, 4, 2, 3, 4
    qb = _bits(rng.standard_normal((1, n, hq, d)))
    kb = _bits(rng.standard_normal((1, n, hkv, d)))
    vb = _bits(rng.standard_normal((1, n, hkv, d)))
    qf, kf, vf = (oa.bf16_bits_to_f64(x).tolist() for x in (qb, kb, vb))
    for layer, window, mask in [("full", 0, None), ("sliding", W, None), ("full", 0, [1, 0])]:
        rows = _all_rows(1, n, hq)
        o, lse = oracle.prefill_rows(qb, kb, vb, 0, rows, hkv=hkv, layer=layer, window=window,
                                     sink=S, recent=R, full_attention_heads=mask)
        for idx, (_, h, i) in enumerate(rows):
            c = h // (hq // hkv)
            logits = []
            for j in range(n):
                if j > i:
                    continue
                if mask is not None and mask[c] == 0:
                    if not (j < S or i - j < R):
                        continue
                elif window > 0 and i - j >= window:
                    continue
                dot = 0.0
                for x in range(d):
                    dot += qf[0][i][h][x] * kf[0][j][c][x]
                logits.append((j, dot / math.sqrt(d)))
            mx = max(s for _, s in logits)
            z = sum(math.exp(s - mx) for _, s in logits)
            out = [sum(math.exp(s - mx) * vf[0][j][c][x] for j, s in logits) / z for x in range(d)]
            np.testing.assert_allclose(o[idx], out, atol=1e-13, rtol=0)
            assert abs(lse[idx] - (mx + math.log(z))) < 1e-13


# ------------------------------------------------------------ conversions
def test_bf16_conversions_match_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = oa.bf16_bits_to_f64(ours)
    ref_back = torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(back, ref_back)


# ---------------------------------------------------------------- golden
def test_workloads_use_the_pages_geometry():
    g = json.load(open(os.path.join(HERE, "golden", "laguna_geometry.json")))
    for cid in (2, 3, 4, 5):
        w = workloads.WORKLOADS[cid]
        assert (w.hq, w.hkv, w.d) == (g["num_q_heads"], g["num_kv_heads"], g["head_dim"])
        assert (w.sink, w.recent) == (g["sink"], g["recent"])
    assert workloads.WORKLOADS[1].window == g["window"] and workloads.WORKLOADS[3].window == g["window"]
    assert workloads.WORKLOADS[1].hq // workloads.WORKLOADS[1].hkv == g["num_q_heads"] // g["num_kv_heads"]
    assert g["layers_sliding"] + g["layers_full"] == g["layers_total"]


# ------------------------------------------------------ attention sink and gate
def test_sink_closed_form_zero_keys_one_hot_values():
    """K = 0 makes every logit 0: each of the n visible keys weighs
    1 / (n + e^b) and the normaliser is n + e^b (sink logit b, zero value)."""
    n, D = 37, 128
    q = np.ones(D)
    k = np.zeros((n, D))
    v = np.zeros((n, D))
    for j in range(n):
        v[j, j] = 1.0
    for b in (-3.0, 0.0, 2.5, 30.0):
        out, lse = oa.attend(q, k, v, 0.125, sink_logit=b)
        assert np.allclose(out[:n], 1.0 / (n + math.exp(b)), rtol=1e-14, atol=0)
        assert np.all(out[n:] == 0)
        assert abs(lse - math.log(n + math.exp(b))) < 1e-12


def test_sink_equals_library_softmax_with_an_extra_zero_value_key():
    """The sink is one more key whose logit is b and whose value is zero:
    torch's float64 softmax attention over the keys plus such a key gives
    the same output."""
    import torch
    rng = np.random.default_rng(7)
    D, n, scale, b = 128, 50, 0.09, 1.7
    q = rng.standard_normal(D)
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    k_sink = q * (b / (scale * (q @ q)))            # scale * <q, k_sink> = b
    ke = np.vstack([k, k_sink])
    ve = np.vstack([v, np.zeros(D)])
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(ke)[None, None],
        torch.from_numpy(ve)[None, None], scale=scale)[0, 0, 0].numpy()
    out, lse = oa.attend(q, k, v, scale, sink_logit=b)
    assert np.abs(out - ref).max() < 1e-12
    s = scale * (ke @ q)
    assert abs(lse - (s.max() + math.log(np.exp(s - s.max()).sum()))) < 1e-12


def test_sink_far_below_every_logit_is_no_sink_and_empty_set_is_sink_only():
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal(128), rng.standard_normal((20, 128)), rng.standard_normal((20, 128))
    o1, l1 = oa.attend(q, k, v, 0.1)
    o2, l2 = oa.attend(q, k, v, 0.1, sink_logit=-800.0)
    assert np.abs(o1 - o2).max() < 1e-15 and abs(l1 - l2) < 1e-15
    o3, l3 = oa.attend(q, k[:0], v[:0], 0.1, sink_logit=0.3)
    assert np.all(o3 == 0) and l3 == 0.3


def test_output_gate_values():
    o = np.linspace(-2, 2, 128)[None]
    assert np.array_equal(oa.output_gate(o, np.zeros_like(o)), o / 2)       # logistic(0) = 1/2
    assert np.abs(oa.output_gate(o, np.full_like(o, 60.0)) - o).max() < 1e-25
    g = np.array([[0.7]])
    assert np.array_equal(oa.output_gate(o, g), oa.output_gate(o, np.full_like(o, 0.7)))  # per head = broadcast
    assert abs(oa.output_gate(np.array([1.0]), np.array([math.log(3.0)]))[0] - 0.75) < 1e-15
