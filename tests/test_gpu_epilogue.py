"""The optional epilogue of the attention calls -- attention-sink logits and the
output gate -- against the float64 oracle (oracle.attend with sink_logit,
oracle.output_gate), for the prefill, the split-K decode (single split and
merged splits) and the block decode.

Every case also checks that the oracle's output with the epilogue differs from
its output without it by far more than the tolerance, so a kernel that skipped
the sink or the gate would fail."""
import zlib

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import MAX_ABS, announce, bits_to_f64, check_close, dev, host_bits

pytestmark = pytest.mark.gpu


def _kw(layer):
    return dict(hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                window=layer.window, sink=layer.sink, recent=layer.recent,
                full_attention_heads=layer.full_attention_heads, scale=layer.scale)


def _epilogue_inputs(seed, lead_shape, hq, sink, gate):
    """(sink float32 [hq] or None, gate bits or None, gate broadcast for the
    oracle or None). gate: None | "elem" (like out) | "head" (out without D)."""
    sl = wl.sink_logits(seed, hq) if sink else None
    if gate is None:
        return sl, None, None
    n = int(np.prod(lead_shape))
    d = 128 if gate == "elem" else 1
    bits = wl.normal_tokens(seed, wl.GATE, 1, 0, n, hq, d)[0].reshape(*lead_shape, hq, d)
    if gate == "head":
        bits = bits[..., 0]
    return sl, bits, bits


def _gate_rows(gbits, idx):
    """Gate values (float64) of the selected output rows, shaped to broadcast
    against [n, D] outputs."""
    g = bits_to_f64(gbits[idx])
    return g if g.ndim == 2 else g[:, None]


def _assert_sensitive(o_ref, l_ref, o_plain, l_plain, what):
    d_out = np.abs(o_ref - o_plain).max()
    d_lse = np.abs(l_ref - l_plain).max()
    assert d_out > 5 * MAX_ABS or d_lse > 0.1, f"{what}: the epilogue barely changes the reference"


PREFILL_CASES = {
    # name: (layer kwargs, batch, tokens, chunk start, sink, gate)
    "sliding_w512_sink_gate_elem": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 2, 1000, 0,
                                    True, "elem"),
    "full_duo_chunk_sink_gate_head": (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), 1, 640, 384,
                                      True, "head"),
    "sliding_w64_sink_only": (dict(kind=1, window=64, num_q_heads=8, num_kv_heads=2), 1, 300, 0, True, None),
    "full_gate_elem_only": (dict(num_q_heads=16, num_kv_heads=2), 1, 200, 0, False, "elem"),
    # a prefill workspace: the full-context query tiles cut into key-range
    # pieces, merged before the sink and the gate are applied
    "full_duo_long_chunk_sink_gate_elem_pieces": (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), 1, 640,
                                                  2048, True, "elem"),
}


@pytest.mark.parametrize("name", list(PREFILL_CASES))
def test_prefill_epilogue(lib, name):
    import torch
    kw, B, T, P, sink, gate = PREFILL_CASES[name]
    announce(f"prefill epilogue {name}")
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    seed = zlib.crc32(name.encode()) % 100000
    q = wl.normal_tokens(seed, wl.Q, B, P, T, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, P + T, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, P + T, hkv, 128)
    past = None
    if P > 0:
        past = lib.KVCache(layer, B, P + T)
        sp = torch.zeros(B, dtype=torch.int32, device="cuda")
        lib.kv_append(layer, past, dev(k[:, :P]), dev(v[:, :P]), sp, max_end_pos=P)
    sl, gbits, _ = _epilogue_inputs(seed, (B, T), hq, sink, gate)
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq, T), dtype=torch.float32, device="cuda")
    ws = None
    if name.endswith("_pieces"):
        ws = lib.prefill_workspace(layer, B, T, [P])
        assert lib.prefill_plan(layer, B, T, P, True)[:, 5].max() > 1, "no query tile was cut"
    lib.attn_prefill(layer, dev(q), dev(k[:, P:]), dev(v[:, P:]), out, start_pos=P, past=past, lse=lse,
                     sink_logits=None if sl is None else torch.from_numpy(sl).cuda(),
                     gate=None if gbits is None else dev(gbits), workspace=ws)
    torch.cuda.synchronize()
    ob, lg = host_bits(out), lse.cpu().numpy()
    rows = np.array([(b, h, t) for b in range(B) for h in range(hq) for t in range(T)], dtype=np.int64)
    o_ref, l_ref = oracle.prefill_rows(q, k, v, P, rows, sink_logits=sl, **_kw(layer))
    o_plain, l_plain = oracle.prefill_rows(q, k, v, P, rows, **_kw(layer))
    if gbits is not None:
        g = _gate_rows(gbits, (rows[:, 0], rows[:, 2], rows[:, 1]))
        o_ref = oracle.output_gate(o_ref, g)
    _assert_sensitive(o_ref, l_ref, o_plain, l_plain, name)
    check_close(bits_to_f64(ob[rows[:, 0], rows[:, 2], rows[:, 1]]), o_ref, name)
    err = np.abs(lg[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64) - l_ref).max()
    assert err < 1e-3, f"{name}: lse error {err}"


DECODE_CASES = {
    # name: (layer kwargs, lengths, sink, gate)
    "duo_multisplit_sink_gate_elem": (dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 1, 0]),
                                      [1, 17, 300, 3000, 0], True, "elem"),
    "sliding_w512_gate_head": (dict(kind=1, window=512), [5, 600, 2000], False, "head"),
    "full_single_split_sink": (dict(num_q_heads=32, num_kv_heads=4), [2, 9, 40], True, None),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_epilogue(lib, name):
    import torch
    kw, lengths, sink, gate = DECODE_CASES[name]
    announce(f"decode epilogue {name}")
    layer = lib.Layer(**kw)
    hq, hkv, B = layer.num_q_heads, layer.num_kv_heads, len(lengths)
    seed = zlib.crc32(name.encode()) % 100000
    k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, lengths, hkv, 128)
    v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, lengths, hkv, 128)
    q = wl.decode_queries(seed, B, hq, 128)
    maxlen = max(lengths)
    cache = lib.KVCache(layer, B, maxlen)
    for b in range(B):
        if lengths[b] > 0:
            sp = torch.tensor([0], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, dev(k[b][None]), dev(v[b][None]), sp, max_end_pos=lengths[b],
                          batch=1, batch_offset=b)
    sl, gbits, _ = _epilogue_inputs(seed, (B,), hq, sink, gate)
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_workspace(layer, B, maxlen)
    lib.attn_decode(layer, cache, dev(q), torch.tensor(lengths, dtype=torch.int32, device="cuda"), maxlen, out,
                    ws, lse=lse, sink_logits=None if sl is None else torch.from_numpy(sl).cuda(),
                    gate=None if gbits is None else dev(gbits))
    torch.cuda.synchronize()
    ob, lg = host_bits(out), lse.cpu().numpy()
    rows = np.array([(b, h) for b in range(B) for h in range(hq) if lengths[b] > 0], dtype=np.int64)

    def kv_of(b, kvh, pos):
        return k[b][pos, kvh], v[b][pos, kvh]

    o_ref, l_ref = oracle.decode_rows(q, kv_of, np.asarray(lengths), rows, sink_logits=sl, **_kw(layer))
    o_plain, l_plain = oracle.decode_rows(q, kv_of, np.asarray(lengths), rows, **_kw(layer))
    if gbits is not None:
        o_ref = oracle.output_gate(o_ref, _gate_rows(gbits, (rows[:, 0], rows[:, 1])))
    _assert_sensitive(o_ref, l_ref, o_plain, l_plain, name)
    check_close(bits_to_f64(ob[rows[:, 0], rows[:, 1]]), o_ref, name)
    err = np.abs(lg[rows[:, 0], rows[:, 1]].astype(np.float64) - l_ref).max()
    assert err < 1e-3, f"{name}: lse error {err}"
    for b in range(B):
        if lengths[b] == 0:  # no keys: zero output; lse is the sink alone (-inf without one)
            assert not bits_to_f64(ob[b]).any()
            want = sl.astype(np.float64) if sl is not None else np.full(hq, -np.inf)
            assert np.array_equal(lg[b].astype(np.float64), want), f"{name}: empty-sequence lse"


BLOCK_CASES = {
    # name: (layer kwargs, past lengths, tokens, sink, gate)
    "duo_T4_sink_gate_head": (dict(full_attention_heads=[0, 1, 0, 0, 1, 0, 0, 0]), [0, 63, 700, 2999], 4,
                              True, "head"),
    "sliding_T8_wrapped_sink_gate_elem": (dict(kind=1, window=512), [100, 512, 513, 2000], 8, True, "elem"),
}


@pytest.mark.parametrize("name", list(BLOCK_CASES))
def test_block_decode_epilogue(lib, name):
    import torch
    kw, past, T, sink, gate = BLOCK_CASES[name]
    announce(f"decode block epilogue {name}")
    layer = lib.Layer(**kw)
    hq, hkv, B = layer.num_q_heads, layer.num_kv_heads, len(past)
    seed = zlib.crc32(name.encode()) % 100000
    ends = [p + T for p in past]
    k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, ends, hkv, 128)
    v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, ends, hkv, 128)
    q = wl.normal_tokens(seed, wl.Q, B, 0, T, hq, 128)
    cache = lib.KVCache(layer, B, max(max(past), 1))
    for b in range(B):
        if past[b] > 0:
            sp = torch.tensor([0], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, dev(k[b][None, :past[b]]), dev(v[b][None, :past[b]]), sp,
                          max_end_pos=past[b], batch=1, batch_offset=b)
    kn = np.stack([k[b][past[b]:past[b] + T] for b in range(B)])
    vn = np.stack([v[b][past[b]:past[b] + T] for b in range(B)])
    sl, gbits, _ = _epilogue_inputs(seed, (B, T), hq, sink, gate)
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_block_workspace(layer, B, T, max(past))
    lib.attn_decode_block(layer, cache, dev(q), dev(kn), dev(vn), torch.tensor(past, dtype=torch.int32, device="cuda"),
                          max(past), out, ws, lse=lse,
                          sink_logits=None if sl is None else torch.from_numpy(sl).cuda(),
                          gate=None if gbits is None else dev(gbits))
    torch.cuda.synchronize()
    ob, lg = host_bits(out), lse.cpu().numpy()
    got, ref, plain, lgot, lref, lplain = [], [], [], [], [], []
    for b in range(B):
        rows = np.array([(0, h, t) for h in range(hq) for t in range(T)], dtype=np.int64)
        o_r, l_r = oracle.prefill_rows(q[b:b + 1], k[b][None], v[b][None], past[b], rows, sink_logits=sl,
                                       **_kw(layer))
        o_p, l_p = oracle.prefill_rows(q[b:b + 1], k[b][None], v[b][None], past[b], rows, **_kw(layer))
        if gbits is not None:
            o_r = oracle.output_gate(o_r, _gate_rows(gbits[b], (rows[:, 2], rows[:, 1])))
        got.append(bits_to_f64(ob[b, rows[:, 2], rows[:, 1]]))
        lgot.append(lg[b, rows[:, 2], rows[:, 1]].astype(np.float64))
        ref.append(o_r)
        plain.append(o_p)
        lref.append(l_r)
        lplain.append(l_p)
    o_ref, l_ref = np.concatenate(ref), np.concatenate(lref)
    _assert_sensitive(o_ref, l_ref, np.concatenate(plain), np.concatenate(lplain), name)
    check_close(np.concatenate(got), o_ref, name)
    err = np.abs(np.concatenate(lgot) - l_ref).max()
    assert err < 1e-3, f"{name}: lse error {err}"


def test_neutral_epilogue_matches_plain_kernels_bit_for_bit(lib):
    """The fused kernels (taken whenever a call passes an epilogue) against the
    plain ones: sink logits of -inf add nothing to the normaliser, and a
    per-head gate of 100 has a sigmoid of exactly 1.0 in float32, so prefill,
    multi-split decode and block decode must reproduce the plain outputs and
    lse bit for bit."""
    import torch
    announce("neutral epilogue: fused kernels == plain kernels")
    layer = lib.Layer(full_attention_heads=[1, 0, 0, 0, 1, 0, 0, 0])
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    B, P, T = 2, 9000, 200
    N = P + T
    q = wl.normal_tokens(91, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(91, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(91, wl.V, B, 0, N, hkv, 128)
    sink = torch.full((hq,), float("-inf"), dtype=torch.float32, device="cuda")
    cache = lib.KVCache(layer, B, N + 8)
    sp0 = torch.zeros(B, dtype=torch.int32, device="cuda")
    lib.kv_append(layer, cache, dev(k[:, :P]), dev(v[:, :P]), sp0, max_end_pos=P)

    def both(run, out_shape, lse_shape):
        res = []
        for neutral in (False, True):
            out = torch.empty(out_shape, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
            gate = torch.full(out_shape[:-1], 100.0, dtype=torch.bfloat16, device="cuda") if neutral else None
            run(out, lse, dict(sink_logits=sink, gate=gate) if neutral else {})
            torch.cuda.synchronize()
            res.append((host_bits(out), lse.cpu().numpy()))
        (o0, l0), (o1, l1) = res
        return np.array_equal(o0, o1) and np.array_equal(l0.view(np.uint32), l1.view(np.uint32))

    qc, kc, vc = dev(q[:, P:]), dev(k[:, P:]), dev(v[:, P:])
    assert both(lambda o, l, e: lib.attn_prefill(layer, qc, kc, vc, o, start_pos=P, past=cache, lse=l, **e),
                (B, T, hq, 128), (B, hq, T)), "prefill"
    seq = torch.tensor([P, 3000], dtype=torch.int32, device="cuda")
    qd = dev(wl.decode_queries(92, B, hq, 128))
    ws = lib.decode_workspace(layer, B, P)
    assert lib.decode_plan(layer, B, P)[0] < P, "the decode should be multi-split"
    assert both(lambda o, l, e: lib.attn_decode(layer, cache, qd, seq, P, o, ws, lse=l, **e),
                (B, hq, 128), (B, hq)), "decode"
    Tb = 4
    qb, kb, vb = (dev(wl.normal_tokens(93, t, B, 0, Tb, h, 128)) for t, h in ((wl.Q, hq), (wl.K, hkv), (wl.V, hkv)))
    wsb = lib.decode_block_workspace(layer, B, Tb, P)
    assert both(lambda o, l, e: lib.attn_decode_block(layer, cache, qb, kb, vb, seq, P, o, wsb, lse=l, **e),
                (B, Tb, hq, 128), (B, Tb, hq)), "block decode"
