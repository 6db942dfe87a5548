"""The fused paths on seeded random layer shapes: the q/k prologue (RMSNorm,
RoPE or YaRN, or both) together with the attention-sink logits and the
output gate (per element or per head), through the prefill (chunked over a
past cache filled by kv_append's k prologue, each chunk's own K through the
standalone prologue), the split-K decode and the verify block.

The reference is the float64 oracle step by step: oracle.qk_prologue rounded
to bf16 (the values the kernels attend with), attention with the sink, then
oracle.output_gate; at the usual bar (max-abs 2e-2, mean-abs 2e-3, lse
1e-3)."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, bits_to_f64, check_close, dev, host_bits
from test_gpu_epilogue import _epilogue_inputs, _gate_rows
from test_gpu_prologue import PLAIN, YARN, _prologue, _ref_bf16, _weight
from test_gpu_random_shapes import _layer, _lengths

pytestmark = pytest.mark.gpu

N_CASES = 6


def _kw(layer):
    return dict(hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                window=layer.window, sink=layer.sink, recent=layer.recent,
                full_attention_heads=layer.full_attention_heads, scale=layer.scale)


def _draw(rng):
    """(rope or None, RMSNorm on?, sink logits on?, gate None | "elem" | "head");
    the prologue always does something."""
    rope = [None, PLAIN, YARN][int(rng.integers(0, 3))]
    norm = bool(rng.integers(0, 2)) or rope is None
    return rope, norm, bool(rng.integers(0, 2)), [None, "elem", "head"][int(rng.integers(0, 3))]


def _check(got, o_ref, lse_got, l_ref, what):
    check_close(got, o_ref, what)
    err = np.abs(lse_got - l_ref).max()
    assert err < 1e-3, f"{what}: lse error {err}"


def _sink_dev(sl):
    import torch
    return None if sl is None else torch.from_numpy(sl).cuda()


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fused_prefill(lib, i):
    import torch
    rng = np.random.default_rng(8100 + i)
    kw = _layer(rng)
    rope, norm, sink, gate = _draw(rng)
    B, N = int(rng.integers(1, 3)), int(rng.integers(2, 700))
    chunk = min(int(rng.choice([N, 128, 333])), N)
    announce(f"random fused prefill {i}: {kw} B={B} N={N} chunk={chunk} rope={rope} norm={norm} "
             f"sink={sink} gate={gate}")
    seed = 8200 + i
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    wq, wk = (_weight(seed), _weight(seed + 1)) if norm else (None, None)
    pq, pk = _prologue(lib, wq, rope), _prologue(lib, wk, rope)
    q = wl.normal_tokens(seed, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, N, hkv, 128)
    sl, gbits, _ = _epilogue_inputs(seed, (B, N), hq, sink, gate)
    cache = lib.KVCache(layer, B, N) if chunk < N else None
    out = torch.empty((B, N, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq, N), dtype=torch.float32, device="cuda")
    for P in range(0, N, chunk):
        T = min(chunk, N - P)
        sp = torch.full((B,), P, dtype=torch.int32, device="cuda")
        kd, vd = dev(k[:, P:P + T]), dev(v[:, P:P + T])
        lib.qk_prologue(pk, kd, sp)  # in place: the chunk's K as the attention sees it
        od = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
        ld = torch.empty((B, hq, T), dtype=torch.float32, device="cuda")
        gd = None if gbits is None else dev(np.ascontiguousarray(gbits[:, P:P + T]))
        lib.attn_prefill(layer, dev(q[:, P:P + T]), kd, vd, od, start_pos=P, past=cache, lse=ld,
                         sink_logits=_sink_dev(sl), gate=gd, q_prologue=pq)
        out[:, P:P + T] = od
        lse[:, :, P:P + T] = ld
        if cache is not None and P + T < N:
            # raw K through the append's own prologue
            lib.kv_append(layer, cache, dev(k[:, P:P + T]), vd, sp, max_end_pos=P + T, k_prologue=pk)
    torch.cuda.synchronize()
    ob, lg = host_bits(out), lse.cpu().numpy()
    qr = np.stack([_ref_bf16(q[b], np.arange(N), wq, rope) for b in range(B)])
    kr = np.stack([_ref_bf16(k[b], np.arange(N), wk, rope) for b in range(B)])
    rows = {(b, h, t) for b in range(B) for h in range(hq) for t in (0, N - 1)}
    for x in np.random.default_rng(seed).choice(B * hq * N, size=min(300, B * hq * N), replace=False):
        b, rem = divmod(int(x), hq * N)
        rows.add((b, *divmod(rem, N)))
    r = np.asarray(sorted(rows), dtype=np.int64)
    o_ref, l_ref = oracle.prefill_rows(qr, kr, v, 0, r, sink_logits=sl, **_kw(layer))
    if gbits is not None:
        o_ref = oracle.output_gate(o_ref, _gate_rows(gbits, (r[:, 0], r[:, 2], r[:, 1])))
    _check(bits_to_f64(ob[r[:, 0], r[:, 2], r[:, 1]]), o_ref, lg[r[:, 0], r[:, 1], r[:, 2]].astype(np.float64),
           l_ref, f"random fused prefill {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fused_decode(lib, i):
    import torch
    rng = np.random.default_rng(8300 + i)
    kw = _layer(rng, groups=(1, 2, 3, 6, 8, 16))
    rope, norm, sink, gate = _draw(rng)
    B = int(rng.integers(1, 6))
    L = _lengths(rng, kw, B)
    announce(f"random fused decode {i}: {kw} lengths={L} rope={rope} norm={norm} sink={sink} gate={gate}")
    seed = 8400 + i
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    wq, wk = (_weight(seed), _weight(seed + 1)) if norm else (None, None)
    pq, pk = _prologue(lib, wq, rope), _prologue(lib, wk, rope)
    k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, L, hkv, 128)
    v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, L, hkv, 128)
    cache = lib.KVCache(layer, B, max(L))
    for b in range(B):
        lib.kv_append(layer, cache, dev(k[b][None]), dev(v[b][None]), torch.tensor([0], dtype=torch.int32,
                      device="cuda"), max_end_pos=L[b], batch=1, batch_offset=b, k_prologue=pk)
    q = wl.decode_queries(seed, B, hq, 128)
    sl, gbits, _ = _epilogue_inputs(seed, (B,), hq, sink, gate)
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_workspace(layer, B, max(L))
    lib.attn_decode(layer, cache, dev(q), torch.tensor(L, dtype=torch.int32, device="cuda"), max(L), out, ws,
                    lse=lse, q_prologue=pq, sink_logits=_sink_dev(sl), gate=None if gbits is None else dev(gbits))
    torch.cuda.synchronize()
    kr = [_ref_bf16(k[b], np.arange(L[b]), wk, rope) for b in range(B)]
    qr = np.stack([_ref_bf16(q[b][None], [L[b] - 1], wq, rope)[0] for b in range(B)])
    r = np.array([(b, h) for b in range(B) for h in range(hq)], dtype=np.int64)
    o_ref, l_ref = oracle.decode_rows(qr, lambda b, kvh, pos: (kr[b][pos, kvh], v[b][pos, kvh]), np.asarray(L),
                                      r, sink_logits=sl, **_kw(layer))
    if gbits is not None:
        o_ref = oracle.output_gate(o_ref, _gate_rows(gbits, (r[:, 0], r[:, 1])))
    _check(bits_to_f64(host_bits(out)[r[:, 0], r[:, 1]]), o_ref, lse.cpu().numpy()[r[:, 0], r[:, 1]], l_ref,
           f"random fused decode {i}")


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fused_decode_block(lib, i):
    import torch
    rng = np.random.default_rng(8500 + i)
    kw = _layer(rng, groups=(1, 2, 3, 6, 8, 16))
    rope, norm, sink, gate = _draw(rng)
    B = int(rng.integers(1, 5))
    past = _lengths(rng, kw, B, lo=0)
    T = int(rng.choice([1, 2, 4, 5, 7, 8, 16]))
    announce(f"random fused decode block {i}: {kw} past={past} T={T} rope={rope} norm={norm} sink={sink} "
             f"gate={gate}")
    seed = 8600 + i
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    wq, wk = (_weight(seed), _weight(seed + 1)) if norm else (None, None)
    pq, pk = _prologue(lib, wq, rope), _prologue(lib, wk, rope)
    ends = [p + T for p in past]
    k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, ends, hkv, 128)
    v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, ends, hkv, 128)
    cache = lib.KVCache(layer, B, max(max(past), 1))
    for b in range(B):
        if past[b] > 0:
            lib.kv_append(layer, cache, dev(k[b][None, :past[b]]), dev(v[b][None, :past[b]]),
                          torch.tensor([0], dtype=torch.int32, device="cuda"), max_end_pos=past[b], batch=1,
                          batch_offset=b, k_prologue=pk)
    q = wl.normal_tokens(seed, wl.Q, B, 0, T, hq, 128)
    pl = torch.tensor(past, dtype=torch.int32, device="cuda")
    knd = dev(np.stack([k[b][past[b]:past[b] + T] for b in range(B)]))
    lib.qk_prologue(pk, knd, pl)  # the block's own K at positions past_b + t
    vn = np.stack([v[b][past[b]:past[b] + T] for b in range(B)])
    sl, gbits, _ = _epilogue_inputs(seed, (B, T), hq, sink, gate)
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_block_workspace(layer, B, T, max(past))
    lib.attn_decode_block(layer, cache, dev(q), knd, dev(vn), pl, max(past), out, ws, lse=lse, q_prologue=pq,
                          sink_logits=_sink_dev(sl), gate=None if gbits is None else dev(gbits))
    torch.cuda.synchronize()
    ob, lg = host_bits(out), lse.cpu().numpy()
    got, ref, lgot, lref = [], [], [], []
    for b in range(B):
        kr = _ref_bf16(k[b], np.arange(ends[b]), wk, rope)
        qr = _ref_bf16(q[b], past[b] + np.arange(T), wq, rope)
        rows = np.array([(0, h, t) for h in range(hq) for t in range(T)], dtype=np.int64)
        o_r, l_r = oracle.prefill_rows(qr[None], kr[None], v[b][None], past[b], rows, sink_logits=sl, **_kw(layer))
        if gbits is not None:
            o_r = oracle.output_gate(o_r, _gate_rows(gbits[b], (rows[:, 2], rows[:, 1])))
        got.append(bits_to_f64(ob[b, rows[:, 2], rows[:, 1]]))
        lgot.append(lg[b, rows[:, 2], rows[:, 1]].astype(np.float64))
        ref.append(o_r)
        lref.append(l_r)
    _check(np.concatenate(got), np.concatenate(ref), np.concatenate(lgot), np.concatenate(lref),
           f"random fused decode block {i}")
