"""duo_attn_decode_block (several query tokens per sequence, attend then
append) against the float64 oracle.

Each sequence has its own cached length; the cache is filled by
duo_kv_append with seeded K/V of positions [0, past_b) and the block's own K/V
are the seeded rows of positions past_b .. past_b + T - 1. The oracle reads
the same K/V by absolute position and evaluates the block's tokens as prefill
rows starting at past_b (never from the GPU caches)."""
import zlib

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, bits_to_f64, check_close, dev, host_bits

pytestmark = pytest.mark.gpu


def _kw(layer):
    return dict(hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                window=layer.window, sink=layer.sink, recent=layer.recent,
                full_attention_heads=layer.full_attention_heads, scale=layer.scale)


def run_block(lib, layer, past, T, seed, cap=None, transform=None):
    """Fill the caches to past_b, run the block decode; returns (q, K/V per
    sequence, out bits [B, T, Hq, D], lse [B, T, Hq]). transform(which, bits,
    positions) -> bits, if given, reshapes the value distribution of q, k or
    v (positions: the absolute position of each row of bits)."""
    import torch
    B, hq, hkv = len(past), layer.num_q_heads, layer.num_kv_heads
    ends = [p + T for p in past]
    k = wl.normal_tokens_ragged(seed, wl.K, [0] * B, ends, hkv, 128)
    v = wl.normal_tokens_ragged(seed, wl.V, [0] * B, ends, hkv, 128)
    q = wl.normal_tokens(seed, wl.Q, B, 0, T, hq, 128)
    if transform is not None:
        k = [transform("k", k[b], np.arange(ends[b])) for b in range(B)]
        v = [transform("v", v[b], np.arange(ends[b])) for b in range(B)]
        q = np.stack([transform("q", q[b], past[b] + np.arange(T)) for b in range(B)])
    cap = cap or max(max(past), 1)
    cache = lib.KVCache(layer, B, cap)
    for b in range(B):
        if past[b] > 0:
            sp = torch.tensor([0], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, dev(k[b][None, :past[b]]), dev(v[b][None, :past[b]]), sp,
                          max_end_pos=past[b], batch=1, batch_offset=b)
    kn = np.stack([k[b][past[b]:past[b] + T] for b in range(B)])
    vn = np.stack([v[b][past[b]:past[b] + T] for b in range(B)])
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_block_workspace(layer, B, T, max(past))
    pl = torch.tensor(past, dtype=torch.int32, device="cuda")
    lib.attn_decode_block(layer, cache, dev(q), dev(kn), dev(vn), pl, max(past), out, ws, lse=lse)
    torch.cuda.synchronize()
    return q, k, v, host_bits(out), lse.cpu().numpy(), (cache, ws, kn, vn, pl, out, lse)


def check_block(layer, past, T, q, k, v, out, lse, what, **tol):
    B, hq = len(past), layer.num_q_heads
    got, ref, lg, lr = [], [], [], []
    for b in range(B):
        rows = [(0, h, t) for h in range(hq) for t in range(T)]
        o_ref, l_ref = oracle.prefill_rows(q[b:b + 1], k[b][None], v[b][None], past[b], rows, **_kw(layer))
        r = np.asarray(rows)
        got.append(bits_to_f64(out[b, r[:, 2], r[:, 1]]))
        lg.append(lse[b, r[:, 2], r[:, 1]].astype(np.float64))
        ref.append(o_ref)
        lr.append(l_ref)
    check_close(np.concatenate(got), np.concatenate(ref), what, **tol)
    err = np.abs(np.concatenate(lg) - np.concatenate(lr)).max()
    assert err < 1e-3, f"{what}: lse error {err}"


CASES = {
    "full_T4_multisplit": (dict(), [1, 700, 2999, 64], 4),
    "full_T8_one_48_column_block": (dict(), [0, 130, 1500], 8),
    "full_T1": (dict(), [5, 1000], 1),
    "sliding_T4_wrapped": (dict(kind=1, window=512), [100, 511, 512, 513, 2000], 4),
    "sliding_T8_window_64": (dict(kind=1, window=64), [0, 63, 64, 70, 300], 8),
    "duo_T4": (dict(full_attention_heads=[0, 1, 0, 0, 1, 0, 0, 0]), [0, 40, 64, 300, 320, 321, 2500], 4),
    "duo_T8_small_band": (dict(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0], sink=4, recent=9),
                          [0, 3, 4, 12, 13, 14, 40], 8),
    "all_streaming_T2": (dict(full_attention_heads=[0] * 8), [64, 319, 320, 1000], 2),
    "group16_T3": (dict(num_q_heads=32, num_kv_heads=2), [77, 1200], 3),
    "duo_T7_partial_second_block": (dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 0, 1]), [0, 5, 700, 3000], 7),
    "duo_T10_two_48_column_blocks_ragged": (dict(full_attention_heads=[1, 0, 0, 0, 0, 1, 0, 0]), [0, 64, 900, 4000], 10),
    "full_T16_two_full_48_column_blocks": (dict(), [3, 333, 2048], 16),
    "group16_T64_largest_block": (dict(num_q_heads=32, num_kv_heads=2, kind=1, window=512), [0, 100, 2000], 64),
    "duo_sliding_layer_T5": (dict(kind=1, window=100, full_attention_heads=[1, 0], sink=5, recent=7,
                                  num_q_heads=4, num_kv_heads=2), [0, 6, 12, 99, 100, 101, 450], 5),
}


@pytest.mark.parametrize("name", list(CASES))
def test_block_decode_parity(lib, name):
    kw, past, T = CASES[name]
    announce(f"decode block {name}")
    layer = lib.Layer(**kw)
    seed = zlib.crc32(name.encode()) % 100000
    q, k, v, out, lse, _ = run_block(lib, layer, past, T, seed)
    check_block(layer, past, T, q, k, v, out, lse, name)


def test_block_of_one_equals_decode_after_append(lib):
    """T = 1: attending before appending the token equals the single-token
    decode after appending it."""
    import torch
    layer = lib.Layer(full_attention_heads=[0, 1, 0, 0, 1, 0, 0, 0])
    past = [0, 63, 300, 2000]
    announce("decode block T=1 vs decode")
    q, k, v, out, lse, (cache, ws, kn, vn, pl, _, _) = run_block(lib, layer, past, 1, 11, cap=4096)
    B = len(past)
    lib.kv_append(layer, cache, dev(kn), dev(vn), pl, max_end_pos=max(past) + 1)
    o2 = torch.empty((B, layer.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    wsd = lib.decode_workspace(layer, B, max(past) + 1)
    sl = torch.tensor([p + 1 for p in past], dtype=torch.int32, device="cuda")
    lib.attn_decode(layer, cache, dev(q[:, 0]), sl, max(past) + 1, o2, wsd)
    torch.cuda.synchronize()
    a = bits_to_f64(out[:, 0]).reshape(-1)
    b_ = bits_to_f64(host_bits(o2)).reshape(-1)
    assert np.abs(a - b_).max() <= 2 ** -7, np.abs(a - b_).max()


def test_block_workspace_reuse_and_smaller_call(lib):
    """A second call on the same workspace (counters left at zero by the
    first) and a later call with fewer tokens give the oracle's result."""
    layer = lib.Layer(full_attention_heads=[1, 1, 0, 0, 0, 0, 0, 0])
    announce("decode block workspace reuse")
    past, T = [900, 2500, 31], 6
    q, k, v, out, lse, (cache, ws, kn, vn, pl, o, l) = run_block(lib, layer, past, T, 21)
    check_block(layer, past, T, q, k, v, out, lse, "reuse call 1")
    import torch
    lib.attn_decode_block(layer, cache, dev(q), dev(kn), dev(vn), pl, max(past), o, ws, lse=l)
    torch.cuda.synchronize()
    check_block(layer, past, T, q, k, v, host_bits(o), l.cpu().numpy(), "reuse call 2")
    T2 = 3
    o3 = torch.empty((len(past), T2, layer.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty((len(past), T2, layer.num_q_heads), dtype=torch.float32, device="cuda")
    lib.attn_decode_block(layer, cache, dev(q[:, :T2]), dev(kn[:, :T2]), dev(vn[:, :T2]), pl, max(past), o3, ws,
                          lse=l3)
    torch.cuda.synchronize()
    check_block(layer, past, T2, q[:, :T2], k, v, host_bits(o3), l3.cpu().numpy(), "reuse call 3 (T=3)")


@pytest.mark.parametrize("T", [4, 6, 8])
def test_block_decode_duo_workload(lib, T):
    """The verify-block launches the bench times: T = 4 (24 columns, one
    32-column block), T = 6 (36 columns, a partly filled 48-column block)
    and T = 8 (48 columns, one 48-column block) tokens
    after the Duo decode workload's contexts (batch 16, 48/8
    heads, contexts U[32768, 131072], its Bernoulli(0.25) mask), every row
    against the oracle."""
    import torch
    w = wl.WORKLOADS[4]
    announce(f"decode block parity {w.name} T={T}")
    mask = wl.duo_mask(w).tolist()
    layer = lib.Layer(full_attention_heads=mask)
    past = wl.context_lengths(w).tolist()
    B, hq, hkv = w.batch, w.hq, w.hkv
    ends = [p + T for p in past]
    k = wl.normal_tokens_ragged(w.seed, wl.K, [0] * B, ends, hkv, 128)
    v = wl.normal_tokens_ragged(w.seed, wl.V, [0] * B, ends, hkv, 128)
    q = wl.normal_tokens(w.seed + 1, wl.Q, B, 0, T, hq, 128)
    cache = lib.KVCache(layer, B, w.len_hi, zero=False)
    for b in range(B):
        for p0 in range(0, past[b], 32768):
            n = min(32768, past[b] - p0)
            lib.kv_append(layer, cache, dev(k[b][None, p0:p0 + n]), dev(v[b][None, p0:p0 + n]),
                          torch.tensor([p0], dtype=torch.int32, device="cuda"), max_end_pos=p0 + n, batch=1,
                          batch_offset=b)
    kn = np.stack([k[b][past[b]:past[b] + T] for b in range(B)])
    vn = np.stack([v[b][past[b]:past[b] + T] for b in range(B)])
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, T, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_block_workspace(layer, B, T, w.len_hi)
    lib.attn_decode_block(layer, cache, dev(q), dev(kn), dev(vn), torch.tensor(past, dtype=torch.int32, device="cuda"),
                          w.len_hi, out, ws, lse=lse)
    torch.cuda.synchronize()
    check_block(layer, past, T, q, k, v, host_bits(out), lse.cpu().numpy(), f"{w.name} T={T}")
