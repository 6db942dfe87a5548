"""duo_attn_prefill against the float64 oracle.

* visibility probes (exact): K = 0 makes every visible key weigh 1/|Vis|;
  V is one-hot at up to 128 probe positions (one output dim per probe), so
  output dim d of row i is nonzero iff probe d is visible to row i, and
  round(exp(lse)) must equal |Vis(i)|;
* parity within max-abs 2e-2 / mean-abs 2e-3 on every row of small and ragged
  cases, the sliding-window prefill workload (batch 1, 12/2 heads, 1024
  tokens, window 512) and chunked Duo prefill, and on 4096 seeded sampled rows
  of the full-attention prefill workload (batch 4, 48/8 heads, 8192 tokens)
  and of the DuoAttention long-context chunked prefill (131072 tokens in
  8192-token chunks, attend then append, as the benchmark runs it).
"""
import math

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, bits_to_f64, check_close, dev, host_bits

pytestmark = pytest.mark.gpu


def _gen(seed, B, N, hq, hkv):
    q = wl.normal_tokens(seed, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, N, hkv, 128)
    return q, k, v


def _layer_kw(layer):
    return dict(hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                window=layer.window, sink=layer.sink, recent=layer.recent,
                full_attention_heads=layer.full_attention_heads, scale=layer.scale)


def run_chunked(lib, layer, q, k, v, chunk, want_lse=True, pieces=False):
    """Prefill [0, N) in chunks (attend, then append). Returns out bits
    [B, N, Hq, D] and lse [B, Hq, N]. pieces: pass a prefill workspace, so
    that long query tiles are cut into key-range pieces."""
    import torch
    B, N, hq, _ = q.shape
    cache = lib.KVCache(layer, B, N) if chunk < N else None
    out = torch.empty((B, N, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq, N), dtype=torch.float32, device="cuda") if want_lse else None
    starts = list(range(0, N, chunk))
    ws = lib.prefill_workspace(layer, B, chunk, starts) if pieces else None
    if pieces:
        cut = [int(lib.prefill_plan(layer, B, min(chunk, N - P), P, True)[:, 5].max()) for P in starts]
        announce(f"prefill pieces per chunk {cut}")
        assert max(cut) > 1, "no query tile was cut: the case does not exercise pieces"
    for P in starts:
        T = min(chunk, N - P)
        qd, kd, vd = dev(q[:, P:P + T]), dev(k[:, P:P + T]), dev(v[:, P:P + T])
        od = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
        ld = torch.empty((B, hq, T), dtype=torch.float32, device="cuda") if want_lse else None
        lib.attn_prefill(layer, qd, kd, vd, od, start_pos=P, past=cache, lse=ld, workspace=ws)
        out[:, P:P + T] = od
        if want_lse:
            lse[:, :, P:P + T] = ld
        if cache is not None and P + T < N:
            sp = torch.full((B,), P, dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, kd, vd, sp, max_end_pos=P + T)
    torch.cuda.synchronize()
    return host_bits(out), (lse.cpu().numpy() if want_lse else None)


def compare_rows(layer, q, k, v, out_bits, lse, rows, what, **tol):
    o_ref, l_ref = oracle.prefill_rows(q, k, v, 0, rows, **_layer_kw(layer))
    r = np.asarray(rows)
    got = bits_to_f64(out_bits[r[:, 0], r[:, 2], r[:, 1]])
    check_close(got, o_ref, what, **tol)
    if lse is not None:
        lg = lse[r[:, 0], r[:, 1], r[:, 2]].astype(np.float64)
        err = np.abs(lg - l_ref).max()
        assert err < 1e-3, f"{what}: lse error {err}"


def all_rows(B, N, hq):
    return [(b, h, t) for b in range(B) for h in range(hq) for t in range(N)]


# ------------------------------------------------------------ visibility probes
PROBE_CASES = {
    "sliding_w512": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 1, 1100, 1100),
    "full_causal": (dict(num_q_heads=12, num_kv_heads=2), 1, 700, 700),
    "duo_s64_r256": (dict(full_attention_heads=[0, 1], num_q_heads=12, num_kv_heads=2), 1, 900, 900),
    "duo_chunked": (dict(full_attention_heads=[0, 1], num_q_heads=12, num_kv_heads=2), 1, 1000, 192),
    "sliding_chunked": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 2, 1300, 300),
    "duo_sliding_layer": (dict(kind=1, window=100, full_attention_heads=[1, 0], sink=5, recent=7,
                               num_q_heads=4, num_kv_heads=2), 1, 400, 130),
}


@pytest.mark.parametrize("name", list(PROBE_CASES))
def test_visibility_probes_exact(lib, name):
    kw, B, N, chunk = PROBE_CASES[name]
    announce(f"prefill probe {name}")
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    rng = np.random.default_rng(1)
    q = wl.normal_tokens(3, wl.Q, B, 0, N, hq, 128)
    k = np.zeros((B, N, hkv, 128), np.uint16)
    v = np.zeros((B, N, hkv, 128), np.uint16)
    special = [0, 1, 4, 5, 6, 7, 63, 64, 65, 99, 100, 127, 128, 255, 256, 257, 319, 320, 321,
               383, 384, 511, 512, 513, 575, 576, 600, 640, N - 2, N - 1]
    probes = sorted({p for p in special if 0 <= p < N})
    probes += sorted(rng.choice(N, size=128 - len(probes), replace=False).tolist())
    probes = probes[:128]
    one = wl.f32_to_bf16_bits(np.array([1.0], np.float32))[0]
    for d, p in enumerate(probes):
        v[:, p, :, d] = one
    out, lse = run_chunked(lib, layer, q, k, v, chunk)
    of = bits_to_f64(out)
    G = hq // hkv
    lk = _layer_kw(layer)
    for h in range(hq):
        streaming = layer.full_attention_heads is not None and layer.full_attention_heads[h // G] == 0
        for i in range(N):
            vis = oracle.visible_positions(i, lk["layer"], lk["window"], streaming, lk["sink"], lk["recent"])
            visset = set(vis.tolist())
            nvis = len(vis)
            for b in range(B):
                row = of[b, i, h]
                expect_nonzero = np.array([p in visset for p in probes])
                got_nonzero = row[:len(probes)] != 0
                if not np.array_equal(got_nonzero, expect_nonzero):
                    bad = np.nonzero(got_nonzero != expect_nonzero)[0][:5]
                    raise AssertionError(f"{name} b={b} h={h} i={i}: probes {[probes[j] for j in bad]} "
                                         f"visible={expect_nonzero[bad]} got={row[bad]}")
                if expect_nonzero.any():
                    np.testing.assert_allclose(row[:len(probes)][expect_nonzero], 1.0 / nvis, rtol=1e-2)
                assert round(math.exp(lse[b, h, i])) == nvis, (name, b, h, i, lse[b, h, i], nvis)


# ------------------------------------------------------------ parity
SMALL = {
    "swa_prefill_b1_h12kv2_s1024_w512": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 1, 1024, 1024, 1),
    "full_ragged_T37": (dict(num_q_heads=12, num_kv_heads=2), 2, 37, 37, 11),
    "full_ragged_T1": (dict(), 1, 1, 1, 12),
    "full_T300_B3": (dict(num_q_heads=12, num_kv_heads=2), 3, 300, 300, 13),
    "duo_T700": (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), 1, 700, 700, 14),
    "duo_all_streaming_T500": (dict(full_attention_heads=[0, 0], num_q_heads=12, num_kv_heads=2), 1, 500, 500, 15),
    "sliding_T2000_w512": (dict(kind=1, window=512, num_q_heads=6, num_kv_heads=1), 1, 2000, 2000, 16),
    "duo_chunked_1000_by_256": (dict(full_attention_heads=[0, 1], num_q_heads=12, num_kv_heads=2), 1, 1000, 256, 17),
    "duo_chunked_ragged_by_333": (dict(full_attention_heads=[1, 0, 0, 0], num_q_heads=24, num_kv_heads=4), 2, 1100, 333, 18),
    "sliding_chunked_by_200": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 1, 1500, 200, 19),
    "full_chunked_by_128": (dict(num_q_heads=6, num_kv_heads=1), 1, 700, 128, 20),
    "group1_mha": (dict(num_q_heads=4, num_kv_heads=4), 1, 260, 260, 21),
    "group16": (dict(num_q_heads=16, num_kv_heads=1), 1, 200, 200, 22),
    "custom_scale": (dict(num_q_heads=6, num_kv_heads=1, scale=0.05), 1, 300, 300, 23),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_prefill_parity_all_rows(lib, name):
    kw, B, N, chunk, seed = SMALL[name]
    announce(f"prefill parity {name}")
    layer = lib.Layer(**kw)
    q, k, v = _gen(seed, B, N, layer.num_q_heads, layer.num_kv_heads)
    out, lse = run_chunked(lib, layer, q, k, v, chunk)
    compare_rows(layer, q, k, v, out, lse, all_rows(B, N, layer.num_q_heads), name)


# key-range pieces (a prefill workspace): 2 to 5 pieces per long query tile,
# ragged chunk and tile edges, every row against the oracle
PIECES = {
    "duo_by_512_pieces": (dict(full_attention_heads=[0, 1], num_q_heads=12, num_kv_heads=2), 1, 2048, 512, 41),
    "duo_ragged_by_333_pieces": (dict(full_attention_heads=[1, 0, 0, 0], num_q_heads=24, num_kv_heads=4),
                                 2, 1600, 333, 42),
    "full_by_1000_pieces": (dict(num_q_heads=6, num_kv_heads=1), 1, 2500, 1000, 43),
}


@pytest.mark.parametrize("name", list(PIECES))
def test_prefill_pieces_parity_all_rows(lib, name):
    kw, B, N, chunk, seed = PIECES[name]
    announce(f"prefill parity {name}")
    layer = lib.Layer(**kw)
    q, k, v = _gen(seed, B, N, layer.num_q_heads, layer.num_kv_heads)
    out, lse = run_chunked(lib, layer, q, k, v, chunk, pieces=True)
    compare_rows(layer, q, k, v, out, lse, all_rows(B, N, layer.num_q_heads), name)
    # the same chunks without a workspace (every tile whole): equal up to the
    # rounding of the merge, and a second call on the same workspace repeats
    # the first bit for bit (its counters were left at zero)
    whole, lse_w = run_chunked(lib, layer, q, k, v, chunk)
    diff = np.abs(bits_to_f64(out) - bits_to_f64(whole))
    assert diff.max() <= 1.6e-2 and diff.mean() <= 1e-4, (diff.max(), diff.mean())
    assert np.abs(lse - lse_w).max() < 1e-4
    again, _ = run_chunked(lib, layer, q, k, v, chunk, pieces=True)
    assert np.array_equal(again, out)


def test_chunked_equals_one_shot(lib):
    announce("prefill chunked == one-shot")
    layer = lib.Layer(full_attention_heads=[0, 1, 0, 0, 0, 0, 1, 0])
    q, k, v = _gen(31, 1, 2048, 48, 8)
    a, _ = run_chunked(lib, layer, q, k, v, 2048)
    b, _ = run_chunked(lib, layer, q, k, v, 512)
    diff = np.abs(bits_to_f64(a) - bits_to_f64(b))
    assert diff.max() <= 1.6e-2, diff.max()


def test_full_prefill_workload_sampled(lib):
    """Full-attention layer prefill: batch 4, 48/8 heads, 8192 tokens; 4096
    seeded rows, always including the boundary rows."""
    w = wl.WORKLOADS[2]
    announce(f"prefill parity {w.name}")
    layer = lib.Layer()
    q, k, v = _gen(w.seed, w.batch, w.seq, w.hq, w.hkv)
    out, lse = run_chunked(lib, layer, q, k, v, w.seq)
    rows = wl.sample_query_rows(w, w.seq, w.oracle_rows,
                                must=(0, 63, 64, 127, 128, 255, 256, 319, 320, 511, 512, 8191))
    compare_rows(layer, q, k, v, out, lse, rows, w.name)


def test_sliding_prefill_headline_shape_sampled(lib):
    """The headline shape (batch 4, 48/8 heads, 8192 tokens) on a 512-token
    sliding-window layer, the layer kind bench.py times beside the full one;
    2048 seeded rows including the window edges."""
    w = wl.WORKLOADS[2]
    announce(f"prefill parity {w.name} sliding w512")
    layer = lib.Layer(kind=lib.SLIDING, window=512)
    q, k, v = _gen(w.seed, w.batch, w.seq, w.hq, w.hkv)
    out, lse = run_chunked(lib, layer, q, k, v, w.seq)
    rows = wl.sample_query_rows(w, w.seq, 2048, must=(0, 511, 512, 513, 1023, 1024, 8191))
    compare_rows(layer, q, k, v, out, lse, rows, w.name + " sliding w512")


def test_duo_chunked_prefill_workload_sampled(lib):
    """DuoAttention long-context chunked prefill at full size: batch 1, 131072
    tokens in 16 chunks of 8192 (attend, then append), 48/8 heads, the seeded
    Bernoulli(0.25) head mask, with a prefill workspace (the full-context
    query tiles cut into key-range pieces, as bench.py runs it); 4096 seeded
    rows including the first and last row of every chunk and the sink /
    recent edges."""
    w = wl.WORKLOADS[5]
    mask = wl.duo_mask(w).tolist()
    announce(f"prefill parity {w.name} mask {mask}")
    layer = lib.Layer(full_attention_heads=mask)
    q, k, v = _gen(w.seed, w.batch, w.seq, w.hq, w.hkv)
    out, lse = run_chunked(lib, layer, q, k, v, w.chunk, pieces=True)  # as bench.py runs it
    rows = wl.sample_query_rows(w, w.seq, w.oracle_rows, chunk=w.chunk,
                                must=(63, 64, 255, 256, 319, 320, 321, 8191 + 320, w.seq - 1))
    G = w.hq // w.hkv
    rows = rows[np.lexsort((rows[:, 2], rows[:, 1] // G, rows[:, 0]))]  # one K/V head at a time
    compare_rows(layer, q, k, v, out, lse, rows, w.name)
