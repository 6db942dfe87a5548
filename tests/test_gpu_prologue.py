"""The q/k prologue (RMSNorm, then RoPE with YaRN) on the GPU against the
float64 oracle (oracle.prologue): the standalone kernel, K on its way into
the cache (duo_kv_append), and q fused into the prefill, decode and block
decode query loads.

Tolerances. A prologue output is one bf16 rounding (at most 2^-8 of its
value) of a float32 result, so it must lie within 2^-8 |ref| + 1e-4 of the
float64 value. The attention consumes bf16 q and k, so its reference takes
the oracle's prologue outputs rounded once to bf16 (oracle.round_bf16) and
keeps the usual bar: max-abs 2e-2 and mean-abs 2e-3 on outputs, 1e-3 on lse
(a rounding decision the float32 kernel takes the other way moves one
channel by one bf16 step, far inside these)."""
import zlib

import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_util import announce, bits_to_f64, check_close, dev, host_bits

pytestmark = pytest.mark.gpu

YARN = dict(theta=500000.0, factor=64.0, original_max_pos=4096, beta_fast=64.0, beta_slow=1.0)
PLAIN = dict(theta=10000.0)
LSE_TOL = 1e-3


def _kw(layer):
    return dict(hkv=layer.num_kv_heads, layer="sliding" if layer.kind == 1 else "full",
                window=layer.window, sink=layer.sink, recent=layer.recent,
                full_attention_heads=layer.full_attention_heads, scale=layer.scale)


def _lib_rope(lib, rope):
    if rope is None:
        return None
    if rope.get("factor", 1.0) <= 1.0:
        return lib.Rope(theta=rope["theta"], factor=1.0)
    return lib.Rope(theta=rope["theta"], factor=rope["factor"], original_max_position=rope["original_max_pos"],
                    beta_fast=rope["beta_fast"], beta_slow=rope["beta_slow"])


def _weight(seed):
    return (1.0 + 0.3 * np.random.default_rng(seed).standard_normal(128)).astype(np.float32)


def _prologue(lib, w, rope, eps=1e-6):
    import torch
    return lib.Prologue(norm_weight=None if w is None else torch.from_numpy(w).cuda(), eps=eps,
                        rope=_lib_rope(lib, rope))


def _ref(bits, pos, w, rope, eps=1e-6):
    """Oracle prologue of rows bits[n, ..., 128] at positions pos[n]."""
    return oracle.qk_prologue(bits, np.asarray(pos), None if w is None else w.astype(np.float64), eps, rope)


def _ref_bf16(bits, pos, w, rope, eps=1e-6):
    """The attention's view of a prologue output: bf16-rounded."""
    return oracle.round_bf16(_ref(bits, pos, w, rope, eps))


def _check_rows(got_bits, ref, what):
    got = bits_to_f64(got_bits)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    worst = float((err / bound).max())
    print(f"[parity] {what}: n={ref.size} max_abs={err.max():.3e} worst/bound={worst:.3f}", flush=True)
    assert np.isfinite(got).all(), what
    assert worst <= 1.0, f"{what}: error {err.max():.3e} beyond the bf16 rounding bound"


STANDALONE = {
    # name: (weight?, rope, eps, batch, tokens, heads, start positions)
    "norm_and_yarn_long_positions": (True, YARN, 1e-6, 3, 40, 8, [0, 131000, 262100]),
    "yarn_only": (False, YARN, 1e-6, 2, 33, 5, [4000, 90000]),
    "plain_rope_only": (False, PLAIN, 1e-6, 1, 50, 3, [7]),
    "norm_only_eps_large": (True, None, 0.5, 2, 17, 48, [0, 3]),
}


@pytest.mark.parametrize("name", list(STANDALONE))
def test_standalone_prologue(lib, name):
    import torch
    use_w, rope, eps, B, T, H, starts = STANDALONE[name]
    announce(f"qk prologue {name}")
    seed = zlib.crc32(name.encode()) % 100000
    x = wl.normal_tokens(seed, wl.K, B, 0, T, H, 128)
    x[0, 0, 0] = 0  # an all-zero row stays zero (and finite)
    w = _weight(seed) if use_w else None
    pro = _prologue(lib, w, rope, eps)
    xd = dev(x)
    y = torch.empty_like(xd)
    sp = torch.tensor(starts, dtype=torch.int32, device="cuda")
    lib.qk_prologue(pro, xd, sp, y)
    lib.qk_prologue(pro, xd, sp)          # in place gives the same bits
    torch.cuda.synchronize()
    yb, xb = host_bits(y), host_bits(xd)
    assert np.array_equal(yb, xb), f"{name}: in-place result differs"
    for b in range(B):
        ref = _ref(x[b], starts[b] + np.arange(T), w, rope, eps)
        _check_rows(yb[b], ref, f"{name} b={b}")
    assert not bits_to_f64(yb[0, 0, 0]).any()


def test_kv_append_with_k_prologue(lib):
    """Written K slots are the prologue of k at their positions; V stays a
    bit copy; a ring keeps the newest positions."""
    import torch
    announce("kv append with k prologue")
    layer = lib.Layer(kind=1, window=64, num_q_heads=4, num_kv_heads=2)
    B, T, starts = 2, 100, [0, 5000]
    k = wl.normal_tokens_ragged(7, wl.K, starts, [T, T], 2, 128)
    v = wl.normal_tokens_ragged(7, wl.V, starts, [T, T], 2, 128)
    w = _weight(7)
    pro = _prologue(lib, w, YARN)
    cache = lib.KVCache(layer, B, 64)
    lib.kv_append(layer, cache, dev(np.stack(k)), dev(np.stack(v)),
                  torch.tensor(starts, dtype=torch.int32, device="cuda"), max_end_pos=5000 + T, k_prologue=pro)
    torch.cuda.synchronize()
    kc, vc = host_bits(cache.k_main), host_bits(cache.v_main)   # [B, Hkv, 64, 128]
    for b in range(B):
        pos = starts[b] + np.arange(T - 64, T)                  # the newest 64 positions
        ref = _ref(k[b][T - 64:], pos, w, YARN)                   # [64, Hkv, 128]
        slots = pos % 64
        _check_rows(kc[b][:, slots].transpose(1, 0, 2), ref, f"k slots b={b}")
        assert np.array_equal(vc[b][:, slots].transpose(1, 0, 2), v[b][T - 64:]), f"v slots b={b}"


def _fill(lib, layer, cache, k, v, past, w, rope):
    import torch
    for b in range(len(past)):
        if past[b] > 0:
            sp = torch.tensor([0], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, dev(k[b][None, :past[b]]), dev(v[b][None, :past[b]]), sp,
                          max_end_pos=past[b], batch=1, batch_offset=b, k_prologue=_prologue(lib, w, rope))


PREFILL = {
    # name: (layer kwargs, batch, chunk start, tokens, rope)
    "full_duo_yarn_chunk_beyond_4096": (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), 1, 4096, 640, YARN),
    "sliding_plain_rope_one_shot": (dict(kind=1, window=512, num_q_heads=12, num_kv_heads=2), 2, 0, 700, PLAIN),
}


@pytest.mark.parametrize("name", list(PREFILL))
def test_prefill_with_prologue(lib, name):
    """Chunk K through the standalone prologue (in place), q through the
    fused prologue, past K through kv_append's prologue."""
    import torch
    kw, B, P, T, rope = PREFILL[name]
    announce(f"prefill prologue {name}")
    layer = lib.Layer(**kw)
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    seed = zlib.crc32(name.encode()) % 100000
    wq, wk = _weight(seed), _weight(seed + 1)
    q = wl.normal_tokens(seed, wl.Q, B, P, T, hq, 128)
    k = wl.normal_tokens(seed, wl.K, B, 0, P + T, hkv, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, P + T, hkv, 128)
    past = None
    if P > 0:
        past = lib.KVCache(layer, B, P + T)
        _fill(lib, layer, past, k, v, [P] * B, wk, rope)
    kd = dev(k[:, P:])
    lib.qk_prologue(_prologue(lib, wk, rope), kd, torch.full((B,), P, dtype=torch.int32, device="cuda"))
    out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq, T), dtype=torch.float32, device="cuda")
    lib.attn_prefill(layer, dev(q), kd, dev(v[:, P:]), out, start_pos=P, past=past, lse=lse,
                     q_prologue=_prologue(lib, wq, rope))
    torch.cuda.synchronize()
    qr = np.stack([_ref_bf16(q[b], P + np.arange(T), wq, rope) for b in range(B)])
    kr = np.stack([_ref_bf16(k[b], np.arange(P + T), wk, rope) for b in range(B)])
    rows = np.array([(b, h, t) for b in range(B) for h in range(hq) for t in range(T)], dtype=np.int64)
    o_ref, l_ref = oracle.prefill_rows(qr, kr, v, P, rows, **_kw(layer))
    ob, lg = host_bits(out), lse.cpu().numpy()
    check_close(bits_to_f64(ob[rows[:, 0], rows[:, 2], rows[:, 1]]), o_ref, name)
    err = np.abs(lg[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64) - l_ref).max()
    assert err < LSE_TOL, f"{name}: lse error {err}"
    # the prologue matters: without it the reference is far away
    o_raw, _ = oracle.prefill_rows(q, k, v, P, rows[:2000], **_kw(layer))
    assert np.abs(o_raw - o_ref[:2000]).max() > 0.1


@pytest.mark.parametrize("T", [4, 7])
def test_decode_and_block_decode_with_prologue(lib, T):
    """Caches filled through kv_append's k prologue; the decode's fused q
    prologue at position L - 1, the block decode's at past + t (its own K
    through the standalone prologue first). T = 4: one 32-column block; T = 7:
    one 48-column block whose third column block is partly filled."""
    import torch
    announce(f"decode + block decode with prologue T={T}")
    layer = lib.Layer(full_attention_heads=[0, 1, 0, 0, 1, 0, 0, 0])
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    lengths = [1, 300, 4500, 20000]
    B = len(lengths)
    wq, wk = _weight(31), _weight(32)
    ends = [L + T for L in lengths]
    k = wl.normal_tokens_ragged(31, wl.K, [0] * B, ends, hkv, 128)
    v = wl.normal_tokens_ragged(31, wl.V, [0] * B, ends, hkv, 128)
    q1 = wl.decode_queries(31, B, hq, 128)
    qb = wl.normal_tokens(32, wl.Q, B, 0, T, hq, 128)
    maxlen = max(lengths)
    cache = lib.KVCache(layer, B, maxlen + T)
    _fill(lib, layer, cache, k, v, lengths, wk, YARN)
    kr = [_ref_bf16(k[b], np.arange(ends[b]), wk, YARN) for b in range(B)]

    # single-token decode: the token at L - 1 is already in the cache
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    ws = lib.decode_workspace(layer, B, maxlen)
    lib.attn_decode(layer, cache, dev(q1), torch.tensor(lengths, dtype=torch.int32, device="cuda"), maxlen, out, ws,
                    lse=lse, q_prologue=_prologue(lib, wq, YARN))
    torch.cuda.synchronize()
    qr = np.stack([_ref_bf16(q1[b][None], [lengths[b] - 1], wq, YARN)[0] for b in range(B)])
    rows = np.array([(b, h) for b in range(B) for h in range(hq)], dtype=np.int64)
    o_ref, l_ref = oracle.decode_rows(qr, lambda b, kvh, pos: (kr[b][pos, kvh], v[b][pos, kvh]),
                                      np.asarray(lengths), rows, **_kw(layer))
    check_close(bits_to_f64(host_bits(out)[rows[:, 0], rows[:, 1]]), o_ref, "decode with q prologue")
    err = np.abs(lse.cpu().numpy()[rows[:, 0], rows[:, 1]] - l_ref).max()
    assert err < LSE_TOL, f"decode lse error {err}"

    # block decode of T tokens after the cached lengths
    kn = np.stack([k[b][lengths[b]:lengths[b] + T] for b in range(B)])
    vn = np.stack([v[b][lengths[b]:lengths[b] + T] for b in range(B)])
    pl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    knd = dev(kn)
    lib.qk_prologue(_prologue(lib, wk, YARN), knd, pl)
    ob = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    lb = torch.empty((B, T, hq), dtype=torch.float32, device="cuda")
    wsb = lib.decode_block_workspace(layer, B, T, maxlen)
    lib.attn_decode_block(layer, cache, dev(qb), knd, dev(vn), pl, maxlen, ob, wsb, lse=lb,
                          q_prologue=_prologue(lib, wq, YARN))
    torch.cuda.synchronize()
    obb, lbb = host_bits(ob), lb.cpu().numpy()
    got, ref, lg, lr = [], [], [], []
    for b in range(B):
        qrb = _ref_bf16(qb[b], lengths[b] + np.arange(T), wq, YARN)[None]
        rws = np.array([(0, h, t) for h in range(hq) for t in range(T)], dtype=np.int64)
        o_r, l_r = oracle.prefill_rows(qrb, kr[b][None], v[b][None], lengths[b], rws, **_kw(layer))
        got.append(bits_to_f64(obb[b, rws[:, 2], rws[:, 1]]))
        lg.append(lbb[b, rws[:, 2], rws[:, 1]].astype(np.float64))
        ref.append(o_r)
        lr.append(l_r)
    check_close(np.concatenate(got), np.concatenate(ref), "block decode with q prologue")
    err = np.abs(np.concatenate(lg) - np.concatenate(lr)).max()
    assert err < LSE_TOL, f"block decode lse error {err}"
