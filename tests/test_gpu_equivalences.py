"""Equivalences across decompositions of the same attention.

* Split-count invariance: a decode planned for a larger length bound cuts
  each sequence into fewer, longer splits; the result may differ only by the
  rounding of the merge.
* Head-order invariance: permuting the KV heads (with their Duo classes and
  their query-head groups) permutes the outputs and changes nothing else, bit
  for bit: each head's arithmetic is the same wherever its class ranks it."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, bits_to_f64, dev, host_bits

pytestmark = pytest.mark.gpu


def _fill(lib, layer, cache, k, v, lengths):
    import torch
    for b, L in enumerate(lengths):
        sp = torch.tensor([0], dtype=torch.int32, device="cuda")
        lib.kv_append(layer, cache, dev(k[b][None, :L]), dev(v[b][None, :L]), sp, max_end_pos=L,
                      batch=1, batch_offset=b)


def _decode(lib, layer, cache, q, lengths, bound):
    import torch
    B, hq = q.shape[0], q.shape[1]
    ws = lib.decode_workspace(layer, B, bound)
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    lib.attn_decode(layer, cache, dev(q), torch.tensor(lengths, dtype=torch.int32, device="cuda"), bound,
                    out, ws, lse=lse)
    torch.cuda.synchronize()
    return host_bits(out), lse.cpu().numpy()


def test_decode_split_count_invariance(lib):
    layer = lib.Layer(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0])
    lengths = [20000, 7, 33333, 41000]
    B, hq, hkv = len(lengths), layer.num_q_heads, layer.num_kv_heads
    cap = 4 * max(lengths)
    k = wl.normal_tokens_ragged(81, wl.K, [0] * B, lengths, hkv, 128)
    v = wl.normal_tokens_ragged(81, wl.V, [0] * B, lengths, hkv, 128)
    q = wl.decode_queries(81, B, hq, 128)
    cache = lib.KVCache(layer, B, cap)
    _fill(lib, layer, cache, k, v, lengths)
    results = []
    for bound in (max(lengths), 2 * max(lengths), cap):
        split, _ = lib.decode_plan(layer, B, bound)
        announce(f"decode split-count invariance: bound {bound}, split {split} keys")
        results.append((split,) + _decode(lib, layer, cache, q, lengths, bound))
    assert len({r[0] for r in results}) == 3, "the bounds should give three different split sizes"
    o0, l0 = bits_to_f64(results[0][1]), results[0][2]
    for split, o, l in results[1:]:
        err = np.abs(bits_to_f64(o) - o0).max()
        assert err <= 2e-2, f"split {split}: output differs by {err}"
        assert np.abs(l - l0).max() < 1e-4, f"split {split}: lse differs"


def _perm_heads(x, perm, g):
    """Reorder axis -2 (heads) of x by KV-head permutation perm, G query
    heads per KV head when g > 1."""
    idx = np.concatenate([np.arange(p * g, (p + 1) * g) for p in perm]) if g > 1 else np.asarray(perm)
    return np.ascontiguousarray(np.take(x, idx, axis=-2))


def test_head_order_invariance(lib):
    import torch
    mask = [1, 0, 0, 1, 0, 0, 0, 1]
    perm = [3, 6, 0, 7, 1, 5, 2, 4]      # new KV head j is old head perm[j]
    layer_a = lib.Layer(full_attention_heads=mask)
    layer_b = lib.Layer(full_attention_heads=[mask[p] for p in perm])
    hq, hkv = layer_a.num_q_heads, layer_a.num_kv_heads
    G = hq // hkv
    B, T, P = 2, 320, 700                 # prefill chunk of 320 after a 700-token past
    N = P + T
    q = wl.normal_tokens(82, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(82, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(82, wl.V, B, 0, N, hkv, 128)
    outs = []
    for layer, qq, kk, vv in ((layer_a, q, k, v),
                              (layer_b, _perm_heads(q, perm, G), _perm_heads(k, perm, 1), _perm_heads(v, perm, 1))):
        announce(f"head-order invariance: mask {layer.full_attention_heads}")
        cache = lib.KVCache(layer, B, N + 1)
        sp0 = torch.zeros(B, dtype=torch.int32, device="cuda")
        lib.kv_append(layer, cache, dev(kk[:, :P]), dev(vv[:, :P]), sp0, max_end_pos=P)
        out = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, hq, T), dtype=torch.float32, device="cuda")
        lib.attn_prefill(layer, dev(qq[:, P:]), dev(kk[:, P:]), dev(vv[:, P:]), out, start_pos=P, past=cache,
                         lse=lse)
        spP = torch.full((B,), P, dtype=torch.int32, device="cuda")
        lib.kv_append(layer, cache, dev(kk[:, P:]), dev(vv[:, P:]), spP, max_end_pos=N)
        qd = wl.decode_queries(83, B, hq, 128)
        qd = qd if layer is layer_a else _perm_heads(qd, perm, G)
        od, ld = _decode(lib, layer, cache, qd, [N, N], N)
        torch.cuda.synchronize()
        outs.append((host_bits(out), lse.cpu().numpy(), od, ld))
    (pa, la, da, dla), (pb, lb, db, dlb) = outs
    idx = np.concatenate([np.arange(p * G, (p + 1) * G) for p in perm])
    assert np.array_equal(pb, pa[:, :, idx]), "prefill outputs are not the permuted ones"
    assert np.array_equal(lb, la[:, idx]), "prefill lse is not the permuted one"
    assert np.array_equal(db, da[:, idx]), "decode outputs are not the permuted ones"
    assert np.array_equal(dlb, dla[:, idx]), "decode lse is not the permuted one"
