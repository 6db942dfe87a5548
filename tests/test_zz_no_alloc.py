"""duo_attn_decode_noalloc (no workspace argument: the library's own device
scratch) against duo_attn_decode with a caller workspace on the same inputs:
bit for bit, and both against the float64 oracle at the usual bar. Two calls
in a row, the second with a smaller batch and shorter contexts, so the second
reuses scratch the first left behind. A multi-split Duo layer exercises the
partials and the arrival counters."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, dev, host_bits
from test_gpu_decode import Seqs, check_decode, fill_cache

pytestmark = pytest.mark.gpu

CALLS = [
    # (layer kwargs, context lengths, seed)
    (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), [9000, 300, 20000], 81),
    (dict(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0]), [5000, 64], 82),
]


def test_noalloc_decode_matches_workspace_decode(lib):
    import torch
    for kw, lengths, seed in CALLS:
        layer = lib.Layer(**kw)
        B, hq, hkv = len(lengths), layer.num_q_heads, layer.num_kv_heads
        announce(f"no-alloc decode B={B} lengths={lengths}")
        seqs = Seqs(seed, lengths, [0] * B, hkv)
        cache = lib.KVCache(layer, B, max(lengths))
        fill_cache(lib, layer, cache, seqs)
        q = dev(wl.decode_queries(seed, B, hq, 128))
        sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        maxlen = max(lengths)
        sk, items = lib.decode_plan(layer, B, maxlen)
        assert len(items) > B * hkv, "the case must have multi-split sequences"
        ws = lib.decode_workspace(layer, B, maxlen)
        out_w = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
        lse_w = torch.empty((B, hq), dtype=torch.float32, device="cuda")
        lib.attn_decode(layer, cache, q, sl, maxlen, out_w, ws, lse=lse_w)
        out_n = torch.empty_like(out_w)
        lse_n = torch.empty_like(lse_w)
        lib.attn_decode_noalloc(layer, cache, q, sl, maxlen, out_n, lse=lse_n)
        torch.cuda.synchronize()
        a, b_ = host_bits(out_n), host_bits(out_w)
        assert np.array_equal(a, b_), "no-alloc decode differs from the workspace decode"
        assert np.array_equal(lse_n.cpu().numpy(), lse_w.cpu().numpy())
        qh = host_bits(q)
        check_decode(layer, qh, seqs, a, lse_n.cpu().numpy(), f"no-alloc decode B={B}")
