"""Guard bands: every buffer the library writes (outputs, lse, caches,
workspaces) is the middle of a larger allocation whose margins hold a canary
bit pattern. After each call the margins must be unchanged bit for bit (no
write outside the buffer), and every element of an output that the call must
produce must have been written (no canary left inside it).

The canary is 0x5A5A per bf16 element (about 1.5e16) and 0x5A5A5A5A per
float32 element: neither can be an attention output or a log-sum-exp here."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu

GUARD = 4096          # elements on each side (16-byte aligned for both dtypes)
C16, C32 = 0x5A5A, 0x5A5A5A5A


class Guarded:
    """A device buffer of `shape` inside canary margins."""

    def __init__(self, shape, dtype):
        import torch
        self.n = int(np.prod(shape))
        self.flat = torch.empty(self.n + 2 * GUARD, dtype=dtype, device="cuda")
        self.bits = self.flat.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)
        self.canary = C16 if dtype == torch.bfloat16 else C32
        self.bits.fill_(self.canary)
        self.t = self.flat[GUARD:GUARD + self.n].view(shape)

    def margins_intact(self):
        b = self.bits
        return bool((b[:GUARD] == self.canary).all()) and bool((b[GUARD + self.n:] == self.canary).all())

    def fully_written(self):
        return not bool((self.bits[GUARD:GUARD + self.n] == self.canary).any())


def guarded_cache(lib, layer, batch, cap):
    """A KVCache whose four tensors sit inside canary margins (unwritten slots
    keep the canary; no call reads them)."""
    import torch
    cache = lib.KVCache(layer, batch, cap, zero=False)
    bands = {}
    for name in ("k_main", "v_main", "k_stream", "v_stream"):
        t = getattr(cache, name)
        if t is not None:
            g = Guarded(tuple(t.shape), torch.bfloat16)
            setattr(cache, name, g.t)
            bands[name] = g
    return cache, bands


def assert_bands(bands, what):
    for name, g in bands.items():
        assert g.margins_intact(), f"{what}: write outside {name}"


def test_prefill_chunks_and_append_stay_inside(lib):
    """Duo full layer, 2 sequences, 700 tokens in chunks of 256 (ragged last
    chunk): every chunk's out / lse and the caches it appends to."""
    import torch
    announce("guard bands: chunked Duo prefill + append")
    layer = lib.Layer(full_attention_heads=[1, 0, 0, 1, 0, 0, 0, 0])
    B, N, C = 2, 700, 256
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    q = wl.normal_tokens(71, wl.Q, B, 0, N, hq, 128)
    k = wl.normal_tokens(71, wl.K, B, 0, N, hkv, 128)
    v = wl.normal_tokens(71, wl.V, B, 0, N, hkv, 128)
    cache, bands = guarded_cache(lib, layer, B, N)
    for P in range(0, N, C):
        T = min(C, N - P)
        out = Guarded((B, T, hq, 128), torch.bfloat16)
        lse = Guarded((B, hq, T), torch.float32)
        kd, vd = dev(k[:, P:P + T]), dev(v[:, P:P + T])
        lib.attn_prefill(layer, dev(q[:, P:P + T]), kd, vd, out.t, start_pos=P,
                         past=cache if P > 0 else None, lse=lse.t)
        sp = torch.full((B,), P, dtype=torch.int32, device="cuda")
        lib.kv_append(layer, cache, kd, vd, sp, max_end_pos=P + T)
        torch.cuda.synchronize()
        assert out.margins_intact() and lse.margins_intact(), f"chunk at {P}: write outside out / lse"
        assert out.fully_written() and lse.fully_written(), f"chunk at {P}: output element left unwritten"
        assert_bands(bands, f"append at {P}")


def test_prefill_pieces_stay_inside(lib):
    """A Duo chunk over a 3000-token past with a prefill workspace (its
    full-context query tiles cut into key-range pieces, a ragged last tile):
    out, lse, the workspace and the cache it reads; twice on one workspace."""
    import torch
    announce("guard bands: prefill pieces")
    layer = lib.Layer(full_attention_heads=[0, 1, 0, 0, 0, 0, 0, 1])
    B, P, T = 2, 3000, 300
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    q = wl.normal_tokens(76, wl.Q, B, P, T, hq, 128)
    k = wl.normal_tokens(76, wl.K, B, 0, P + T, hkv, 128)
    v = wl.normal_tokens(76, wl.V, B, 0, P + T, hkv, 128)
    cache, bands = guarded_cache(lib, layer, B, P + T)
    sp = torch.zeros(B, dtype=torch.int32, device="cuda")
    lib.kv_append(layer, cache, dev(k[:, :P]), dev(v[:, :P]), sp, max_end_pos=P)
    assert lib.prefill_plan(layer, B, T, P, True)[:, 5].max() > 1, "no query tile was cut"
    nws = (lib.prefill_workspace_bytes(layer, B, T, P) + 3) // 4
    ws = Guarded((nws,), torch.float32)
    lib.init_decode_workspace(ws.t)
    out = Guarded((B, T, hq, 128), torch.bfloat16)
    lse = Guarded((B, hq, T), torch.float32)
    for _ in range(2):
        lib.attn_prefill(layer, dev(q), dev(k[:, P:]), dev(v[:, P:]), out.t, start_pos=P, past=cache,
                         lse=lse.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert out.margins_intact() and lse.margins_intact() and ws.margins_intact(), "prefill wrote outside"
    assert out.fully_written() and lse.fully_written(), "prefill left an output element unwritten"
    assert_bands(bands, "prefill pieces")


def test_decode_stays_inside(lib):
    """Sliding layer with wrapped rings and a Duo layer with multi-split
    sequences: out, lse, workspace and caches."""
    import torch
    for layer, lengths, cap in ((lib.Layer(kind=lib.SLIDING, window=512), [300, 1500, 2100], 512),
                                (lib.Layer(full_attention_heads=[0, 1, 0, 0, 0, 0, 1, 0]), [5000, 37, 12000], 12000)):
        announce(f"guard bands: decode kind={layer.kind} lengths={lengths}")
        B, hq, hkv = len(lengths), layer.num_q_heads, layer.num_kv_heads
        cache, bands = guarded_cache(lib, layer, B, cap)
        for b, L in enumerate(lengths):
            lo = max(0, L - cap) if layer.main_ring else 0
            kk = wl.normal_tokens(72 + b, wl.K, 1, lo, L - lo, hkv, 128)
            vv = wl.normal_tokens(72 + b, wl.V, 1, lo, L - lo, hkv, 128)
            sp = torch.tensor([lo], dtype=torch.int32, device="cuda")
            lib.kv_append(layer, cache, dev(kk), dev(vv), sp, max_end_pos=L, batch=1, batch_offset=b)
        maxlen = max(lengths)
        nws = (lib.decode_workspace_bytes(layer, B, maxlen) + 3) // 4
        ws = Guarded((nws,), torch.float32)
        lib.init_decode_workspace(ws.t)
        out = Guarded((B, hq, 128), torch.bfloat16)
        lse = Guarded((B, hq), torch.float32)
        q = dev(wl.decode_queries(73, B, hq, 128))
        sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
        for _ in range(2):  # the second call reuses the workspace its first call left
            lib.attn_decode(layer, cache, q, sl, maxlen, out.t, ws.t, lse=lse.t)
        torch.cuda.synchronize()
        assert out.margins_intact() and lse.margins_intact() and ws.margins_intact(), "decode wrote outside"
        assert out.fully_written() and lse.fully_written(), "decode left an output element unwritten"
        assert_bands(bands, "decode / append")


def test_block_decode_and_prologue_stay_inside(lib):
    """Verify block of 6 tokens (36 columns: two column blocks) on a Duo layer, and the
    standalone q/k prologue: out, lse, workspace, caches, prologue output."""
    import torch
    announce("guard bands: block decode T6 + qk_prologue")
    layer = lib.Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 1])
    past = [3000, 64, 900]
    B, T, hq, hkv = len(past), 6, layer.num_q_heads, layer.num_kv_heads
    cache, bands = guarded_cache(lib, layer, B, max(past))
    for b, L in enumerate(past):
        kk = wl.normal_tokens(74 + b, wl.K, 1, 0, L, hkv, 128)
        vv = wl.normal_tokens(74 + b, wl.V, 1, 0, L, hkv, 128)
        sp = torch.tensor([0], dtype=torch.int32, device="cuda")
        lib.kv_append(layer, cache, dev(kk), dev(vv), sp, max_end_pos=L, batch=1, batch_offset=b)
    nws = (lib.decode_block_workspace_bytes(layer, B, T, max(past)) + 3) // 4
    ws = Guarded((nws,), torch.float32)
    lib.init_decode_workspace(ws.t)
    out = Guarded((B, T, hq, 128), torch.bfloat16)
    lse = Guarded((B, T, hq), torch.float32)
    qb = dev(wl.normal_tokens(75, wl.Q, B, 0, T, hq, 128))
    kb = dev(wl.normal_tokens(75, wl.K, B, 0, T, hkv, 128))
    vb = dev(wl.normal_tokens(75, wl.V, B, 0, T, hkv, 128))
    pl = torch.tensor(past, dtype=torch.int32, device="cuda")
    lib.attn_decode_block(layer, cache, qb, kb, vb, pl, max(past), out.t, ws.t, lse=lse.t)
    torch.cuda.synchronize()
    assert out.margins_intact() and lse.margins_intact() and ws.margins_intact(), "block decode wrote outside"
    assert out.fully_written() and lse.fully_written(), "block decode left an output element unwritten"
    assert_bands(bands, "block decode")

    w = torch.from_numpy((1 + 0.1 * np.arange(128) / 128).astype(np.float32)).cuda()
    y = Guarded((B, T, hq, 128), torch.bfloat16)
    lib.qk_prologue(lib.Prologue(norm_weight=w, rope=lib.Rope()), qb, pl, y=y.t)
    torch.cuda.synchronize()
    assert y.margins_intact(), "qk_prologue wrote outside its output"
    assert y.fully_written(), "qk_prologue left an element unwritten"
