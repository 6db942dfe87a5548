"""The attention calls under HIP graph capture: one decode step (append the
new token's K with its prologue, then attend with the q prologue and the
sink; a verify block; a prefill chunk) is captured once and replayed several
times, with eager work and synchronisations between the replays. Every
replay must reproduce the eager results bit for bit: the library allocates
nothing, records no memset, and the decode leaves its arrival counters at
zero for the next replay."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, dev, host_bits

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays_match_eager(lib):
    import torch
    announce("graph capture of a decode step")
    layer = lib.Layer(full_attention_heads=[0, 1, 0, 0, 1, 0, 0, 0])
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    lengths = [100, 2000, 5000]
    B, T = len(lengths), 4
    cap = max(lengths) + 64
    k = wl.normal_tokens_ragged(41, wl.K, [0] * B, lengths, hkv, 128)
    v = wl.normal_tokens_ragged(41, wl.V, [0] * B, lengths, hkv, 128)
    cache = lib.KVCache(layer, B, cap)
    for b in range(B):
        lib.kv_append(layer, cache, dev(k[b][None]), dev(v[b][None]), torch.tensor([0], dtype=torch.int32,
                      device="cuda"), max_end_pos=lengths[b], batch=1, batch_offset=b)
    w = torch.from_numpy((1 + 0.3 * np.random.default_rng(3).standard_normal(128)).astype(np.float32)).cuda()
    pro = lib.Prologue(norm_weight=w, rope=lib.Rope())
    sink = torch.from_numpy(wl.sink_logits(41, hq)).cuda()

    # inputs of the step, all resident before capture
    kn = dev(wl.normal_tokens(42, wl.K, B, 0, 1, hkv, 128))
    vn = dev(wl.normal_tokens(42, wl.V, B, 0, 1, hkv, 128))
    q1 = dev(wl.decode_queries(42, B, hq, 128))
    qb = dev(wl.normal_tokens(43, wl.Q, B, 0, T, hq, 128))
    kb = dev(wl.normal_tokens(43, wl.K, B, 0, T, hkv, 128))
    vb = dev(wl.normal_tokens(43, wl.V, B, 0, T, hkv, 128))
    qc = dev(wl.normal_tokens(44, wl.Q, 1, 0, 256, hq, 128))
    kc = dev(wl.normal_tokens(44, wl.K, 1, 0, 256, hkv, 128))
    vc = dev(wl.normal_tokens(44, wl.V, 1, 0, 256, hkv, 128))
    pos = torch.tensor(lengths, dtype=torch.int32, device="cuda")        # the new token's position
    seq = torch.tensor([x + 1 for x in lengths], dtype=torch.int32, device="cuda")
    maxlen = max(lengths) + 1
    ws = lib.decode_workspace(layer, B, maxlen)
    wsb = lib.decode_block_workspace(layer, B, T, maxlen)
    out = torch.empty((B, hq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, hq), dtype=torch.float32, device="cuda")
    outb = torch.empty((B, T, hq, 128), dtype=torch.bfloat16, device="cuda")
    outc = torch.empty((1, 256, hq, 128), dtype=torch.bfloat16, device="cuda")
    lc = lib.Layer(kind=lib.SLIDING, window=512)
    # a chunk over the Duo cache's longest sequence with a prefill workspace:
    # its full-context query tiles are cut into pieces merged in the launch
    # (arrival counters return to zero inside each replay)
    P = lengths[2]
    qp = dev(wl.normal_tokens(45, wl.Q, 1, P, 256, hq, 128))
    kp = dev(wl.normal_tokens(45, wl.K, 1, P, 256, hkv, 128))
    vp = dev(wl.normal_tokens(45, wl.V, 1, P, 256, hkv, 128))
    outp = torch.empty((1, 256, hq, 128), dtype=torch.bfloat16, device="cuda")
    wsp = lib.prefill_workspace(layer, 1, 256, [P])
    assert lib.prefill_plan(layer, 1, 256, P, True)[:, 5].max() > 1, "no query tile was cut"
    past2 = lib.KVCache(layer, 1, cap)
    past2.k_main, past2.v_main = cache.k_main[2:3], cache.v_main[2:3]
    past2.k_stream, past2.v_stream = cache.k_stream[2:3], cache.v_stream[2:3]

    def step():
        lib.kv_append(layer, cache, kn, vn, pos, max_end_pos=maxlen, k_prologue=pro)
        lib.attn_decode(layer, cache, q1, seq, maxlen, out, ws, lse=lse, q_prologue=pro, sink_logits=sink)
        lib.attn_decode_block(layer, cache, qb, kb, vb, seq, maxlen, outb, wsb, sink_logits=sink)
        lib.attn_prefill(lc, qc, kc, vc, outc)
        lib.attn_prefill(layer, qp, kp, vp, outp, start_pos=P, past=past2, workspace=wsp)

    step()
    torch.cuda.synchronize()
    want = [host_bits(out), lse.cpu().numpy().copy(), host_bits(outb), host_bits(outc), host_bits(outp)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                              # warm-up on the capture stream's side
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.zero_()
        outb.zero_()
        outc.zero_()
        outp.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = [host_bits(out), lse.cpu().numpy(), host_bits(outb), host_bits(outc), host_bits(outp)]
        for name, a, b_ in zip(("decode", "lse", "block", "prefill", "prefill pieces"), got, want):
            assert np.array_equal(a, b_), f"replay {r}: {name} differs from the eager result"
        torch.ones(1024, device="cuda").sum().item()   # eager work between replays
