"""duo_device_errors: device-side arguments that break the library's contracts
(a KV append past a contiguous cache's capacity, a decode length past that
capacity or past the planned max_seq_len) are clamped inside the caller's
buffers by the kernels and reported in the device error word; in-contract
calls leave it clear.

The out-of-contract data is planted from the host (device start positions and
lengths), and every kernel still runs within its buffers: the append drops the
rows past the capacity, the decode reads at most the capacity and the planned
splits."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce, dev, host_bits

pytestmark = pytest.mark.gpu


def _fill(lib, layer, cache, B, L, seed):
    import torch
    k = wl.normal_tokens(seed, wl.K, B, 0, L, layer.num_kv_heads, 128)
    v = wl.normal_tokens(seed, wl.V, B, 0, L, layer.num_kv_heads, 128)
    sp = torch.zeros(B, dtype=torch.int32, device="cuda")
    lib.kv_append(layer, cache, dev(k), dev(v), sp, max_end_pos=L)
    torch.cuda.synchronize()
    return k, v


def _decode(lib, layer, cache, B, lengths, max_len, seed):
    import torch
    q = wl.normal_tokens(seed, wl.Q, B, 0, 1, layer.num_q_heads, 128)[:, 0]
    ws = lib.decode_workspace(layer, B, max_len)
    out = torch.empty((B, layer.num_q_heads, 128), dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor(lengths, dtype=torch.int32, device="cuda")
    lib.attn_decode(layer, cache, dev(q), sl, max_len, out, ws)
    torch.cuda.synchronize()
    return host_bits(out)


def test_in_contract_calls_leave_the_word_clear(lib):
    announce("device errors: in-contract append and decode")
    import torch
    layer = lib.Layer(num_q_heads=12, num_kv_heads=2, full_attention_heads=[1, 0])
    lib.device_errors(clear=True)
    assert lib.device_errors() == 0
    cache = lib.KVCache(layer, 2, 700)
    _fill(lib, layer, cache, 2, 600, 31)
    _decode(lib, layer, cache, 2, [600, 350], 600, 32)
    torch.cuda.synchronize()
    assert lib.device_errors() == 0


def test_append_past_capacity_is_dropped_and_reported(lib):
    announce("device errors: append past a contiguous cache's capacity")
    import torch
    layer = lib.Layer(num_q_heads=12, num_kv_heads=2, full_attention_heads=[1, 0])
    cap, T = 300, 64
    cache = lib.KVCache(layer, 1, cap)
    lib.device_errors(clear=True)
    k = wl.normal_tokens(33, wl.K, 1, 0, T, 2, 128)
    v = wl.normal_tokens(33, wl.V, 1, 0, T, 2, 128)
    # positions 270..333: the host bound claims they end at the capacity; the
    # device start position says otherwise
    sp = torch.tensor([cap - 30], dtype=torch.int32, device="cuda")
    lib.kv_append(layer, cache, dev(k), dev(v), sp, max_end_pos=cap)
    torch.cuda.synchronize()
    bits = lib.device_errors(clear=True)
    assert bits == lib.DEVICE_APPEND_PAST_CAPACITY, bits
    # the 30 positions inside the cache were written, bit for bit
    km = host_bits(cache.k_main)[0, 0]
    assert np.array_equal(km[cap - 30:cap], np.asarray(k)[0, :30, 0])
    assert lib.device_errors() == 0


def test_decode_lengths_past_capacity_and_plan_are_cut_and_reported(lib):
    announce("device errors: decode lengths past the capacity and past max_seq_len")
    layer = lib.Layer(num_q_heads=12, num_kv_heads=2, full_attention_heads=[1, 0])
    cap = 900
    cache = lib.KVCache(layer, 2, cap)
    _fill(lib, layer, cache, 2, cap, 34)
    lib.device_errors(clear=True)
    # past the planned maximum (max_seq_len 500) but inside the cache
    _decode(lib, layer, cache, 2, [800, 400], 500, 35)
    assert lib.device_errors(clear=True) == lib.DEVICE_LENGTH_PAST_PLAN
    # past the contiguous cache's capacity (and so past max_seq_len, which the
    # host keeps within the capacity): taken as the capacity, which the plan
    # covers
    a = _decode(lib, layer, cache, 2, [cap + 50, 400], cap, 36)
    assert lib.device_errors(clear=True) == lib.DEVICE_LENGTH_PAST_CAPACITY
    # the full-context head of that row reads exactly the capacity's keys
    b = _decode(lib, layer, cache, 2, [cap, 400], cap, 36)
    assert np.array_equal(a[:, :6], b[:, :6])
    assert lib.device_errors() == 0
