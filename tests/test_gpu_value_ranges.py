"""Value distributions that stress the online softmax: peaked rows (q and k
scaled by 4, logits of standard deviation 16), logits that rise with the key
position (k scaled by 1 + position / 64, so the running maximum keeps
moving), and sparse spike keys (k scaled by 8 at every 97th position, so the
maximum jumps by large steps, up or down, in the middle of a row). Each
regime runs through the prefill (one-shot and chunked over a past cache), the
split-K decode and the verify block on a Duo layer and a sliding-window
layer, against the float64 oracle row by row at the bar below.

Scaling is applied to the float32 values of the seeded bf16 inputs, followed
by a round to bf16; the oracle reads the same rounded bits.

The bar is the one the arithmetic gives once rows are peaked: the kernels
round the softmax weights to bf16 for the PV product (unit roundoff 2^-8,
relative), which moves an output by at most 2^-8 max |v|, and round the
output to bf16, which moves it by at most 2^-8 |o|. A peaked row's output is
close to a single V row, so |o| reaches max |v| (about 4.7 here) and the
flat 2e-2 bar of the other tests, made for averages of many keys, no longer
bounds it. Each element must lie within 2^-8 (max |v| + |o|) + 1e-3 of the
oracle; the mean-error bar stays 2e-3."""
import numpy as np
import pytest

import workloads as wl
from gpu_util import announce
from test_gpu_decode import Seqs, check_decode, fill_cache, lows_for, run_decode
from test_gpu_decode_block import check_block, run_block
from test_gpu_prefill import all_rows, compare_rows, run_chunked

pytestmark = pytest.mark.gpu

LAYERS = {
    "duo": dict(num_q_heads=12, num_kv_heads=2, full_attention_heads=[1, 0]),
    "sliding_w128": dict(kind=1, window=128, num_q_heads=12, num_kv_heads=2),
}


def _scale(bits, factor):
    """bf16 bits times a factor broadcast over the leading (position) axis."""
    f = np.asarray(factor, dtype=np.float32).reshape((-1,) + (1,) * (bits.ndim - 1))
    return wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(bits) * f)


def _peaked(which, bits, pos):
    return bits if which == "v" else _scale(bits, np.full(len(pos), 4.0))


def _rising(which, bits, pos):
    return _scale(bits, 1.0 + np.asarray(pos) / 64.0) if which == "k" else bits


def _spikes(which, bits, pos):
    return _scale(bits, np.where(np.asarray(pos) % 97 == 13, 8.0, 1.0)) if which == "k" else bits


REGIMES = {"peaked": _peaked, "rising": _rising, "spikes": _spikes}


def _tol(v_bits):
    vmax = float(np.abs(wl.bf16_bits_to_f32(np.concatenate([np.ravel(x) for x in v_bits]))).max())
    return dict(max_abs=2.0 ** -8 * vmax + 1e-3, rel=2.0 ** -8)


@pytest.mark.parametrize("chunk", [400, 128])
@pytest.mark.parametrize("regime", list(REGIMES))
@pytest.mark.parametrize("name", list(LAYERS))
def test_value_range_prefill(lib, name, regime, chunk):
    announce(f"value range prefill {name} {regime} chunk {chunk}")
    layer = lib.Layer(**LAYERS[name])
    xf = REGIMES[regime]
    B, N, hq, hkv = 2, 400, layer.num_q_heads, layer.num_kv_heads
    pos = np.arange(N)
    q = np.stack([xf("q", b, pos) for b in wl.normal_tokens(51, wl.Q, B, 0, N, hq, 128)])
    k = np.stack([xf("k", b, pos) for b in wl.normal_tokens(51, wl.K, B, 0, N, hkv, 128)])
    v = np.stack([xf("v", b, pos) for b in wl.normal_tokens(51, wl.V, B, 0, N, hkv, 128)])
    out, lse = run_chunked(lib, layer, q, k, v, chunk)
    compare_rows(layer, q, k, v, out, lse, all_rows(B, N, hq), f"{name} {regime} prefill", **_tol(v))


@pytest.mark.parametrize("regime", list(REGIMES))
@pytest.mark.parametrize("name", list(LAYERS))
def test_value_range_decode(lib, name, regime):
    announce(f"value range decode {name} {regime}")
    layer = lib.Layer(**LAYERS[name])
    xf = REGIMES[regime]
    L = [1, 100, 700, 1300]  # the longest rows take several splits
    seqs = Seqs(52, L, lows_for(layer, L), layer.num_kv_heads)
    for b in range(len(L)):
        p = np.arange(seqs.lo[b], L[b])
        seqs.k[b] = xf("k", seqs.k[b], p)
        seqs.v[b] = xf("v", seqs.v[b], p)
    cache = lib.KVCache(layer, len(L), max(L))
    fill_cache(lib, layer, cache, seqs, chunk=300)
    q = np.stack([xf("q", qb[None], [L[b] - 1])[0]
                  for b, qb in enumerate(wl.decode_queries(53, len(L), layer.num_q_heads, 128))])
    out, lse = run_decode(lib, layer, cache, q, L, max(L))
    check_decode(layer, q, seqs, out, lse, f"{name} {regime} decode", **_tol(seqs.v))


@pytest.mark.parametrize("T", [3, 6])
@pytest.mark.parametrize("regime", list(REGIMES))
@pytest.mark.parametrize("name", list(LAYERS))
def test_value_range_decode_block(lib, name, regime, T):
    announce(f"value range decode block {name} {regime} T {T}")
    layer = lib.Layer(**LAYERS[name])
    past = [0, 300, 1200]
    q, k, v, out, lse, _ = run_block(lib, layer, past, T, 54, transform=REGIMES[regime])
    check_block(layer, past, T, q, k, v, out, lse, f"{name} {regime} decode block T={T}", **_tol(v))
