"""C-ABI contract on the CPU (no GPU): the library loads, exports every symbol
include/duo_attn.h declares, rejects bad arguments before any launch, and
its host-side plans are complete and skip masked tiles."""
import ctypes
import os
import re

import numpy as np
import pytest

import gqa_sliding_window_amd as g
from gqa_sliding_window_amd import Layer, FULL, SLIDING

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "duo_attn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(duo_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    raw = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert lib.load().duo_attn_version() == 2


def _err(fn, *a, **k):
    with pytest.raises(g.DuoError) as e:
        fn(*a, **k)
    return e.value.code


class FakeTensor:
    """Host stand-in carrying a pointer and a shape (validation only; the
    calls below fail before anything reaches the GPU)."""
    def __init__(self, shape, ptr=0x100000):
        self.shape = shape
        self._p = ptr

    def data_ptr(self):
        return self._p

    def numel(self):
        return int(np.prod(self.shape))

    def element_size(self):
        return 4


def test_layer_validation_errors(lib):
    q = FakeTensor((1, 8, 48, 128))
    kv = FakeTensor((1, 8, 8, 128))
    o = FakeTensor((1, 8, 48, 128))
    assert _err(g.attn_prefill, Layer(head_dim=64), q, kv, kv, o, stream=0) == -2
    assert _err(g.attn_prefill, Layer(num_q_heads=47), q, kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(num_q_heads=34 * 2, num_kv_heads=34), q, kv, kv, o, stream=0) == -2
    assert _err(g.attn_prefill, Layer(num_q_heads=17, num_kv_heads=1), q, kv, kv, o, stream=0) == -2
    assert _err(g.attn_prefill, Layer(kind=7), q, kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(sink=-1), q, kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(full_attention_heads=[0] * 8, recent=0), q, kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(scale=float("inf")), q, kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(scale=-1.0), q, kv, kv, o, stream=0) == -1
    # misaligned and null pointers
    assert _err(g.attn_prefill, Layer(), FakeTensor(q.shape, 0x100002), kv, kv, o, stream=0) == -1
    assert _err(g.attn_prefill, Layer(), FakeTensor(q.shape, 0), kv, kv, o, stream=0) == -1
    # start_pos > 0 without the past cache
    assert _err(g.attn_prefill, Layer(), q, kv, kv, o, start_pos=5, stream=0) == -1
    assert "past cache" in lib.load().duo_last_error().decode()


class FakeCache:
    def __init__(self, k_main=0x200000, v_main=0x300000, cap=1024, k_stream=0x400000, v_stream=0x500000):
        self.vals = (k_main, v_main, cap, k_stream, v_stream)

    def _c(self, batch_offset=0):
        return g._Cache(*self.vals)


def test_cache_validation_errors(lib):
    kv = FakeTensor((2, 16, 8, 128))
    sp = FakeTensor((2,))
    L = Layer()
    # capacity exceeded for a contiguous cache
    assert _err(g.kv_append, L, FakeCache(cap=100), kv, kv, sp, max_end_pos=200, stream=0) == -3
    # sliding ring must have capacity == window
    assert _err(g.kv_append, Layer(kind=SLIDING, window=512), FakeCache(cap=500), kv, kv, sp,
                max_end_pos=16, stream=0) == -1
    # streaming heads need the stream cache
    assert _err(g.kv_append, Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0]),
                FakeCache(k_stream=0, v_stream=0), kv, kv, sp, max_end_pos=16, stream=0) == -1
    # misaligned cache
    assert _err(g.kv_append, L, FakeCache(k_main=0x200008), kv, kv, sp, max_end_pos=16, stream=0) == -1
    # max_end_pos below the chunk length
    assert _err(g.kv_append, L, FakeCache(), kv, kv, sp, max_end_pos=3, stream=0) == -1
    # prefill start_pos beyond capacity
    q = FakeTensor((2, 16, 48, 128))
    assert _err(g.attn_prefill, L, q, kv, kv, q, start_pos=2000, past=FakeCache(cap=1024), stream=0) == -3


def test_decode_validation_errors(lib):
    q = FakeTensor((4, 48, 128))
    sl = FakeTensor((4,))
    L = Layer()
    need = g.decode_workspace_bytes(L, 4, 1000)
    assert need > 0
    ws_small = FakeTensor((need // 4 - 1,), 0x600000)
    assert _err(g.attn_decode, L, FakeCache(cap=1000), q, sl, 1000, q, ws_small, stream=0) == -4
    ws_mis = FakeTensor((need // 4 + 64,), 0x600010)
    assert _err(g.attn_decode, L, FakeCache(cap=1000), q, sl, 1000, q, ws_mis, stream=0) == -4
    ws = FakeTensor((need // 4,), 0x600000)
    assert _err(g.attn_decode, L, FakeCache(cap=999), q, sl, 1000, q, ws, stream=0) == -3
    assert _err(g.attn_decode, L, FakeCache(cap=1000), q, sl, 0, q, ws, stream=0) == -1
    assert g.decode_workspace_bytes(Layer(head_dim=64), 4, 1000) == 0


def test_empty_calls_are_noops(lib):
    kv = FakeTensor((0, 16, 8, 128))
    g.kv_append(Layer(), FakeCache(), kv, kv, FakeTensor((0,)), max_end_pos=16, stream=0)
    q = FakeTensor((2, 0, 48, 128))
    g.attn_prefill(Layer(), q, q, q, q, stream=0)


def test_head_plan(lib):
    cls, rank, nm, ns = g.head_plan(Layer(full_attention_heads=[0, 1, 1, 0, 0, 1, 0, 0]))
    assert cls == [1, 0, 0, 1, 1, 0, 1, 1]
    assert rank == [0, 0, 1, 1, 2, 2, 3, 4]
    assert (nm, ns) == (3, 5)
    cls, rank, nm, ns = g.head_plan(Layer())
    assert cls == [0] * 8 and rank == list(range(8)) and (nm, ns) == (8, 0)


def test_cache_bytes(lib):
    L = Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0])
    m, s = g.kv_cache_bytes(L, 16, 131072)
    assert m == 16 * 1 * 131072 * 256 and s == 16 * 7 * 320 * 256
    m, s = g.kv_cache_bytes(Layer(kind=SLIDING, window=512), 64, 10 ** 6)
    assert m == 64 * 8 * 512 * 256 and s == 0


def _expected_tiles(layer, qa, qb, streaming):
    def tiles(lo, hi):
        return hi // 64 - lo // 64 + 1
    if not streaming:
        lo = max(0, qa - layer.window + 1) if layer.main_ring else 0
        return tiles(lo, qb)
    n = 0
    if layer.sink > 0:
        n += tiles(0, min(qb, layer.sink - 1))
    lo = max(layer.sink, qa - layer.recent + 1)
    if lo <= qb:
        n += tiles(lo, qb)
    return n


@pytest.mark.parametrize("case", [
    dict(layer=Layer(), B=2, T=1000, P=0),
    dict(layer=Layer(num_q_heads=12, num_kv_heads=2), B=1, T=1000, P=0),
    dict(layer=Layer(kind=SLIDING, window=512, num_q_heads=12, num_kv_heads=2), B=1, T=1024, P=0),
    dict(layer=Layer(full_attention_heads=[0, 0, 0, 0, 1, 0, 1, 0]), B=1, T=8192, P=16384),
    dict(layer=Layer(full_attention_heads=[0] * 8), B=3, T=77, P=5),
])
def test_prefill_plan_covers_every_tile_once_and_skips_masked(lib, case):
    L, B, T, P = case["layer"], case["B"], case["T"], case["P"]
    items = g.prefill_plan(L, B, T, P)
    real = items[items[:, 0] >= 0]
    rows = g.prefill_tile_rows(L)
    G = L.num_q_heads // L.num_kv_heads
    hpw = 2 if G % 2 == 0 else 1
    assert rows == 128 // hpw and (real[:, 6] == hpw).all()
    nqt = (T + rows - 1) // rows
    assert len(real) * hpw == B * L.num_q_heads * nqt
    heads = [(b, h + j, qt) for b, h, qt in real[:, :3] for j in range(hpw)]
    assert len(set(heads)) == len(heads) == B * L.num_q_heads * nqt
    assert all(h // G == (h + hpw - 1) // G for h in real[:, 1])  # one KV head per workgroup
    assert (real[:, 4] == 0).all() and (real[:, 5] == 1).all()  # no pieces without a workspace
    mask = L.full_attention_heads
    for b, h, qt, nt, _, _, _ in real:
        qa = P + rows * qt
        qb = min(qa + rows - 1, P + T - 1)
        streaming = mask is not None and mask[h // G] == 0
        assert nt == _expected_tiles(L, qa, qb, streaming)
    # XCD order (workgroup i runs on XCD i % 8). With whole 8-wide stripes of
    # (batch, KV head) groups, each XCD walks its own groups one at a time
    # (every unit of a group on one XCD, one contiguous run per group),
    # heaviest query tile first within the run. Otherwise all groups advance
    # together, and for a full layer the tile count never increases along an
    # XCD's sequence.
    groups_main = B * (L.num_kv_heads if mask is None else sum(1 for m in mask if m))
    xcd_of_group = {}
    for x in range(8):
        seq = [r for r in items[x::8] if r[0] >= 0]
        if mask is None and L.kind == FULL and groups_main % 8 == 0:
            keys = [(int(r[0]), int(r[1]) // G) for r in seq]
            runs = [k for i, k in enumerate(keys) if i == 0 or keys[i - 1] != k]
            assert len(runs) == len(set(runs)), "a group's units are not contiguous on its XCD"
            for k in set(keys):
                assert xcd_of_group.setdefault(k, x) == x, "a group spans two XCDs"
                nts = [int(r[3]) for r, kk in zip(seq, keys) if kk == k]
                assert all(a >= b for a, b in zip(nts, nts[1:]))
        elif mask is None and L.kind == FULL:
            nts = [int(r[3]) for r in seq]
            assert all(a >= b for a, b in zip(nts, nts[1:]))


@pytest.mark.parametrize("case", [
    dict(layer=Layer(full_attention_heads=[0, 0, 0, 0, 1, 0, 1, 0]), B=1, T=8192, P=8192 * 15),
    dict(layer=Layer(full_attention_heads=[0, 0, 0, 0, 1, 0, 1, 0]), B=1, T=8192, P=0),
    dict(layer=Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0]), B=1, T=1000, P=40000),
    dict(layer=Layer(num_q_heads=12, num_kv_heads=2), B=1, T=333, P=70000),
])
def test_prefill_plan_pieces_cover_each_query_tile_once(lib, case):
    """With a workspace, long full-context query tiles are cut into key-range
    pieces: the pieces of a (batch, head, query tile) are numbered 0..pieces-1
    and their key tiles add up to the tile's visible key tiles; streaming
    heads are never cut; the workspace covers every piece's partial."""
    L, B, T, P = case["layer"], case["B"], case["T"], case["P"]
    items = g.prefill_plan(L, B, T, P, with_workspace=True)
    real = items[items[:, 0] >= 0]
    rows = g.prefill_tile_rows(L)
    G = L.num_q_heads // L.num_kv_heads
    mask = L.full_attention_heads
    by_tile = {}
    for b, h, qt, nt, piece, pieces, hpw in real:
        for j in range(hpw):
            by_tile.setdefault((b, h + j, qt), []).append((piece, pieces, nt))
    nqt = (T + rows - 1) // rows
    assert len(by_tile) == B * L.num_q_heads * nqt
    cut = 0
    for (b, h, qt), ps in by_tile.items():
        qa = P + rows * qt
        qb = min(qa + rows - 1, P + T - 1)
        streaming = mask is not None and mask[h // G] == 0
        used = {p[1] for p in ps}
        assert len(used) == 1
        used = used.pop()
        nonempty = sorted(p[0] for p in ps if p[2] > 0)
        assert nonempty == list(range(used))
        assert sum(p[2] for p in ps) == _expected_tiles(L, qa, qb, streaming)
        if streaming:
            assert used == 1
        cut += used > 1
    nbytes = g.prefill_workspace_bytes(L, B, T, P)
    if cut:
        n_pieces = max(p[0] for ps in by_tile.values() for p in ps) + 1
        n_main_wgs = B * L.n_main * nqt * G // int(real[0, 6])
        assert nbytes >= n_main_wgs * n_pieces * (4 * 2 * 8 * 64 * 4 + 4 * 2 * 16 * 2) * 4
    else:
        assert nbytes == 0
    if P == 8192 * 15:
        assert cut  # the long chunk is cut


def test_decode_plan(lib):
    sk, items = g.decode_plan(Layer(kind=SLIDING, window=512), 64, 32768)
    assert sk >= 128 and sk % 32 == 0
    assert len(items) == 64 * 8 * ((512 + sk - 1) // sk)
    L = Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0])
    sk, items = g.decode_plan(L, 16, 131072)
    full = items[items[:, 3] == 0]
    stream = items[items[:, 3] == 1]
    assert len(full) == 16 * ((131072 + sk - 1) // sk)
    assert len(stream) == 16 * 7 * ((320 + sk - 1) // sk)
    assert set(full[:, 1].tolist()) == {0} and set(stream[:, 1].tolist()) == set(range(1, 8))
    assert (items[:, 3][:len(full)] == 0).all()   # main-class (long) items come first


def test_visible_pairs_closed_forms(lib):
    """bench.py's algorithmic FLOP count against the figures derived by hand
    for the 1 x 1024 sliding prefill and the 4 x 8192 full prefill, and
    against a direct sum of |Vis(i)| for a chunk of a Duo layer."""
    import bench
    L = Layer(kind=SLIDING, window=512, num_q_heads=12, num_kv_heads=2)
    assert bench.prefill_flops(g, L, 1, 1024) == 2417491968
    assert bench.prefill_flops(g, Layer(), 4, 8192) == 3298937536512
    D = Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 1])
    direct = 0
    for i in range(300, 300 + 700):
        direct += 2 * (i + 1) * 6 + 6 * 6 * min(i + 1, 64 + 256)
    assert bench.prefill_flops(g, D, 1, 700, 300) == 4 * 128 * direct


def test_epilogue_validation_errors(lib):
    """Bad epilogues are refused on the host before any launch."""
    q = FakeTensor((1, 8, 48, 128))
    kv = FakeTensor((1, 8, 8, 128))
    o = FakeTensor((1, 8, 48, 128))
    # gate shaped neither like out nor like out without its last dimension
    with pytest.raises(ValueError):
        g.attn_prefill(Layer(), q, kv, kv, o, gate=FakeTensor((1, 8, 48, 64), 0x800000), stream=0)
    # misaligned gate / sink logits
    assert _err(g.attn_prefill, Layer(), q, kv, kv, o, gate=FakeTensor(o.shape, 0x800008), stream=0) == -1
    assert _err(g.attn_prefill, Layer(), q, kv, kv, o, sink_logits=FakeTensor((48,), 0x700002), stream=0) == -1
    # gate_mode without a gate, a gate without a mode, an unknown mode
    for sl, gate, mode in ((0, 0, 1), (0, 0x800000, 0), (0, 0x800000, 3)):
        e = g._Epilogue(sl, gate, mode)
        rc = lib.load().duo_attn_prefill(ctypes.byref(Layer()._c()), None, 1, q.data_ptr(), kv.data_ptr(),
                                         kv.data_ptr(), 8, 0, o.data_ptr(), None, None, 0, None,
                                         ctypes.byref(e), None)
        assert rc == -1, (sl, gate, mode)
        assert "gate" in lib.load().duo_last_error().decode()
    # decode and block decode check the epilogue too
    qd, sl_ = FakeTensor((4, 48, 128)), FakeTensor((4,))
    ws = FakeTensor((g.decode_workspace_bytes(Layer(), 4, 1000) // 4,), 0x600000)
    assert _err(g.attn_decode, Layer(), FakeCache(cap=1000), qd, sl_, 1000, qd, ws,
                gate=FakeTensor((4, 48), 0x800004), stream=0) == -1
    qb = FakeTensor((4, 2, 48, 128))
    kvb = FakeTensor((4, 2, 8, 128))
    wsb = FakeTensor((g.decode_block_workspace_bytes(Layer(), 4, 2, 1000) // 4,), 0x600000)
    assert _err(g.attn_decode_block, Layer(), FakeCache(cap=1000), qb, kvb, kvb, sl_, 1000, qb, wsb,
                sink_logits=FakeTensor((48,), 0x700001), stream=0) == -1


def test_prologue_validation_errors(lib):
    """Bad prologues are refused on the host before any launch."""
    x = FakeTensor((2, 4, 8, 128))
    sp = FakeTensor((2,))
    bad = [
        g.Prologue(rope=g.Rope(theta=1.0)),
        g.Prologue(rope=g.Rope(factor=float("nan"))),
        g.Prologue(rope=g.Rope(attention_factor=0.0)),
        g.Prologue(rope=g.Rope(beta_fast=1.0, beta_slow=1.0)),
        g.Prologue(rope=g.Rope(original_max_position=0)),
        g.Prologue(eps=-1.0),
        g.Prologue(norm_weight=FakeTensor((128,), 0x700002)),
    ]
    for pro in bad:
        assert _err(g.qk_prologue, pro, x, sp, stream=0) == -1, pro
        assert _err(g.kv_append, Layer(), FakeCache(), x, x, sp, max_end_pos=16, k_prologue=pro, stream=0) == -1
        q = FakeTensor((2, 4, 48, 128))
        assert _err(g.attn_prefill, Layer(), q, x, x, q, q_prologue=pro, stream=0) == -1
    # plain RoPE with factor <= 1 needs no YaRN fields
    assert len(g.rope_frequencies(g.Rope(theta=10000.0, factor=1.0, original_max_position=0, beta_fast=0,
                                         beta_slow=0))) == 64
    assert _err(g.qk_prologue, g.Prologue(), FakeTensor((2, 4, 8, 128), 0x100008), sp, stream=0) == -1


@pytest.mark.parametrize("rope", [dict(), dict(factor=1.0), dict(theta=10000.0, factor=8.0, original_max_position=2048,
                                                                  beta_fast=32.0, beta_slow=1.0),
                                  dict(factor=4.0, beta_fast=2.0, beta_slow=1.5)])
def test_rope_frequencies_match_the_oracle(lib, rope):
    """The library's host-computed rotary frequencies (YaRN blend included)
    against the oracle's, two independent implementations of the same
    published formula."""
    import oracle
    r = g.Rope(**rope)
    got = np.array(g.rope_frequencies(r))
    want = oracle.rope_frequencies(np.float64(np.float32(r.theta)), float(np.float32(r.factor)),
                                   r.original_max_position, float(np.float32(r.beta_fast)),
                                   float(np.float32(r.beta_slow)))
    assert np.allclose(got, want, rtol=1e-13, atol=0)


def test_position_limit(lib):
    """Positions stay 1024 below 2^31 (32-bit device positions with tile
    bounds formed past the last one)."""
    top = (1 << 31) - 1 - 1024
    q = FakeTensor((1, 8, 48, 128))
    kv = FakeTensor((1, 8, 8, 128))
    L = Layer(kind=SLIDING, window=512)
    ring = FakeCache(cap=512)
    # the last allowed chunk (start_pos + num_tokens = top) passes the position
    # check and is refused only for its misaligned lse, so nothing launches
    assert _err(g.attn_prefill, L, q, kv, kv, q, start_pos=top - 8, past=ring, stream=0, lse=FakeTensor((1,), 2)) == -1
    assert "lse" in lib.load().duo_last_error().decode()
    assert _err(g.attn_prefill, L, q, kv, kv, q, start_pos=top - 7, past=ring, stream=0) == -1
    assert "positions exceed" in lib.load().duo_last_error().decode()
    assert _err(g.kv_append, L, ring, kv, kv, FakeTensor((1,)), max_end_pos=top + 1, stream=0) == -1
    assert g.decode_workspace_bytes(L, 4, top) > 0
    assert g.decode_workspace_bytes(L, 4, top + 1) == 0


def test_binding_rejects_misshaped_tensors():
    """The binding checks dtype, shape, packing and device of torch tensors
    before any call: the C ABI sees bare pointers and could not."""
    import torch
    L = Layer()
    q = torch.zeros(1, 8, 48, 128, dtype=torch.bfloat16)
    kv = torch.zeros(1, 8, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        g.attn_prefill(L, q.float(), kv, kv, q, stream=0)
    with pytest.raises(ValueError, match="shape"):
        g.attn_prefill(L, q, torch.zeros(1, 8, 4, 128, dtype=torch.bfloat16), kv, q, stream=0)
    with pytest.raises(ValueError, match="shape"):
        g.attn_prefill(L, q, kv, kv, q, lse=torch.zeros(1, 8, 48), stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        g.attn_prefill(L, q, kv, kv, q.transpose(1, 2).contiguous().transpose(1, 2), stream=0)
    with pytest.raises(ValueError, match="device memory"):
        g.attn_prefill(L, q, kv, kv, q, stream=0)
    with pytest.raises(ValueError, match="sink_logits"):
        g.attn_prefill(L, q, kv, kv, q, sink_logits=torch.zeros(8), stream=0)
    qd = torch.zeros(2, 48, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="seq_lens"):
        g.attn_decode(L, FakeCache(), qd, torch.zeros(2, dtype=torch.int64), 16, qd, FakeTensor((64,)), stream=0)
    with pytest.raises(ValueError, match="start_pos"):
        g.kv_append(L, FakeCache(), kv, kv, torch.zeros(1, dtype=torch.int64), max_end_pos=16, stream=0)
    with pytest.raises(ValueError, match="leading extent"):
        g.kv_append(L, FakeCache(), kv, kv, torch.zeros(0, dtype=torch.int32), max_end_pos=16, stream=0)
    with pytest.raises(ValueError, match="norm_weight"):
        g.qk_prologue(g.Prologue(norm_weight=torch.zeros(64)), q, torch.zeros(1, dtype=torch.int32))


@pytest.mark.parametrize("other", [
    dict(full_attention_heads=[1, 1, 0, 0, 0, 0, 0, 0]),          # another class split
    dict(full_attention_heads=[0, 1, 0, 0, 0, 0, 0, 0]),          # same counts, other heads
    dict(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0], sink=32),  # shorter sink + recent ring
    dict(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0], recent=128),
    dict(kind=SLIDING, window=512),                               # a ring where a full cache was built
    dict(),                                                       # no Duo routing: every head full
])
def test_binding_rejects_a_cache_built_for_another_layer(lib, other):
    """A KVCache keeps its layer: a call with a layer of other head classes,
    sink/recent or window is refused before the C ABI, which only sees the
    cache's pointers and would read and write past its tensors."""
    import torch
    built = Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0])
    cache = g.KVCache(built, 2, 64, device="cpu")
    call = Layer(**other)
    kv = torch.zeros(2, 4, 8, 128, dtype=torch.bfloat16)
    sp = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="another layer geometry"):
        g.kv_append(call, cache, kv, kv, sp, max_end_pos=4, stream=0)
    q = torch.zeros(2, 48, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="another layer geometry"):
        g.attn_decode(call, cache, q, sp, 16, q, torch.zeros(64), stream=0)
    qp = torch.zeros(2, 4, 48, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="another layer geometry"):
        g.attn_prefill(call, qp, kv, kv, qp, start_pos=8, past=cache, stream=0)
    # the layer it was built for passes the cache checks (and stops at the
    # device check: these are host tensors)
    with pytest.raises(ValueError, match="device memory"):
        g.kv_append(built, cache, kv, kv, sp, max_end_pos=4, stream=0)


def test_binding_rejects_a_resized_cache_tensor(lib):
    import torch
    L = Layer(full_attention_heads=[1, 0, 0, 0, 0, 0, 0, 0])
    cache = g.KVCache(L, 1, 64, device="cpu")
    cache.k_stream = torch.zeros(1, 7, 100, 128, dtype=torch.bfloat16)
    kv = torch.zeros(1, 4, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="k_stream"):
        g.kv_append(L, cache, kv, kv, torch.zeros(1, dtype=torch.int32), max_end_pos=4, stream=0)


def test_noalloc_decode_refuses_sizes_beyond_its_scratch(lib):
    """duo_attn_decode_noalloc keeps its partials in 32 MiB of library-held
    scratch: a decode whose workspace would be larger is refused on the host,
    with the sizes in the message, before any launch."""
    L = Layer()
    B, maxlen = 2048, 1024
    need = g.decode_workspace_bytes(L, B, maxlen)
    assert need > 32 << 20
    q = FakeTensor((B, 48, 128))
    sl = FakeTensor((B,))
    rc = lib.load().duo_attn_decode_noalloc(ctypes.byref(L._c()), ctypes.byref(FakeCache(cap=maxlen)._c()), B,
                                            q.data_ptr(), sl.data_ptr(), maxlen, q.data_ptr(), None, None, None,
                                            None)
    assert rc == -4
    msg = lib.load().duo_last_error().decode()
    assert str(need) in msg and str(32 << 20) in msg
    # within the limit the host-side checks pass on to the usual argument errors
    assert lib.load().duo_attn_decode_noalloc(ctypes.byref(L._c()), ctypes.byref(FakeCache(cap=1000)._c()), 4,
                                              q.data_ptr(), None, 1000, q.data_ptr(), None, None, None,
                                              None) == -1
