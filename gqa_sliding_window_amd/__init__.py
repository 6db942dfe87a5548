"""Python binding of the duo_attn C ABI (include/duo_attn.h).

Argument marshalling only: every step of the attention path runs in the HIP
kernels of libduoattn.so. Torch tensors supply device pointers and the
current HIP stream. There is no fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libduoattn.so")

FULL = 0
SLIDING = 1
HEAD_DIM = 128

DUO_OK = 0
# duo_device_errors bits
DEVICE_APPEND_PAST_CAPACITY = 1
DEVICE_LENGTH_PAST_CAPACITY = 2
DEVICE_LENGTH_PAST_PLAN = 4
ERRORS = {-1: "DUO_ERR_INVALID_ARG", -2: "DUO_ERR_UNSUPPORTED", -3: "DUO_ERR_CAPACITY",
          -4: "DUO_ERR_WORKSPACE", -5: "DUO_ERR_HIP"}


class DuoError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class _Layer(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("sink", ctypes.c_int32), ("recent", ctypes.c_int32),
                ("full_attention_heads", ctypes.POINTER(ctypes.c_uint8)), ("scale", ctypes.c_float)]


class _Cache(ctypes.Structure):
    _fields_ = [("k_main", ctypes.c_void_p), ("v_main", ctypes.c_void_p),
                ("main_capacity", ctypes.c_int64),
                ("k_stream", ctypes.c_void_p), ("v_stream", ctypes.c_void_p)]


class _Epilogue(ctypes.Structure):
    _fields_ = [("sink_logits", ctypes.c_void_p), ("gate", ctypes.c_void_p), ("gate_mode", ctypes.c_int32)]


GATE_NONE, GATE_PER_ELEMENT, GATE_PER_HEAD = 0, 1, 2


class _Rope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_float), ("factor", ctypes.c_float), ("original_max_position", ctypes.c_int32),
                ("beta_fast", ctypes.c_float), ("beta_slow", ctypes.c_float), ("attention_factor", ctypes.c_float)]


class _Prologue(ctypes.Structure):
    _fields_ = [("norm_weight", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("rope", ctypes.POINTER(_Rope))]


@dataclass
class Rope:
    """Rotary settings (duo_rope). The defaults are the YaRN parameters the
    Laguna-M.1-8bit post prints for full-attention layers; factor <= 1 gives
    plain RoPE."""
    theta: float = 500000.0
    factor: float = 64.0
    original_max_position: int = 4096
    beta_fast: float = 64.0
    beta_slow: float = 1.0
    attention_factor: float = 1.0


@dataclass
class Prologue:
    """RMSNorm weight (device float32 [128] or None) and rotary settings
    (Rope or None) applied to q or k (duo_prologue)."""
    norm_weight: object = None
    eps: float = 1e-6
    rope: Optional[Rope] = None

    def _c(self):
        r = None
        if self.rope is not None:
            self._rope_c = _Rope(self.rope.theta, self.rope.factor, self.rope.original_max_position,
                                 self.rope.beta_fast, self.rope.beta_slow, self.rope.attention_factor)
            r = ctypes.pointer(self._rope_c)
        return _Prologue(_ptr(self.norm_weight), float(self.eps), r)


def _prologue(pro: Optional[Prologue]):
    return None if pro is None else ctypes.byref(pro._c())

_lib = None


def load(path: str = LIB_PATH):
    """Load libduoattn.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with gqa_sliding_window_amd.build.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    LP, CP, EP = ctypes.POINTER(_Layer), ctypes.POINTER(_Cache), ctypes.POINTER(_Epilogue)
    PP = ctypes.POINTER(_Prologue)
    I32P, I64P = ctypes.POINTER(i32), ctypes.POINTER(i64)
    sigs = {
        "duo_kv_append": (ctypes.c_int, [LP, CP, i32, P, P, i32, P, i64, PP, P]),
        "duo_attn_prefill": (ctypes.c_int, [LP, CP, i32, P, P, P, i32, i64, P, P, P, sz, PP, EP, P]),
        "duo_attn_prefill_workspace_bytes": (sz, [LP, i32, i32, i64]),
        "duo_attn_decode": (ctypes.c_int, [LP, CP, i32, P, P, i64, P, P, P, sz, PP, EP, P]),
        "duo_attn_decode_noalloc": (ctypes.c_int, [LP, CP, i32, P, P, i64, P, P, PP, EP, P]),
        "duo_qk_prologue": (ctypes.c_int, [PP, i32, i32, i32, P, P, P, P]),
        "duo_rope_frequencies": (ctypes.c_int, [ctypes.POINTER(_Rope), ctypes.POINTER(ctypes.c_double)]),
        "duo_attn_decode_workspace_bytes": (sz, [LP, i32, i64]),
        "duo_attn_decode_block": (ctypes.c_int, [LP, CP, i32, P, P, P, i32, P, i64, P, P, P, sz, PP, EP, P]),
        "duo_attn_decode_block_workspace_bytes": (sz, [LP, i32, i32, i64]),
        "duo_attn_decode_workspace_init": (ctypes.c_int, [P, sz, P]),
        "duo_kv_cache_bytes": (ctypes.c_int, [LP, i32, i64, I64P, I64P]),
        "duo_kv_cache_report": (ctypes.c_int, [LP, i32, i64, I32P, ctypes.POINTER(_CacheReport)]),
        "duo_head_plan": (ctypes.c_int, [LP, I32P, I32P, I32P, I32P]),
        "duo_prefill_plan": (ctypes.c_int, [LP, i32, i32, i64, i32, I32P, I64P]),
        "duo_decode_plan": (ctypes.c_int, [LP, i32, i64, I32P, I32P, I64P]),
        "duo_last_error": (ctypes.c_char_p, []),
        "duo_attn_version": (ctypes.c_int, []),
        "duo_prefill_tile_rows": (ctypes.c_int, [LP]),
        "duo_device_errors": (ctypes.c_int, [ctypes.POINTER(ctypes.c_uint32), i32]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != DUO_OK:
        raise DuoError(rc, load().duo_last_error().decode())


@dataclass
class Layer:
    """One attention layer (see duo_layer in include/duo_attn.h)."""
    num_q_heads: int = 48
    num_kv_heads: int = 8
    kind: int = FULL
    window: int = 0
    sink: int = 64
    recent: int = 256
    full_attention_heads: Optional[Sequence[int]] = None
    scale: float = 0.0
    head_dim: int = HEAD_DIM

    def _c(self):
        mask = None
        if self.full_attention_heads is not None:
            arr = (ctypes.c_uint8 * len(self.full_attention_heads))(*[int(x) for x in self.full_attention_heads])
            mask = ctypes.cast(arr, ctypes.POINTER(ctypes.c_uint8))
            self._keep = arr  # keep alive for the call
        return _Layer(self.num_q_heads, self.num_kv_heads, self.head_dim, self.kind, self.window,
                      self.sink, self.recent, mask, float(self.scale))

    @property
    def n_main(self) -> int:
        """Full-context KV heads, from the library's head-class plan."""
        return head_plan(self)[2]

    @property
    def n_stream(self) -> int:
        """Streaming KV heads, from the library's head-class plan."""
        return head_plan(self)[3]

    @property
    def main_ring(self) -> bool:
        return self.kind == SLIDING and self.window > 0


def _ptr(t) -> int:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _need(t, name: str, shape, dtype: str):
    """Reject a tensor that the kernels would misread: wrong dtype or shape
    (None in `shape` matches any extent) or not densely packed (its device
    is checked by _need_device). The C ABI takes bare pointers and cannot check these.
    Anything that is not a torch tensor (a raw address, an object with a
    data_ptr) passes unchecked."""
    import torch
    if not isinstance(t, torch.Tensor):
        return
    want = getattr(torch, dtype)
    if t.dtype != want:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {want}")
    if shape is not None:
        got = tuple(t.shape)
        if len(got) != len(shape) or any(w is not None and g != w for g, w in zip(got, shape)):
            exp = tuple("*" if w is None else w for w in shape)
            raise ValueError(f"{name}: shape {got}, expected {exp}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_device(**tensors):
    """Every torch tensor given is in device memory (checked after the
    dtype and shape checks of all arguments)."""
    import torch
    for name, t in tensors.items():
        if isinstance(t, torch.Tensor) and not t.is_cuda:
            raise ValueError(f"{name} must be in device memory")


def _need_batch(t, name: str, batch: int):
    """t's leading extent covers `batch` sequences."""
    import torch
    if isinstance(t, torch.Tensor) and t.shape[0] < batch:
        raise ValueError(f"{name}: leading extent {t.shape[0]} < batch {batch}")


def _cache_geometry(layer: "Layer"):
    """What fixes a cache's extents and slot contract for a layer: KV heads,
    which of them stream, the ring of a sliding layer, sink and recent."""
    streaming = tuple(c == 1 for c in head_plan(layer)[0])
    return {"num_kv_heads": layer.num_kv_heads, "streaming_heads": streaming, "main_ring": layer.main_ring,
            "window": layer.window if layer.main_ring else 0, "sink": layer.sink, "recent": layer.recent}


def _layer_key(layer: "Layer"):
    mask = None if layer.full_attention_heads is None else tuple(int(x) for x in layer.full_attention_heads)
    return (layer.num_q_heads, layer.num_kv_heads, layer.head_dim, layer.kind, layer.window, layer.sink,
            layer.recent, mask)


def _need_cache(cache, layer: "Layer", batch: int, batch_offset: int = 0):
    """A KVCache used by a call must cover its batch rows and have been built
    for a layer with the same head classes and sizes: the C ABI receives bare
    pointers, and a cache with fewer heads of a class, a shorter sink + recent
    ring or another window would be read and written past its tensors."""
    if not isinstance(cache, KVCache):
        return
    if batch_offset < 0 or batch_offset + batch > cache.batch:
        raise ValueError(f"cache holds {cache.batch} sequences; the call uses [{batch_offset}, {batch_offset + batch})")
    # checked once per (layer, cache tensors): the per-call cost stays far
    # below a decode kernel's
    key = (_layer_key(layer), id(cache.k_main), id(cache.v_main), id(cache.k_stream), id(cache.v_stream))
    if key in cache._checked:
        return
    want, have = _cache_geometry(layer), _cache_geometry(cache.layer)
    diff = [k for k in want if want[k] != have[k]]
    if diff:
        raise ValueError("cache was built for another layer geometry: "
                         + ", ".join(f"{k} {have[k]} (call: {want[k]})" for k in diff))
    nm, ns, sr = layer.n_main, layer.n_stream, layer.sink + layer.recent
    for t, name, shape in ((cache.k_main, "k_main", (cache.batch, nm, cache.capacity, HEAD_DIM)),
                           (cache.v_main, "v_main", (cache.batch, nm, cache.capacity, HEAD_DIM)),
                           (cache.k_stream, "k_stream", (cache.batch, ns, sr, HEAD_DIM)),
                           (cache.v_stream, "v_stream", (cache.batch, ns, sr, HEAD_DIM))):
        if shape[1] == 0:
            continue
        if t is None or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"cache.{name}: {None if t is None else tuple(t.shape)}, expected {shape} contiguous")
    cache._checked.add(key)


def _need_prologue(pro, name: str):
    if pro is not None:
        _need(pro.norm_weight, f"{name}.norm_weight", (HEAD_DIM,), "float32")
        _need_device(**{f"{name}.norm_weight": pro.norm_weight})


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


class KVCache:
    """A layer's static KV cache in device memory (torch tensors, bf16)."""

    def __init__(self, layer: Layer, batch: int, capacity: int, device="cuda", zero=True):
        import torch
        self.layer = layer
        self.batch = batch
        self._checked = set()
        self.capacity = layer.window if layer.main_ring else capacity
        alloc = torch.zeros if zero else torch.empty
        nm, ns = layer.n_main, layer.n_stream
        sr = layer.sink + layer.recent
        self.k_main = alloc((batch, nm, self.capacity, HEAD_DIM), dtype=torch.bfloat16, device=device) if nm else None
        self.v_main = alloc((batch, nm, self.capacity, HEAD_DIM), dtype=torch.bfloat16, device=device) if nm else None
        self.k_stream = alloc((batch, ns, sr, HEAD_DIM), dtype=torch.bfloat16, device=device) if ns else None
        self.v_stream = alloc((batch, ns, sr, HEAD_DIM), dtype=torch.bfloat16, device=device) if ns else None

    def _c(self, batch_offset: int = 0):
        def off(t):
            if t is None:
                return None
            return t[batch_offset].data_ptr() if batch_offset else t.data_ptr()
        return _Cache(off(self.k_main), off(self.v_main), self.capacity,
                      off(self.k_stream), off(self.v_stream))


def kv_append(layer: Layer, cache: KVCache, k_new, v_new, start_pos, max_end_pos: int,
              batch: Optional[int] = None, batch_offset: int = 0, stream=None,
              k_prologue: Optional[Prologue] = None):
    """duo_kv_append: k_new/v_new [B, T, Hkv, 128] bf16, start_pos int32 [B]
    (device); k_prologue transforms K on its way into the cache."""
    B = k_new.shape[0] if batch is None else batch
    T = k_new.shape[1]
    hkv = layer.num_kv_heads
    _need(k_new, "k_new", (None, T, hkv, HEAD_DIM), "bfloat16")
    _need(v_new, "v_new", (None, T, hkv, HEAD_DIM), "bfloat16")
    _need(start_pos, "start_pos", (None,), "int32")
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (start_pos, "start_pos")):
        _need_batch(t, n, B)
    _need_cache(cache, layer, B, batch_offset)
    _need_prologue(k_prologue, "k_prologue")
    _need_device(k_new=k_new, v_new=v_new, start_pos=start_pos)
    lib = load()
    cl, cc = layer._c(), cache._c(batch_offset)
    _check(lib.duo_kv_append(ctypes.byref(cl), ctypes.byref(cc), B, _ptr(k_new), _ptr(v_new), T,
                             _ptr(start_pos), int(max_end_pos), _prologue(k_prologue), _stream(stream)))


def rope_frequencies(rope: Rope):
    """duo_rope_frequencies: the 64 rotary angular frequencies (host)."""
    out = (ctypes.c_double * 64)()
    r = _Rope(rope.theta, rope.factor, rope.original_max_position, rope.beta_fast, rope.beta_slow,
              rope.attention_factor)
    _check(load().duo_rope_frequencies(ctypes.byref(r), out))
    return list(out)


def qk_prologue(prologue: Prologue, x, start_pos, y=None, stream=None):
    """duo_qk_prologue: y = prologue(x) for x [B, T, H, 128] bf16 at
    positions start_pos[b] + t (start_pos int32 [B], device); in place when
    y is None. Returns y."""
    y = x if y is None else y
    B, T, H = x.shape[0], x.shape[1], x.shape[2]
    _need(x, "x", (B, T, H, HEAD_DIM), "bfloat16")
    _need(y, "y", (B, T, H, HEAD_DIM), "bfloat16")
    _need(start_pos, "start_pos", (B,), "int32")
    _need_prologue(prologue, "prologue")
    _need_device(x=x, y=y, start_pos=start_pos)
    _check(load().duo_qk_prologue(_prologue(prologue), B, T, H, _ptr(x), _ptr(y), _ptr(start_pos),
                                  _stream(stream)))
    return y


def _epilogue(out, sink_logits, gate):
    """duo_epilogue for the call, or None. sink_logits: float32 [Hq];
    gate: bf16 shaped like `out` (one value per element) or like `out`
    without its last dimension (one value per row and head)."""
    if sink_logits is None and gate is None:
        return None
    hq = out.shape[-2]
    _need(sink_logits, "sink_logits", (hq,), "float32")
    mode = GATE_NONE
    if gate is not None:
        _need(gate, "gate", None, "bfloat16")
        if tuple(gate.shape) == tuple(out.shape):
            mode = GATE_PER_ELEMENT
        elif tuple(gate.shape) == tuple(out.shape[:-1]):
            mode = GATE_PER_HEAD
        else:
            raise ValueError(f"gate shape {tuple(gate.shape)} matches neither {tuple(out.shape)} "
                             f"nor {tuple(out.shape[:-1])}")
    _need_device(sink_logits=sink_logits, gate=gate)
    return ctypes.byref(_Epilogue(_ptr(sink_logits), _ptr(gate), mode))


def attn_prefill(layer: Layer, q, k, v, out, start_pos: int = 0, past: Optional[KVCache] = None,
                 lse=None, stream=None, sink_logits=None, gate=None, q_prologue: Optional[Prologue] = None,
                 workspace=None):
    """duo_attn_prefill: q [B, T, Hq, 128], k/v [B, T, Hkv, 128], out like q;
    optional attention-sink logits and output gate (see _epilogue); an
    optional zero-initialised workspace (prefill_workspace) lets the library
    cut long query tiles into key-range pieces."""
    B, T = q.shape[0], q.shape[1]
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    _need(q, "q", (B, T, hq, HEAD_DIM), "bfloat16")
    _need(k, "k", (B, T, hkv, HEAD_DIM), "bfloat16")
    _need(v, "v", (B, T, hkv, HEAD_DIM), "bfloat16")
    _need(out, "out", (B, T, hq, HEAD_DIM), "bfloat16")
    _need(lse, "lse", (B, hq, T), "float32")
    _need_prologue(q_prologue, "q_prologue")
    if past is not None:
        _need_cache(past, layer, B)
    epi = _epilogue(out, sink_logits, gate)
    _need(workspace, "workspace", None, "float32")
    _need_device(q=q, k=k, v=v, out=out, lse=lse, workspace=workspace)
    lib = load()
    cl = layer._c()
    cc = past._c() if past is not None else None
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.duo_attn_prefill(ctypes.byref(cl), ctypes.byref(cc) if cc is not None else None, B,
                                _ptr(q), _ptr(k), _ptr(v), T, int(start_pos), _ptr(out), _ptr(lse),
                                _ptr(workspace), nbytes, _prologue(q_prologue), epi, _stream(stream)))


def prefill_workspace_bytes(layer: Layer, batch: int, num_tokens: int, start_pos: int = 0) -> int:
    """duo_attn_prefill_workspace_bytes (0: no query tile would be cut)."""
    cl = layer._c()
    return int(load().duo_attn_prefill_workspace_bytes(ctypes.byref(cl), batch, int(num_tokens), int(start_pos)))


def prefill_workspace(layer: Layer, batch: int, num_tokens: int, start_positions, device="cuda"):
    """A zero-filled prefill workspace large enough for chunks of num_tokens
    tokens at each of the given start positions (None if none needs one)."""
    import torch
    need = max(prefill_workspace_bytes(layer, batch, num_tokens, int(p)) for p in start_positions)
    if need == 0:
        return None
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=device)
    init_decode_workspace(ws)
    return ws


def decode_workspace_bytes(layer: Layer, batch: int, max_seq_len: int) -> int:
    cl = layer._c()
    return int(load().duo_attn_decode_workspace_bytes(ctypes.byref(cl), batch, int(max_seq_len)))


def decode_workspace(layer: Layer, batch: int, max_seq_len: int, device="cuda"):
    """A zero-filled decode workspace (float32 tensor, 256-byte aligned by the
    caching allocator)."""
    import torch
    n = (decode_workspace_bytes(layer, batch, max_seq_len) + 3) // 4
    ws = torch.empty(max(n, 64), dtype=torch.float32, device=device)
    init_decode_workspace(ws)
    return ws


def init_decode_workspace(ws, stream=None):
    nbytes = ws.numel() * ws.element_size()
    _check(load().duo_attn_decode_workspace_init(_ptr(ws), nbytes, _stream(stream)))


def attn_decode(layer: Layer, cache: KVCache, q, seq_lens, max_seq_len: int, out, workspace,
                lse=None, stream=None, sink_logits=None, gate=None, q_prologue: Optional[Prologue] = None):
    """duo_attn_decode: q [B, Hq, 128], seq_lens int32 [B] (device), out like q."""
    B = q.shape[0]
    hq = layer.num_q_heads
    _need(q, "q", (B, hq, HEAD_DIM), "bfloat16")
    _need(seq_lens, "seq_lens", (B,), "int32")
    _need(out, "out", (B, hq, HEAD_DIM), "bfloat16")
    _need(lse, "lse", (B, hq), "float32")
    _need(workspace, "workspace", None, "float32")
    _need_prologue(q_prologue, "q_prologue")
    _need_cache(cache, layer, B)
    epi = _epilogue(out, sink_logits, gate)
    _need_device(q=q, seq_lens=seq_lens, out=out, lse=lse, workspace=workspace)
    lib = load()
    cl, cc = layer._c(), cache._c()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.duo_attn_decode(ctypes.byref(cl), ctypes.byref(cc), B, _ptr(q), _ptr(seq_lens),
                               int(max_seq_len), _ptr(out), _ptr(lse), _ptr(workspace), nbytes,
                               _prologue(q_prologue), epi, _stream(stream)))


def attn_decode_noalloc(layer: Layer, cache: KVCache, q, seq_lens, max_seq_len: int, out, lse=None,
                        stream=None, sink_logits=None, gate=None, q_prologue: Optional[Prologue] = None):
    """duo_attn_decode_noalloc: attn_decode without a workspace (the library's
    own scratch; calls on one GPU must not overlap)."""
    B = q.shape[0]
    hq = layer.num_q_heads
    _need(q, "q", (B, hq, HEAD_DIM), "bfloat16")
    _need(seq_lens, "seq_lens", (B,), "int32")
    _need(out, "out", (B, hq, HEAD_DIM), "bfloat16")
    _need(lse, "lse", (B, hq), "float32")
    _need_prologue(q_prologue, "q_prologue")
    _need_cache(cache, layer, B)
    epi = _epilogue(out, sink_logits, gate)
    _need_device(q=q, seq_lens=seq_lens, out=out, lse=lse)
    lib = load()
    cl, cc = layer._c(), cache._c()
    _check(lib.duo_attn_decode_noalloc(ctypes.byref(cl), ctypes.byref(cc), B, _ptr(q), _ptr(seq_lens),
                                       int(max_seq_len), _ptr(out), _ptr(lse), _prologue(q_prologue), epi,
                                       _stream(stream)))


def decode_block_workspace_bytes(layer: Layer, batch: int, num_tokens: int, max_past_len: int) -> int:
    cl = layer._c()
    return int(load().duo_attn_decode_block_workspace_bytes(ctypes.byref(cl), batch, int(num_tokens),
                                                            int(max_past_len)))


def decode_block_workspace(layer: Layer, batch: int, num_tokens: int, max_past_len: int, device="cuda"):
    """A zero-filled block-decode workspace."""
    import torch
    n = (decode_block_workspace_bytes(layer, batch, num_tokens, max_past_len) + 3) // 4
    ws = torch.empty(max(n, 64), dtype=torch.float32, device=device)
    init_decode_workspace(ws)
    return ws


def attn_decode_block(layer: Layer, cache: KVCache, q, k_new, v_new, past_lens, max_past_len: int, out,
                      workspace, lse=None, stream=None, sink_logits=None, gate=None,
                      q_prologue: Optional[Prologue] = None):
    """duo_attn_decode_block: q/out [B, T, Hq, 128], k_new/v_new [B, T, Hkv, 128],
    past_lens int32 [B] (device): cached positions before the block."""
    B, T = q.shape[0], q.shape[1]
    hq, hkv = layer.num_q_heads, layer.num_kv_heads
    _need(q, "q", (B, T, hq, HEAD_DIM), "bfloat16")
    _need(k_new, "k_new", (B, T, hkv, HEAD_DIM), "bfloat16")
    _need(v_new, "v_new", (B, T, hkv, HEAD_DIM), "bfloat16")
    _need(past_lens, "past_lens", (B,), "int32")
    _need(out, "out", (B, T, hq, HEAD_DIM), "bfloat16")
    _need(lse, "lse", (B, T, hq), "float32")
    _need(workspace, "workspace", None, "float32")
    _need_prologue(q_prologue, "q_prologue")
    _need_cache(cache, layer, B)
    epi = _epilogue(out, sink_logits, gate)
    _need_device(q=q, k_new=k_new, v_new=v_new, past_lens=past_lens, out=out, lse=lse, workspace=workspace)
    lib = load()
    cl, cc = layer._c(), cache._c()
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.duo_attn_decode_block(ctypes.byref(cl), ctypes.byref(cc), B, _ptr(q), _ptr(k_new), _ptr(v_new),
                                     T, _ptr(past_lens), int(max_past_len), _ptr(out), _ptr(lse),
                                     _ptr(workspace), nbytes, _prologue(q_prologue),
                                     epi, _stream(stream)))


_plans = {}


def device_errors(clear: bool = False) -> int:
    """duo_device_errors: bits of out-of-contract device data the kernels
    clamped on the current device since the last clear (waits for the
    device)."""
    bits = ctypes.c_uint32(0)
    _check(load().duo_device_errors(ctypes.byref(bits), 1 if clear else 0))
    return int(bits.value)


def head_plan(layer: Layer):
    """duo_head_plan: (class per KV head, rank per KV head, n_main, n_stream);
    memoised per layer description."""
    key = _layer_key(layer)
    hit = _plans.get(key)
    if hit is not None:
        return list(hit[0]), list(hit[1]), hit[2], hit[3]
    lib = load()
    n = layer.num_kv_heads
    cls, rank = (ctypes.c_int32 * n)(), (ctypes.c_int32 * n)()
    nm, ns = ctypes.c_int32(), ctypes.c_int32()
    cl = layer._c()
    _check(lib.duo_head_plan(ctypes.byref(cl), cls, rank, ctypes.byref(nm), ctypes.byref(ns)))
    _plans[key] = (tuple(cls), tuple(rank), nm.value, ns.value)
    return list(cls), list(rank), nm.value, ns.value


def prefill_tile_rows(layer: Layer) -> int:
    """Query rows per prefill work item of this layer (64 or 128)."""
    cl = layer._c()
    rows = int(load().duo_prefill_tile_rows(ctypes.byref(cl)))
    if rows < 0:
        _check(rows)
    return rows


def prefill_plan(layer: Layer, batch: int, num_tokens: int, start_pos: int = 0, with_workspace: bool = False):
    """Per workgroup (batch, q_head, q_tile, key_tiles, piece, pieces, heads);
    padding rows are (-1, -1, -1, 0, 0, 0, 0)."""
    import numpy as np
    lib = load()
    cl = layer._c()
    n = ctypes.c_int64()
    ws = 1 if with_workspace else 0
    _check(lib.duo_prefill_plan(ctypes.byref(cl), batch, num_tokens, start_pos, ws, None, ctypes.byref(n)))
    items = np.zeros((n.value, 7), dtype=np.int32)
    _check(lib.duo_prefill_plan(ctypes.byref(cl), batch, num_tokens, start_pos, ws,
                                items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n)))
    return items


def decode_plan(layer: Layer, batch: int, max_seq_len: int):
    """(split_keys, items[n, 4] = (batch, kv_head, split, class))."""
    import numpy as np
    lib = load()
    cl = layer._c()
    n, sk = ctypes.c_int64(), ctypes.c_int32()
    _check(lib.duo_decode_plan(ctypes.byref(cl), batch, max_seq_len, ctypes.byref(sk), None, ctypes.byref(n)))
    items = np.zeros((n.value, 4), dtype=np.int32)
    _check(lib.duo_decode_plan(ctypes.byref(cl), batch, max_seq_len, ctypes.byref(sk),
                               items.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(n)))
    return sk.value, items


def kv_cache_bytes(layer: Layer, batch: int, capacity: int):
    lib = load()
    cl = layer._c()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    _check(lib.duo_kv_cache_bytes(ctypes.byref(cl), batch, capacity, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


class _CacheReport(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "main_slots", "stream_slots", "main_active", "stream_active", "main_bytes", "stream_bytes",
        "base_slots", "base_active", "base_bytes")]


def kv_cache_report(layer: Layer, batch: int, capacity: int, seq_lens) -> dict:
    """Allocated / occupied slots and K+V bytes per head class for host
    lengths seq_lens[batch], beside the same layer without Duo routing."""
    import numpy as np
    lib = load()
    cl = layer._c()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if lens.shape != (batch,):
        raise ValueError("seq_lens must have shape (batch,)")
    rep = _CacheReport()
    _check(lib.duo_kv_cache_report(ctypes.byref(cl), batch, capacity,
                                   lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ctypes.byref(rep)))
    return {n: getattr(rep, n) for n, _ in _CacheReport._fields_}
