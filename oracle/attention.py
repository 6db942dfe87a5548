"""Float64 reference attention, written from the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring). No blocking, no online
softmax, no tiling: for each query row the visible key positions are listed,
the logits are formed, a softmax is taken and the weighted sum of values is
returned, all in float64 on the exact bf16 values the GPU receives.

Readings of the pages (where they are silent or disagree), used throughout:

R1 Window width. The blog post on Laguna-M.1-8bit (section on how the sliding
   window works) describes each token looking back over a fixed-width window;
   the SGLang cookbook (section 1) gives the window as 512. Read as: the
   window holds W positions including the query itself, j in [i-W+1, i].
R2 Causal window. The Laguna-XS-2.1 post (section on the golden rule of
   sliding-window attention) describes the window as reaching to both sides;
   the Laguna-M.1-8bit post describes only earlier tokens, and both name
   create_sliding_window_causal_mask. Read as causal.
R3 "Recent" includes the current token: j in [i-R+1, i] (model card,
   "Why It Works": streaming heads hold the newest positions).
R4 Sink and recent sets overlap for small i; the visible set is their union.
R5 Sink tokens are absolute positions 0..S-1 of the whole sequence.
R6 Query head h reads KV head floor(h / G), G = Hq / Hkv (contiguous groups;
   model card, "Changes": heads are reordered consistently across
   Q/K/V/gating/output, so query heads travel with their KV head).
R7 Routing is per KV head; all G query heads of a group share the class
   (model card, "Summary" and "Training": per-KV-head scores).
R8 The routing mask is binary, nonzero = full-context head.
R9 On a sliding layer a streaming-class head uses sink+recent and a
   full-class head uses the layer's own window.
R10 window <= 0 means no window (Laguna-M.1-8bit post, implementation
   section: sliding_window is None for non-sliding layers and 0 appears with
   all-full layer types).
R11 Default scale is 1/sqrt(D).
R12 Decode: a sequence of length L has its current token at position L-1
   already in the cache; the query attends positions 0..L-1 by the same rule.
R17 Block decode (T tokens after past_b cached positions): token t is at
   position past_b + t and attends by the same rule, so the block's rows are
   prefill rows starting at past_b.
R15 Attention sink of a sliding layer (Laguna-M.1-8bit post, section on the
   sliding-window optimisations: a learnable bias added for sliding-window
   layers): one logit per query head, in the units of the scaled logits,
   that enters the softmax normaliser with a zero value row.
R16 Output gate (same post, attention output gating; the gating options it
   lists are one gate per (head, channel) or one per head broadcast over the
   channels): the attention output times the logistic function of the gating
   projection's value. The logistic form is the plainest reading; the post
   does not name the nonlinearity.
"""
from __future__ import annotations

import numpy as np

FULL_LAYER = "full"
SLIDING_LAYER = "sliding"


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def values_f64(x) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns (converted exactly); float arrays
    are values already (for instance the prologue's float64 outputs)."""
    x = np.asarray(x)
    return bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def kv_head_of(h: int, hq: int, hkv: int) -> int:
    """Reading R6: contiguous groups of G = hq / hkv query heads."""
    return h // (hq // hkv)


def head_is_streaming(full_attention_heads, kvh: int) -> bool:
    """Readings R7/R8: None means every head keeps full context."""
    if full_attention_heads is None:
        return False
    return int(full_attention_heads[kvh]) == 0


def visible_positions(i: int, layer: str, window: int, streaming: bool,
                      sink: int, recent: int) -> np.ndarray:
    """Sorted key positions that query position ``i`` attends.

    * full-context head on a full layer: every position 0..i (model card,
      "Why It Works": full-context heads hold every earlier position; Laguna-M.1
      post, mask generation: create_causal_mask);
    * full-context head on a sliding layer with window W > 0: the W positions
      ending at i (readings R1, R2, R10);
    * streaming head: the first ``sink`` positions that are <= i, together with
      the ``recent`` positions ending at i (model card, "Summary" and "Why It
      Works"; readings R3-R5, R9).
    """
    if streaming:
        sink_part = np.arange(0, min(sink, i + 1), dtype=np.int64)
        recent_part = np.arange(max(0, i - recent + 1), i + 1, dtype=np.int64)
        return np.union1d(sink_part, recent_part)
    if layer == SLIDING_LAYER and window > 0:
        return np.arange(max(0, i - window + 1), i + 1, dtype=np.int64)
    return np.arange(0, i + 1, dtype=np.int64)


def attend(qvec: np.ndarray, kmat: np.ndarray, vmat: np.ndarray, scale: float, sink_logit=None):
    """Softmax attention of one query over the given keys/values (float64).

    logits s_j = scale * <q, k_j>; weights w_j = exp(s_j - max s) / sum;
    output sum_j w_j v_j; lse = max s + ln(sum exp(s_j - max s)).
    Returns (output[D], lse). An empty key set returns zeros and -inf.

    sink_logit (reading R15): the learnable bias of a sliding layer's
    attention sink (Laguna-M.1-8bit blog post, section on the sliding-window
    optimisations) joins the normaliser as one more logit whose value row is
    zero: the denominator gains exp(sink_logit) and lse includes it.
    """
    s = scale * (kmat @ qvec) if kmat.shape[0] else np.zeros(0)
    if sink_logit is None:
        if kmat.shape[0] == 0:
            return np.zeros(qvec.shape[0]), -np.inf
        m = s.max()
        w = np.exp(s - m)
        z = w.sum()
        return (w @ vmat) / z, m + np.log(z)
    b = float(sink_logit)
    m = max(s.max(), b) if len(s) else b
    w = np.exp(s - m)
    z = w.sum() + np.exp(b - m)
    out = (w @ vmat) / z if len(s) else np.zeros(qvec.shape[0])
    return out, m + np.log(z)


def output_gate(out: np.ndarray, gate: np.ndarray) -> np.ndarray:
    """Gated attention output (reading R16): each output channel times the
    logistic function of its gate value, which comes from the layer's gating
    projection (Laguna-M.1-8bit blog post, attention output gating: one gate
    per (head, channel), or one per head broadcast over the head's channels).
    `gate` broadcasts against `out` ([n, D] or [n, 1])."""
    return out / (1.0 + np.exp(-np.asarray(gate, dtype=np.float64)))


def _rows(vis: np.ndarray):
    """Index for the visible rows: a slice when they are consecutive (a view,
    no copy), else the index array itself. Selects the same rows either way."""
    if len(vis) and vis[-1] - vis[0] + 1 == len(vis):
        return slice(int(vis[0]), int(vis[-1]) + 1)
    return vis


def _layer_scale(d: int, scale):
    return 1.0 / np.sqrt(d) if not scale else float(scale)


def prefill_rows(q, k_pos, v_pos, start_pos: int, rows, *, hkv: int, layer: str,
                 window: int = 0, sink: int = 64, recent: int = 256,
                 full_attention_heads=None, scale=None, sink_logits=None):
    """Reference outputs for selected prefill query rows.

    q      : uint16 bf16 bits [B, T, Hq, D] -- queries at positions
             start_pos .. start_pos+T-1 (float arrays: values, see values_f64).
    k_pos, v_pos : uint16 bf16 bits [B, N, Hkv, D] indexed by absolute
             position (N >= start_pos + T); every position a row can see
             must be filled.
    rows   : iterable of (b, h, t) with t the row inside the chunk.
    sink_logits : None or [Hq] attention-sink logits (see ``attend``).
    Returns (out float64 [n, D], lse float64 [n]).
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    hq, d = q.shape[2], q.shape[3]
    sc = _layer_scale(d, scale)
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    cache = {}
    for n, (b, h, t) in enumerate(rows):
        kvh = kv_head_of(int(h), hq, hkv)
        i = start_pos + int(t)
        vis = visible_positions(i, layer, window, head_is_streaming(full_attention_heads, kvh),
                                sink, recent)
        key = (int(b), kvh)
        if key not in cache:
            cache.clear()
            cache[key] = (values_f64(k_pos[b, :, kvh]), values_f64(v_pos[b, :, kvh]))
        kf, vf = cache[key]
        sel = _rows(vis)
        sl = None if sink_logits is None else sink_logits[int(h)]
        out[n], lse[n] = attend(values_f64(q[b, t, h]), kf[sel], vf[sel], sc, sl)
    return out, lse


def decode_rows(q, kv_of, lengths, rows, *, hkv: int, layer: str, window: int = 0,
                sink: int = 64, recent: int = 256, full_attention_heads=None, scale=None,
                sink_logits=None):
    """Reference outputs for decode: one query per sequence at position L_b - 1
    (reading R12).

    q       : uint16 bf16 bits [B, Hq, D].
    kv_of   : callable (b, kvh, positions) -> (k bits [n, D], v bits [n, D])
              giving keys/values by absolute position.
    lengths : int [B], L_b >= 1.
    rows    : iterable of (b, h).
    Returns (out float64 [n, D], lse float64 [n]).
    """
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
    hq, d = q.shape[1], q.shape[2]
    sc = _layer_scale(d, scale)
    out = np.zeros((len(rows), d))
    lse = np.zeros(len(rows))
    cache = {}
    for n, (b, h) in enumerate(rows):
        kvh = kv_head_of(int(h), hq, hkv)
        i = int(lengths[b]) - 1
        vis = visible_positions(i, layer, window, head_is_streaming(full_attention_heads, kvh),
                                sink, recent)
        key = (int(b), kvh)
        if key not in cache:
            cache.clear()
            kb, vb = kv_of(int(b), kvh, vis)
            cache[key] = (values_f64(kb), values_f64(vb))
        kf, vf = cache[key]
        sl = None if sink_logits is None else sink_logits[int(h)]
        out[n], lse[n] = attend(values_f64(q[b, h]), kf, vf, sc, sl)
    return out, lse
