"""Float64 reference for the input side of attention: RMSNorm of q and k, then
the rotary position embedding (RoPE) with YaRN frequency scaling.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain definitions on the
exact bf16 values the GPU receives; no tables shared with the HIP path.

Passages followed:
* Laguna-XS-2.1 blog post, section on the sliding-window optimisations: q and
  k are RMS-normalised before the rotary embedding is applied.
* Laguna-M.1-8bit blog post, section on YaRN dynamic RoPE: the configuration
  of full-attention layers is rope_theta 500000, rope_type yarn, factor 64,
  original_max_position_embeddings 4096, beta_slow 1, beta_fast 64,
  attention_factor 1, partial_rotary_factor 1 (all 128 channels rotate).
* YaRN ("YaRN: Efficient Context Window Extension of Large Language Models",
  Peng et al., 2023), section 3.2, "NTK-by-parts" interpolation: frequencies
  that turn many times within the original context are kept, those that turn
  less than once are divided by the scale factor, and a linear ramp blends
  the two in between.

Readings (the pages are silent on these):
R18 RMSNorm acts on each head's 128 channels separately, with one learnable
    weight vector of 128 values per tensor (q or k) shared by all heads:
    y = x / sqrt(mean(x^2) + eps) * w.
R19 The rotation pairs channel i with channel i + 64 (the "rotate half"
    layout) and turns the pair (x_i, x_{i+64}) by the angle pos * f_i in the
    positive sense: (x_i cos - x_{i+64} sin, x_{i+64} cos + x_i sin), both
    times attention_factor.
R20 YaRN's ramp runs over the pair index i between the correction indices
    low = floor(c(beta_fast)) and high = ceil(c(beta_slow)), clipped to
    [0, 127], where c(r) is the (fractional) pair index whose frequency turns
    r times over original_max_position_embeddings positions. This is the form
    the configuration's "rope_type: yarn" names in the model's code base; the
    paper states the same ramp in terms of the turn count instead.
R21 The pages print RoPE parameters only for full-attention layers; a
    sliding layer's rotary settings are the caller's (factor <= 1 means plain
    RoPE with the given theta).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import bf16_bits_to_f64

D = 128
HALF = D // 2


def rms_norm(x, weight, eps: float) -> np.ndarray:
    """Reading R18: RMSNorm over the last axis (one head's channels)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def yarn_correction_index(turns: float, theta: float, original_max_pos: int, dim: int = D) -> float:
    """Fractional pair index whose base frequency theta^(-2i/dim) makes
    ``turns`` full turns over ``original_max_pos`` positions (solving
    original_max_pos * theta^(-2i/dim) = 2 pi turns for i)."""
    return dim * math.log(original_max_pos / (2.0 * math.pi * turns)) / (2.0 * math.log(theta))


def rope_frequencies(theta: float, factor: float = 1.0, original_max_pos: int = 4096,
                     beta_fast: float = 64.0, beta_slow: float = 1.0, dim: int = D) -> np.ndarray:
    """Angular frequency f_i (radians per position) of each rotary pair.

    Plain RoPE: f_i = theta^(-2i/dim). With YaRN (factor > 1; section 3.2 of
    the paper, reading R20) each f_i is a blend of itself (weight 1 - r_i) and
    f_i / factor (weight r_i), with r_i the clipped linear ramp over the pair
    index between the two correction indices."""
    i = np.arange(dim // 2, dtype=np.float64)
    base = theta ** (-2.0 * i / dim)
    if factor <= 1.0:
        return base
    low = max(math.floor(yarn_correction_index(beta_fast, theta, original_max_pos, dim)), 0)
    high = min(math.ceil(yarn_correction_index(beta_slow, theta, original_max_pos, dim)), dim - 1)
    if high == low:
        high += 0.001
    ramp = np.clip((i - low) / (high - low), 0.0, 1.0)
    return base / factor * ramp + base * (1.0 - ramp)


def rope_rotate(x, positions, freqs, attention_factor: float = 1.0) -> np.ndarray:
    """Reading R19: rotate the pairs (i, i + 64) of x[n, ..., D], row n at
    positions[n], by the angle positions[n] * freqs[i]."""
    x = np.asarray(x, dtype=np.float64)
    ang = np.outer(np.asarray(positions, dtype=np.float64), np.asarray(freqs, dtype=np.float64))
    ang = ang.reshape((len(ang),) + (1,) * (x.ndim - 2) + (HALF,))
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :HALF], x[..., HALF:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1) * attention_factor


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (8 significant bits, ties to even),
    returned as float64. The attention consumes bf16 q and k (bf16 matrix
    products with float32 accumulation), so a prologue's float64 output is
    rounded once before the attention uses it."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(np.ldexp(m, 8)), e - 8)


def qk_prologue(x_bits, positions, weight=None, eps: float = 1e-6, rope=None) -> np.ndarray:
    """The prologue on one tensor: x_bits uint16 bf16 bits [n, heads, D] (or
    [n, D]) at positions[n]; RMSNorm when ``weight`` is given, then RoPE when
    ``rope`` (a dict of rope_frequencies' arguments plus optional
    attention_factor) is given. Returns float64, unrounded."""
    x = bf16_bits_to_f64(x_bits) if np.asarray(x_bits).dtype == np.uint16 else np.asarray(x_bits, np.float64)
    if weight is not None:
        x = rms_norm(x, weight, eps)
    if rope is not None:
        kw = dict(rope)
        af = kw.pop("attention_factor", 1.0)
        x = rope_rotate(x, positions, rope_frequencies(**kw), af)
    return x
