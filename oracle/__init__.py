"""Plain float64 CPU oracle for hybrid GQA / sliding-window / DuoAttention
attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may use it. It shares no code with the HIP path.

Every function states the passage of the pages it follows:

* Hugging Face model card "DuoAttention Laguna Adapter" (sections "Summary",
  "Why It Works", "Changes In This Submission") -- full-context KV heads keep
  every earlier token; streaming KV heads hold only the first positions of the
  sequence and a window of the newest ones (sink 64, recent 256); head
  routing is per KV head.
* Blog post on Laguna-M.1-8bit attention, sections on how the sliding window
  works, its implementation (per-layer ``layer_types`` / ``sliding_window``)
  and mask generation (``create_causal_mask`` /
  ``create_sliding_window_causal_mask``) -- each token looks back over a
  window of fixed width; full layers are causal.
* SGLang cookbook "Laguna-XS-2.1", section 1 "Model Introduction" -- 48 Q /
  8 KV heads, window 512.

Readings where the pages are silent are listed in ``oracle.attention`` and
``oracle.prologue`` (RMSNorm and rotary embedding of q and k).
"""
from .attention import (  # noqa: F401
    FULL_LAYER, SLIDING_LAYER, bf16_bits_to_f64, kv_head_of, head_is_streaming,
    visible_positions, attend, output_gate, prefill_rows, decode_rows,
)
from .cache_model import ShadowCache  # noqa: F401
from .prologue import (  # noqa: F401
    rms_norm, yarn_correction_index, rope_frequencies, rope_rotate, qk_prologue, round_bf16,
)
