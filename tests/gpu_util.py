"""Helpers for the GPU parity tests: host bf16 bits <-> device tensors, and the
tolerance check (max-abs 2e-2, mean-abs 2e-3 against the float64 oracle)."""
import sys

import numpy as np

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_bits(t) -> np.ndarray:
    return t.detach().cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def check_close(got: np.ndarray, ref: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS, rel=0.0):
    """Elementwise |got - ref| <= max_abs + rel |ref|, and the mean error
    <= mean_abs."""
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    print(f"[parity] {what}: n={err.shape[0]} max_abs={mx:.3e} mean_abs={mn:.3e}", file=sys.stderr, flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    over = err - (max_abs + rel * np.abs(ref))
    worst = np.unravel_index(int(np.argmax(over)), over.shape)
    assert over[worst] <= 0, (f"{what}: error {err[worst]:.3e} at {worst} (reference {ref[worst]:.4f}) "
                              f"> {max_abs} + {rel} |reference|")
    assert mn <= mean_abs, f"{what}: mean abs error {mn:.3e} > {mean_abs}"
    return mx, mn


def announce(msg: str):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)
