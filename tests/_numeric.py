"""Small numpy helpers shared by the tests (no method arithmetic here):
bfloat16 bit patterns <-> float64, and an independent round-to-nearest-even
to bfloat16 that compares the neighbouring bfloat16 values explicitly."""
import numpy as np


def bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits).astype(np.int64).astype(np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Nearest bfloat16 to each finite v (ties to the even pattern), found by
    comparing the candidate patterns around v in float64."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    t = (a.astype(np.float32).view(np.uint32) >> 16).astype(np.int64)
    cands = np.clip(np.stack([t - 1, t, t + 1]), 0, 0x7F80)
    err = np.abs(bits_to_f64(cands) - a[None])
    emin = err.min(axis=0)
    is_min = err == emin[None]
    unique = is_min.sum(axis=0) == 1
    choice = np.where(is_min & ((cands % 2 == 0) | unique[None]), cands, -1).max(axis=0)
    sign = np.where(np.signbit(v), 0x8000, 0)
    return (choice | sign).astype(np.uint16)
