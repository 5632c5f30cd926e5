"""Acceptance rule for comparing a kernel's output with the fp64 oracle (test infrastructure only).

fp32 outputs: max abs error <= 1e-4.

bf16 outputs: an element passes when it lies within 1e-2 of the oracle value, or when it is one of the two
bf16 values that bracket the oracle value (for |o| >= 2 the bf16 spacing exceeds 1e-2, so a correctly
rounded output may sit up to half that spacing away, and an output that rounds the other way is the
bracket's other end). The mean abs error over all elements must be <= 2e-3. Nothing here is additive: an
element more than 1e-2 away that is not a bracketing bf16 value fails whatever the rounding of o.
"""
from __future__ import annotations

import numpy as np

FP32_MAX_ABS = 1e-4
BF16_MAX_ABS = 1e-2
BF16_MEAN_ABS = 2e-3


def _bf16_key(bits: np.ndarray) -> np.ndarray:
    """Order-preserving integer for bf16 bit patterns (-0 and +0 both map to 0)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _bf16_from_key(key: np.ndarray) -> np.ndarray:
    k = key.astype(np.int64)
    bits = np.where(k < 0, 0x8000 | (-k), k).astype(np.uint32)
    return (bits << 16).view(np.float32).astype(np.float64)


def bf16_round_down_up(o: np.ndarray):
    """(lo, hi): the largest bf16 value <= o and the smallest bf16 value >= o (equal when o is a bf16 value).
    Finite o within the bf16 range only. Truncating the fp32 rounding of o to its top 16 bits gives a bf16
    value c with no bf16 value strictly between c and o, so lo and hi are among c and its two neighbours."""
    o = np.asarray(o, dtype=np.float64)
    key = _bf16_key((o.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    cands = [_bf16_from_key(key + d) for d in (-1, 0, 1)]
    lo = np.full(o.shape, -np.inf)
    hi = np.full(o.shape, np.inf)
    for c in cands:
        lo = np.where((c <= o) & (c > lo), c, lo)
        hi = np.where((c >= o) & (c < hi), c, hi)
    return lo, hi


def bf16_failures(got: np.ndarray, want: np.ndarray) -> np.ndarray:
    """Boolean mask of the elements that fail the bf16 max rule (got holds bf16 values widened to fp64)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    near = np.abs(got - want) <= BF16_MAX_ABS
    lo, hi = bf16_round_down_up(want)
    return ~(near | (got == lo) | (got == hi))


def check(got: np.ndarray, want: np.ndarray, bf16: bool, what: str = ""):
    """Raises AssertionError unless got meets the rule for its dtype; returns (max abs err, mean abs err)."""
    got = np.asarray(got, dtype=np.float64).reshape(np.shape(want))
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - want)
    if not bf16:
        assert err.max() <= FP32_MAX_ABS, f"{what}: max abs err {err.max():.3e} > {FP32_MAX_ABS}"
    else:
        bad = bf16_failures(got, want)
        if bad.any():
            i = int(np.flatnonzero(bad.reshape(-1))[0])
            raise AssertionError(f"{what}: {int(bad.sum())} elements off by more than {BF16_MAX_ABS} and not a "
                                 f"bf16 neighbour of the oracle value (first: flat index {i}, got "
                                 f"{got.reshape(-1)[i]!r}, oracle {want.reshape(-1)[i]!r}); max abs err "
                                 f"{err.max():.3e}")
        assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs err {err.mean():.3e} > {BF16_MEAN_ABS}"
    return float(err.max()), float(err.mean())
