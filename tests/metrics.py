"""Comparison metrics used by the parity tests (no layer arithmetic here)."""
import numpy as np


def max_row_rel_err(got, ref):
    """max over rows of max_c |got - ref| / max_c |ref|.

    A row whose reference is all zero must be exactly zero in ``got`` (its
    error is reported as +inf otherwise)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} != {ref.shape}")
    if got.size == 0:
        return 0.0
    got2 = got.reshape(got.shape[0], -1) if got.ndim > 1 else got.reshape(1, -1)
    ref2 = ref.reshape(ref.shape[0], -1) if ref.ndim > 1 else ref.reshape(1, -1)
    if not np.isfinite(got2).all():
        return float("inf")
    num = np.abs(got2 - ref2).max(axis=1)
    den = np.abs(ref2).max(axis=1)
    zero = den == 0
    if np.any(num[zero] != 0):
        return float("inf")
    den = np.where(zero, 1.0, den)
    return float((num / den).max())


def whole_rel_err(got, ref):
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    num = np.abs(got - ref).max()
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)
