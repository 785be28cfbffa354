"""Scalar linear recurrence oracle (float64).  Test infrastructure only.

Follows "Selective-scan CUDA kernels", section "The problem": the recurrence
h[t] = a[t] * h[t-1] + b[t] with h[-1] = 0, and the associative (but not
commutative) combine of two affine steps.  Rows are independent.
"""
from __future__ import annotations

import numpy as np


def scan_loop(a, b, h_init=None):
    """h[r, t] = a[r, t] * h[r, t-1] + b[r, t], h[r, -1] = h_init[r] (default 0).

    Inputs are upcast exactly to float64; the loop runs over t and is
    vectorised over rows only.  NaN/Inf propagate with no special handling.
    """
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape or a.ndim != 2:
        raise ValueError("a and b must both be [rows, L]")
    rows, length = a.shape
    h = np.zeros(rows) if h_init is None else np.asarray(h_init, np.float64).copy()
    out = np.empty((rows, length), dtype=np.float64)
    for t in range(length):
        h = a[:, t] * h + b[:, t]
        out[:, t] = h
    return out


def combine(first, second):
    """Compose two affine steps, ``first`` applied before ``second``.

    (a1, b1) then (a2, b2) maps h -> a2 (a1 h + b1) + b2, i.e. the pair
    (a1 a2, a2 b1 + b2).  The order of the operands matters.
    """
    a1, b1 = first
    a2, b2 = second
    return (a1 * a2, a2 * b1 + b2)


def scan_error_scale(a, b):
    """Scale of the rounding error of an evaluation of the scan, per element.

    With h_abs = scan(|a|, |b|) (the sum of the absolute values of the terms
    of h[t]), one rounding of relative size u per combine adds at most about
    u * h_abs[t] at step t, and that error is carried forward by the later a's
    like any other term.  The accumulated error at t is therefore bounded by a
    small multiple of u * scan(|a|, h_abs)[t], which this returns (divided by
    u).  Parity bounds are stated against it.
    """
    aa = np.abs(np.asarray(a, dtype=np.float64))
    h_abs = scan_loop(aa, np.abs(np.asarray(b, dtype=np.float64)))
    return scan_loop(aa, h_abs)
