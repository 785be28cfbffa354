"""Error measures for parity checks.  Test infrastructure only.

The rel-L2 measure and the first-mismatch report follow the verification
discipline of "Day 79: Tile programming with cuTile" (compare against a
float64 reference over the identical rounded inputs; report the first failing
index with both values; look at whether errors come in tile-sized bands).
"""
from __future__ import annotations

import numpy as np


def rel_l2(out, ref):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((out - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)


def first_mismatch(out, ref, rtol, atol):
    """Index, got, expected of the first element (C order) with
    |out - ref| > atol + rtol |ref|, or None.  ``atol`` may be an array of
    per-element bounds (broadcast against ``ref``).  An element whose
    difference is NaN (a NaN in either array) counts as a mismatch."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    bad = ~(np.abs(out - ref) <= atol + rtol * np.abs(ref))
    if not bad.any():
        return None
    idx = np.unravel_index(int(np.argmax(bad)), bad.shape)
    return tuple(int(i) for i in idx), float(out[idx]), float(ref[idx])


def count_mismatch(out, ref, rtol, atol):
    """Number of elements that fail the bound of ``first_mismatch``."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    return int(np.count_nonzero(~(np.abs(out - ref) <= atol + rtol * np.abs(ref))))


def band_report(out, ref, tile, axis=1):
    """rel-L2 over the first and the last ``tile`` positions along ``axis``, so
    a tail or tile-band error cannot hide inside a global norm."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    n = out.shape[axis]
    head = [slice(None)] * out.ndim
    tail = [slice(None)] * out.ndim
    head[axis] = slice(0, min(tile, n))
    tail[axis] = slice(max(n - tile, 0), n)
    return (rel_l2(out[tuple(head)], ref[tuple(head)]),
            rel_l2(out[tuple(tail)], ref[tuple(tail)]))


def band_errors(out, ref, tile, axis=1):
    """rel-L2 of every band of ``tile`` consecutive positions along ``axis``
    (the last band may be shorter), in order: a wrong chunk or tile shows up
    as one bad band however small its share of the global norm."""
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    n = out.shape[axis]
    errs = []
    for s in range(0, n, tile):
        sl = [slice(None)] * out.ndim
        sl[axis] = slice(s, min(s + tile, n))
        errs.append(rel_l2(out[tuple(sl)], ref[tuple(sl)]))
    return errs
