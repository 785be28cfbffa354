"""Parity checks of the HIP path against the float64 oracle (test helpers).

Every check compares whole outputs: the global rel-L2 against the tolerance
the method is held to (1e-5 for fp32 inputs, 2e-2 for bf16 inputs with fp32
state), the rel-L2 of every chunk-long band along the sequence, and an
element-wise bound

    |got - ref| <= c_abs * u * scale + c_rel * u * |ref|

where u is the unit roundoff of the operand type and ``scale`` is the sum of
the absolute values of the terms that form the element (``oracle.ssd.
ssd_abs_terms`` for the SSD, ``oracle.scan.scan_error_scale`` for the scan).
The constants are derived from the roundings each path performs:

* bf16 SSD, y: every term of an output passes through at most three bf16
  roundings of its factors (the decayed X~ or the decayed C B^T weights, C B^T
  itself, the bf16 copy of the state for C h^T), each of relative size u, and
  y is rounded to bf16 once at the end (u |y|).  3u, doubled for fp32
  accumulation and the hardware exp2: c_abs = 8, c_rel = 2 (u = 2^-9).
* bf16 SSD, final state: one rounding per term (X~), fp32 from there on:
  c_abs = 4, c_rel = 0 (u = 2^-9).
* fp32 SSD: fp32 products and sums over at most a chunk of tokens and the
  state: c_abs = 1024, c_rel = 4 (u = 2^-24).
* scan: one fp32 rounding per combine, carried forward by the later a's
  (``scan_error_scale`` accounts for that, assuming every rounding adds with
  the same sign), plus the ~25 levels of combines of the parallel evaluation
  (items, wave, workgroup, look-back), each rounding at most u times the
  absolute terms of its partial sum, which the scale exceeds once the decays
  carry more than a few steps: c_abs = 16 (u = 2^-24); a bf16 h adds its one
  rounding: c_rel = 2 (u = 2^-9).

Full-size workloads are checked in a process pool: each worker regenerates
the seeded inputs itself (``chunked_linear_scan_amd.workloads`` holds only
the random draws) and compares one (batch, head-block) slice, so only the GPU
outputs travel to the workers.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import compare, scan as oscan, ssd as ossd

U_BF16 = 2.0 ** -9
U_F32 = 2.0 ** -24
TOL_F32 = 1e-5
TOL_BF16 = 2e-2

# (c_abs, u_abs, c_rel, u_rel) for y and for the final state
SSD_BOUNDS = {
    "bf16": {"y": (8.0, U_BF16, 2.0, U_BF16), "h": (4.0, U_BF16, 0.0, U_BF16)},
    "f32": {"y": (1024.0, U_F32, 4.0, U_F32), "h": (1024.0, U_F32, 4.0, U_F32)},
}


def _np64(t):
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        return t.to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _stats(got, ref, scale, bound, band):
    """Sums for the rel-L2, the element-wise bound check and the band check."""
    c_abs, u_abs, c_rel, u_rel = bound
    atol = c_abs * u_abs * scale
    rtol = c_rel * u_rel
    out = {"d2": float(np.sum((got - ref) ** 2)), "r2": float(np.sum(ref ** 2)),
           "bad": compare.count_mismatch(got, ref, rtol, atol), "first": None,
           "finite": bool(np.isfinite(got).all()), "band": 0.0}
    if out["bad"]:
        idx, g, r = compare.first_mismatch(got, ref, rtol, atol)
        out["first"] = (idx, g, r, float(atol[idx]) + rtol * abs(r))
    if band:
        # got / ref are [Bt, L, H, P] or [L, P]-like with the sequence on axis 1
        out["band"] = max(compare.band_errors(got, ref, band, axis=1))
    return out


def ssd_slice_stats(x, dt, A, B, C, D, h0, y_got, h_got, dtype, band):
    """Oracle and comparison for one set of (batch, head) sequences."""
    y, h = ossd.ssd_loop(x, dt, A, B, C, D, h0)
    ya, ha = ossd.ssd_abs_terms(x, dt, A, B, C, D, h0)
    sy = _stats(np.asarray(y_got, np.float64), y, ya, SSD_BOUNDS[dtype]["y"], band)
    sh = None
    if h_got is not None:
        sh = _stats(np.asarray(h_got, np.float64), h, ha, SSD_BOUNDS[dtype]["h"], 0)
    return sy, sh


def _merge(parts):
    out = {"d2": 0.0, "r2": 0.0, "bad": 0, "first": None, "finite": True, "band": 0.0}
    for p in parts:
        out["d2"] += p["d2"]
        out["r2"] += p["r2"]
        out["bad"] += p["bad"]
        out["finite"] = out["finite"] and p["finite"]
        out["band"] = max(out["band"], p["band"])
        if out["first"] is None and p["first"] is not None:
            out["first"] = p["first"]
    out["rel_l2"] = math.sqrt(out["d2"] / out["r2"]) if out["r2"] > 0 else math.sqrt(out["d2"])
    return out


def _assert(st, tol, label, band):
    print(f"  {label}: rel-L2 {st['rel_l2']:.3e}, worst band {st['band']:.3e}, "
          f"elements over the bound {st['bad']}", flush=True)
    assert st["finite"], (label, "non-finite output")
    assert st["rel_l2"] <= tol, (label, st["rel_l2"], st["first"])
    if band:
        assert st["band"] <= tol, (label, "band", st["band"])
    assert st["bad"] == 0, (label, "element-wise bound", st["bad"], "first (index, got, ref, bound):",
                            st["first"])


def check_with_scale(got, ref, scale, bound, tol, label, band=0):
    """rel-L2 <= tol, bands (along axis 1) <= tol and the element-wise bound
    ``bound`` = (c_abs, u_abs, c_rel, u_rel) against ``scale``."""
    _assert(_merge([_stats(np.asarray(got, np.float64), ref, scale, bound, band)]), tol, label, band)


def _dtype_name(x):
    return "bf16" if x.dtype == torch.bfloat16 else "f32"


def check_ssd(inp, y_got, h_got, chunk, label=""):
    """Whole-output parity of one ssd_fwd result for a small problem (oracle
    in this process).  inp: host tensors x, dt, A, B, C, D, h0."""
    dtype = _dtype_name(inp["x"])
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    sy, sh = ssd_slice_stats(*(_np64(inp.get(k)) for k in ("x", "dt", "A", "B", "C", "D", "h0")),
                             y_got, h_got, dtype, chunk)
    _assert(_merge([sy]), tol, f"{label} y", chunk)
    if sh is not None:
        _assert(_merge([sh]), tol, f"{label} h_final", 0)


# ---------------------------------------------------------------------------
# full-size workloads: a process pool over (batch, head-block) slices
# ---------------------------------------------------------------------------
_CACHE = {}


def _workload_inputs(name):
    if name not in _CACHE:
        from chunked_linear_scan_amd import workloads
        _CACHE.clear()
        _CACHE[name] = workloads.ssd_workload(name)
    return _CACHE[name]


def _ssd_pool_job(job):
    name, b, h0_, h1_, y_got, h_got, band = job
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    inp = _workload_inputs(name)
    H, G = inp["x"].shape[2], inp["B"].shape[2]
    g = h0_ // (H // G)
    sl = lambda t: None if t is None else t.to(torch.float64).numpy()
    x = sl(inp["x"][b:b + 1, :, h0_:h1_])
    dt = sl(inp["dt"][b:b + 1, :, h0_:h1_])
    B = sl(inp["B"][b:b + 1, :, g:g + 1])
    C = sl(inp["C"][b:b + 1, :, g:g + 1])
    A = sl(inp["A"][h0_:h1_])
    D = sl(inp["D"][h0_:h1_])
    h0 = None if inp["h0"] is None else sl(inp["h0"][b:b + 1, h0_:h1_])
    dtype = "bf16" if inp["x"].dtype == torch.bfloat16 else "f32"
    sy, sh = ssd_slice_stats(x, dt, A, B, C, D, h0, y_got, h_got, dtype, band)
    # report mismatches at their index in the whole output
    if sy["first"] is not None:
        (bb, t, hh, pp), g, r, bd = sy["first"]
        sy["first"] = ((bb + b, t, hh + h0_, pp), g, r, bd)
    if sh is not None and sh["first"] is not None:
        (bb, hh, pp, ss), g, r, bd = sh["first"]
        sh["first"] = ((bb + b, hh + h0_, pp, ss), g, r, bd)
    return sy, sh


def pool_size():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(16, n))


def check_ssd_workload(name, y_got, h_got, label=""):
    """Whole-output parity of ssd_fwd on a named full-size workload.  y_got
    [Bt,L,H,P] and h_got [Bt,H,P,S] as float32 numpy arrays."""
    import multiprocessing as mp
    from chunked_linear_scan_amd import workloads
    shape, _ = workloads.SSD_WORKLOADS[name]
    Bt, H, G = shape.batch, shape.nheads, shape.ngroups
    hpg = H // G
    procs = pool_size()
    # head blocks inside one group, about two jobs per process
    per = max(1, min(hpg, (Bt * H) // (2 * procs)))
    while hpg % per:
        per -= 1
    jobs = []
    for b in range(Bt):
        for h in range(0, H, per):
            jobs.append((name, b, h, h + per, y_got[b:b + 1, :, h:h + per], h_got[b:b + 1, h:h + per],
                         shape.chunk))
    print(f"  oracle over {len(jobs)} slices of {per} head(s) on {procs} processes", flush=True)
    with mp.get_context("spawn").Pool(procs) as pool:
        res = pool.map(_ssd_pool_job, jobs, chunksize=1)
    tol = TOL_BF16 if shape.dtype == "bf16" else TOL_F32
    _assert(_merge([r[0] for r in res]), tol, f"{label or name} y", shape.chunk)
    _assert(_merge([r[1] for r in res]), tol, f"{label or name} h_final", 0)


# ---------------------------------------------------------------------------
# scalar scan
# ---------------------------------------------------------------------------
U_F16 = 2.0 ** -11


def check_scan(a, b, h_got, out_bf16=False, label="", row_tol_factor=10.0, elementwise=True, band=8192,
               out_f16=False):
    """Whole-output parity of a scan result: rel-L2 <= 1e-5 (bf16 h: 1e-2,
    fp16 h: 1e-3),
    every row's rel-L2 within ``row_tol_factor`` of that, the rel-L2 of every
    ``band``-long stretch of the rows (a tile of the kernels) within the same
    factor, and the element-wise bound against ``scan_error_scale``.
    ``elementwise=False`` leaves out the element-wise bound (only for rows of
    millions of elements, where its two extra float64 loops take minutes)."""
    a64, b64 = _np64(a), _np64(b)
    ref = oscan.scan_loop(a64, b64)
    scale = oscan.scan_error_scale(a64, b64) if elementwise else np.full(ref.shape, np.inf)
    got = np.asarray(h_got, np.float64)
    tol = 1e-2 if out_bf16 else (1e-3 if out_f16 else TOL_F32)
    bound = (16.0, U_F32, 2.0 if (out_bf16 or out_f16) else 4.0,
             U_BF16 if out_bf16 else (U_F16 if out_f16 else U_F32))
    st = _merge([_stats(got, ref, scale, bound, 0)])
    _assert(st, tol, f"{label} h", 0)
    if band and got.shape[1] > band:
        worst = max(compare.band_errors(got, ref, band, axis=1))
        assert worst <= row_tol_factor * tol, (label, "band", worst)
    rows = [compare.rel_l2(got[r], ref[r]) for r in range(got.shape[0])]
    assert max(rows) <= row_tol_factor * tol, (label, "row", int(np.argmax(rows)), max(rows))
    return got, ref


# ---------------------------------------------------------------------------
# one decode token
# ---------------------------------------------------------------------------
def check_step(c, y_got, h_got, label=""):
    """Parity of one ssd_step: the new state (fp32: rel-L2 <= 1e-5) and y
    (1e-5 for fp32 inputs, 1e-2 for bf16 inputs, where y is rounded to bf16
    once), each with an element-wise bound against the absolute terms (the
    step with |h|, |x|, |B|, |C|, |D|)."""
    args = [_np64(c[k]) for k in ("h", "x", "dt", "A", "B", "C", "D")]
    ry, rh = ossd.ssd_step(*args)
    absargs = [None if v is None else np.abs(v) for v in args]
    absargs[2], absargs[3] = args[2], args[3]
    ya, ha = ossd.ssd_step(*absargs)
    bf16 = c["x"].dtype == torch.bfloat16
    hb = (64.0, U_F32, 4.0, U_F32)
    yb = (64.0, U_F32, 2.0, U_BF16) if bf16 else (64.0, U_F32, 4.0, U_F32)
    _assert(_merge([_stats(np.asarray(h_got, np.float64), rh, ha, hb, 0)]), TOL_F32, f"{label} state", 0)
    _assert(_merge([_stats(np.asarray(y_got, np.float64), ry, ya, yb, 0)]), 1e-2 if bf16 else TOL_F32,
            f"{label} y", 0)
