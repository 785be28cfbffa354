"""Mamba-2 SSD forward oracle (float64).  Test infrastructure only.

Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
NVIDIA cuTile", section "Mamba-2 architecture":

* the recurrence  h_t = exp(A dt_t) h_{t-1} + dt_t B_t x_t^T  (outer product),
  with a_t = A dt_t and b_t = dt_t B_t, the state h_t an S x P matrix;
* the output  y_t = c_t^T h_t + D x_t.  The page's renamed form writes h_{t-1}
  in the output, while its chunked output formula (causal mask that keeps the
  diagonal) and the compute_out kernel's mask (row index >= column index) use
  h_t; this oracle takes h_t (the token's own update is seen by its output).

Shapes (row-major, as the page's kernels lay them out): x [Bt,L,H,P],
dt [Bt,L,H], A [H], B and C [Bt,L,G,S], D [H], initial/final state
[Bt,H,P,S] (head-dim rows, state columns, i.e. h_t transposed).  Head h reads
B/C group h // (H/G) (the fwd_pass_state kernel's head-to-group map).
"""
from __future__ import annotations

import numpy as np


def _f64(v):
    return None if v is None else np.asarray(v, dtype=np.float64)


def _check(x, dt, A, B, C):
    Bt, L, H, P = x.shape
    if dt.shape != (Bt, L, H) or A.shape != (H,):
        raise ValueError("dt must be [Bt,L,H] and A [H]")
    if B.ndim != 4 or B.shape[:2] != (Bt, L) or C.shape != B.shape:
        raise ValueError("B and C must be [Bt,L,G,S]")
    G = B.shape[2]
    if H % G:
        raise ValueError("heads must be a multiple of groups")
    return Bt, L, H, P, G, B.shape[3]


def ssd_loop(x, dt, A, B, C, D=None, h0=None, y_uses_previous_state=False):
    """Token-by-token SSD recurrence.  Returns (y [Bt,L,H,P], h_final [Bt,H,P,S]).

    The state is kept as the page writes it, S x P per (batch, head); the loop
    runs over tokens and is vectorised over batch and heads.

    ``y_uses_previous_state=True`` evaluates y_t = c_t^T h_{t-1} + D x_t
    instead, the page's renamed form read literally; it exists only so tests
    can show that reading is distinguishable (it is not the oracle).
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, h0))
    Bt, L, H, P, G, S = _check(x, dt, A, B, C)
    grp = np.arange(H) // (H // G)
    h = np.zeros((Bt, H, S, P)) if h0 is None else np.swapaxes(h0, 2, 3).copy()
    Dv = np.zeros(H) if D is None else D
    y = np.empty((Bt, L, H, P))
    for t in range(L):
        decay = np.exp(A[None, :] * dt[:, t, :])                 # exp(a_t)  [Bt,H]
        b_t = dt[:, t, :, None] * B[:, t, grp, :]                # b_t = dt_t B_t  [Bt,H,S]
        c_t = C[:, t, grp, :]                                    # [Bt,H,S]
        h_prev = h
        h = decay[:, :, None, None] * h + b_t[:, :, :, None] * x[:, t, :, None, :]
        h_out = h_prev if y_uses_previous_state else h
        y[:, t] = np.matmul(c_t[:, :, None, :], h_out)[:, :, 0, :] + Dv[None, :, None] * x[:, t]
    return y, np.swapaxes(h, 2, 3).copy()


def ssd_bruteforce(x, dt, A, B, C, D=None, h0=None):
    """Unrolled recurrence evaluated as a direct sum (tiny inputs only).

    h_t = exp(sum_{k<=t} a_k) h0 + sum_{j<=t} exp(sum_{j<k<=t} a_k) b_j x_j^T,
    then y_t = c_t^T h_t + D x_t.  O(L^2) work per (batch, head); it builds
    every h_t explicitly, which is what the chunked method avoids.
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, h0))
    Bt, L, H, P, G, S = _check(x, dt, A, B, C)
    hpg = H // G
    y = np.empty((Bt, L, H, P))
    hfin = np.empty((Bt, H, P, S))
    for bb in range(Bt):
        for hh in range(H):
            g = hh // hpg
            a = A[hh] * dt[bb, :, hh]
            for t in range(L):
                state = np.zeros((S, P))
                if h0 is not None:
                    state += np.exp(a[: t + 1].sum()) * h0[bb, hh].T
                for j in range(t + 1):
                    w = np.exp(a[j + 1: t + 1].sum())
                    state += w * dt[bb, j, hh] * np.outer(B[bb, j, g], x[bb, j, hh])
                dterm = 0.0 if D is None else D[hh]
                y[bb, t, hh] = C[bb, t, g] @ state + dterm * x[bb, t, hh]
                if t == L - 1:
                    hfin[bb, hh] = state.T
    return y, hfin


def ssd_linear_attention(x, dt, B, C, D=None, h0=None):
    """The decay-free case (all a_t = 0) in the page's linear-attention form.

    Y = C h0 + ((C Bd^T) . M) X + D X per (batch, head), with Bd the stacked
    rows b_t = dt_t B_t and M the causal mask that keeps the diagonal.  This is
    the closed form the page derives before adding the decay back.
    """
    x, dt, B, C, D, h0 = map(_f64, (x, dt, B, C, D, h0))
    Bt, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    hpg = H // G
    M = np.tril(np.ones((L, L)))
    y = np.empty((Bt, L, H, P))
    for bb in range(Bt):
        for hh in range(H):
            g = hh // hpg
            Cm, X = C[bb, :, g, :], x[bb, :, hh, :]
            Bd = dt[bb, :, hh, None] * B[bb, :, g, :]
            Y = ((Cm @ Bd.T) * M) @ X
            if h0 is not None:
                Y += Cm @ h0[bb, hh].T
            if D is not None:
                Y += D[hh] * X
            y[bb, :, hh, :] = Y
    return y


def ssd_step(h, x, dt, A, B, C, D=None):
    """One token of the recurrence, for sequential inference (decode).

    The page ("Mamba-2 architecture") calls the recurrent form ideal for
    sequential inference: with a = A dt and b = dt B_t, the state becomes
    exp(a) h + b x^T and the output is c^T of the new state plus D x (the
    same reading as ``ssd_loop``: the token's own update is seen by its
    output).

    h [Bt,H,P,S] (head-dim rows, state columns, as ``ssd_loop`` returns it),
    x [Bt,H,P], dt [Bt,H], A [H], B and C [Bt,G,S], D [H] or None.  Returns
    (y [Bt,H,P], the new state [Bt,H,P,S]); the inputs are not modified.
    """
    h, x, dt, A, B, C, D = map(_f64, (h, x, dt, A, B, C, D))
    Bt, H, P = x.shape
    if h.shape[:3] != (Bt, H, P) or dt.shape != (Bt, H) or A.shape != (H,):
        raise ValueError("h must be [Bt,H,P,S], dt [Bt,H] and A [H]")
    if B.ndim != 3 or B.shape[0] != Bt or C.shape != B.shape or B.shape[2] != h.shape[3]:
        raise ValueError("B and C must be [Bt,G,S]")
    G = B.shape[1]
    if H % G:
        raise ValueError("heads must be a multiple of groups")
    grp = np.arange(H) // (H // G)
    decay = np.exp(A[None, :] * dt)                        # exp(a)            [Bt,H]
    b = dt[:, :, None] * B[:, grp, :]                      # b = dt B          [Bt,H,S]
    c = C[:, grp, :]                                       #                   [Bt,H,S]
    h_new = decay[:, :, None, None] * h + x[:, :, :, None] * b[:, :, None, :]
    y = np.einsum("bhps,bhs->bhp", h_new, c)
    if D is not None:
        y = y + D[None, :, None] * x
    return y, h_new


def ssd_abs_terms(x, dt, A, B, C, D=None, h0=None):
    """Sum of the absolute values of the terms that form each output.

    Every y_t and h_t of ``ssd_loop`` is a sum of products of inputs with
    positive decay weights exp(sum a_k) (dt >= 0): h_t = sum_j w_tj dt_j B_j
    x_j^T + w_t0 h0 and y_t = c_t^T h_t + D x_t.  Replacing x, B, C, D and h0
    by their absolute values turns every term into its absolute value, so the
    same loop returns (y_abs, h_abs) with y_abs = sum |term| >= |y|.  A
    rounding error of relative size u in each term's factors is therefore
    bounded, element by element, by a small multiple of u * y_abs: this is
    the scale the element-wise parity bounds are stated against.  Requires
    dt >= 0.
    """
    dt = _f64(dt)
    if np.any(dt < 0):
        raise ValueError("ssd_abs_terms needs dt >= 0 (positive decay weights)")
    ab = lambda v: None if v is None else np.abs(_f64(v))
    return ssd_loop(ab(x), dt, A, ab(B), ab(C), ab(D), ab(h0))
