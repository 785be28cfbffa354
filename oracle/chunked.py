"""Float64 mirror of the chunked SSD algebra.  Test infrastructure only.

Follows "Accelerating Mamba-2 with high-performance forward pass kernels in
NVIDIA cuTile", section "Mamba-2 architecture" (log-space cumulative sum G,
the decayed state jump, and the decayed chunk output formula) and the three
kernel sections (cumulative sum within each chunk; state at each chunk start;
per-chunk output from that state).

Per (batch, head) and per chunk of T tokens (the last chunk may be shorter):

* G     = inclusive cumulative sum of a_t = A dt_t inside the chunk;
* Y     = exp(G) . (C h_start) + ((exp(G_i - G_j) . (C Bd^T)) . M) X + D X,
          where Bd stacks b_t = dt_t B_t and M keeps i >= j;
* h_end = exp(G_last) h_start + (exp(G_last - G) . Bd)^T X.

A ragged last chunk is read as the recurrence over its real tokens only
(G_last is G at the last real token).  The state is S x P as on the page.
This is a second, independent formulation used to pin the token loop
(chunk-size invariance); it is not the oracle.
"""
from __future__ import annotations

import numpy as np


def ssd_chunked(x, dt, A, B, C, D=None, h0=None, chunk=32, keep_diagonal=True):
    """Chunked SSD forward in float64.  ``keep_diagonal=False`` drops the mask's
    diagonal (a strictly causal mask); it exists only so tests can show that
    reading is distinguishable from the page's mask, and is not the method."""
    x, dt, A, B, C = (np.asarray(v, np.float64) for v in (x, dt, A, B, C))
    D = None if D is None else np.asarray(D, np.float64)
    h0 = None if h0 is None else np.asarray(h0, np.float64)
    Bt, L, H, P = x.shape
    G, S = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.empty((Bt, L, H, P))
    hfin = np.empty((Bt, H, P, S))
    for bb in range(Bt):
        for hh in range(H):
            g = hh // hpg
            state = np.zeros((S, P)) if h0 is None else h0[bb, hh].T.copy()
            for c0 in range(0, L, chunk):
                c1 = min(c0 + chunk, L)
                a = A[hh] * dt[bb, c0:c1, hh]
                Gc = np.cumsum(a)
                X = x[bb, c0:c1, hh, :]
                Cm = C[bb, c0:c1, g, :]
                Bd = dt[bb, c0:c1, hh, None] * B[bb, c0:c1, g, :]
                n = c1 - c0
                mask = np.tril(np.ones((n, n), dtype=bool), k=0 if keep_diagonal else -1)
                # only the kept (i >= j) exponents are formed, so none is positive
                seg = np.where(mask, Gc[:, None] - Gc[None, :], -np.inf)
                Y = np.exp(Gc)[:, None] * (Cm @ state)
                Y += (np.exp(seg) * (Cm @ Bd.T)) @ X
                if D is not None:
                    Y += D[hh] * X
                y[bb, c0:c1, hh, :] = Y
                state = np.exp(Gc[-1]) * state + (np.exp(Gc[-1] - Gc)[:, None] * Bd).T @ X
            hfin[bb, hh] = state.T
    return y, hfin
