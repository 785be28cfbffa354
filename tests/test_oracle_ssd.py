"""Pins for the float64 SSD oracle (CPU only).

Each test ties ``oracle.ssd.ssd_loop`` to something other than itself: a
hand-worked fixture, the brute-force unrolled sum, the decay-free
linear-attention closed form, the dt = 0 identity, chunk-size invariance of the
independent chunked formulation, state carry across calls, the scalar-scan
special case, and mutants (h_{t-1} output, strict mask, swapped groups) that
must be caught.  ``oracle.ssd.ssd_step`` (one decode token) is tied to numbers
worked by hand, to the dt = 0 and full-decay identities, and, rolled over a
sequence, to the independent chunked formulation.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import chunked, scan, ssd


def rand_case(seed, Bt=2, L=23, H=4, P=3, S=5, G=2, h0=True, D=True, dt_shift=-2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((Bt, L, H, P))
    B = rng.standard_normal((Bt, L, G, S))
    C = rng.standard_normal((Bt, L, G, S))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, L, H)) + dt_shift))
    A = -np.exp(rng.uniform(0.0, math.log(16.0), H))
    Dv = rng.standard_normal(H) if D else None
    hv = 0.3 * rng.standard_normal((Bt, H, P, S)) if h0 else None
    return x, dt, A, B, C, Dv, hv


def load_hand(golden_dir):
    with open(os.path.join(golden_dir, "ssd_hand_L2.json")) as f:
        g = json.load(f)
    A = np.array([-math.log(2.0)])
    arr = {k: np.array(g[k], dtype=np.float64) for k in ("dt", "x", "B", "C", "D", "h0_PxS")}
    return g, arr["x"], arr["dt"], A, arr["B"], arr["C"], arr["D"], arr["h0_PxS"]


def test_hand_worked_fixture(golden_dir):
    g, x, dt, A, B, C, D, h0 = load_hand(golden_dir)
    y, hf = ssd.ssd_loop(x, dt, A, B, C, D, h0)
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(hf, np.array(g["h_final_PxS"]), rtol=0, atol=1e-12)


def test_previous_state_output_mutant_is_caught(golden_dir):
    g, x, dt, A, B, C, D, h0 = load_hand(golden_dir)
    y_prev, _ = ssd.ssd_loop(x, dt, A, B, C, D, h0, y_uses_previous_state=True)
    np.testing.assert_allclose(y_prev, np.array(g["y_if_output_used_previous_state"]), atol=1e-12)
    assert np.abs(y_prev - np.array(g["y"])).max() > 0.5


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_unrolled_sum(seed):
    case = rand_case(seed, Bt=1, L=17, H=2, P=3, S=4, G=1 + seed % 2)
    y, hf = ssd.ssd_loop(*case)
    yb, hb = ssd.ssd_bruteforce(*case)
    assert np.abs(y - yb).max() < 1e-12 * max(1.0, np.abs(yb).max())
    assert np.abs(hf - hb).max() < 1e-12 * max(1.0, np.abs(hb).max())


@pytest.mark.parametrize("seed", range(3))
def test_decay_free_is_linear_attention(seed):
    x, dt, A, B, C, D, h0 = rand_case(seed, L=19)
    y, _ = ssd.ssd_loop(x, dt, np.zeros_like(A), B, C, D, h0)
    yl = ssd.ssd_linear_attention(x, dt, B, C, D, h0)
    assert np.abs(y - yl).max() < 1e-11


def test_zero_timestep_keeps_state():
    x, dt, A, B, C, D, h0 = rand_case(5)
    dt0 = np.zeros_like(dt)
    y, hf = ssd.ssd_loop(x, dt0, A, B, C, D, h0)
    np.testing.assert_allclose(hf, h0, rtol=0, atol=0)
    H = x.shape[2]
    grp = np.arange(H) // (H // B.shape[2])
    expect = np.einsum("blhs,bhps->blhp", C[:, :, grp, :], h0) + D[None, None, :, None] * x
    assert np.abs(y - expect).max() < 1e-12


def test_single_token_by_hand_formula():
    x, dt, A, B, C, D, h0 = rand_case(6, Bt=1, L=1, H=1, G=1)
    y, hf = ssd.ssd_loop(x, dt, A, B, C, D, h0)
    a0 = A[0] * dt[0, 0, 0]
    h_S_by_P = math.exp(a0) * h0[0, 0].T + dt[0, 0, 0] * np.outer(B[0, 0, 0], x[0, 0, 0])
    expect = C[0, 0, 0] @ h_S_by_P + D[0] * x[0, 0, 0]
    assert np.abs(y[0, 0, 0] - expect).max() < 1e-13
    assert np.abs(hf[0, 0] - h_S_by_P.T).max() < 1e-13


@pytest.mark.parametrize("chunk", [1, 2, 4, 7, 8, 16, 23, 64])
def test_chunked_formulation_matches_loop(chunk):
    case = rand_case(7, L=23)
    y, hf = ssd.ssd_loop(*case)
    yc, hc = chunked.ssd_chunked(*case, chunk=chunk)
    assert np.abs(y - yc).max() < 1e-11
    assert np.abs(hf - hc).max() < 1e-11


def test_strict_mask_mutant_is_caught():
    case = rand_case(8, L=16)
    y, _ = ssd.ssd_loop(*case)
    ym, _ = chunked.ssd_chunked(*case, chunk=8, keep_diagonal=False)
    assert np.abs(y - ym).max() > 1e-2


def test_chained_calls_carry_state():
    x, dt, A, B, C, D, h0 = rand_case(9, L=30)
    y, hf = ssd.ssd_loop(x, dt, A, B, C, D, h0)
    L1 = 11
    y1, h1 = ssd.ssd_loop(x[:, :L1], dt[:, :L1], A, B[:, :L1], C[:, :L1], D, h0)
    y2, h2 = ssd.ssd_loop(x[:, L1:], dt[:, L1:], A, B[:, L1:], C[:, L1:], D, h1)
    assert np.abs(np.concatenate([y1, y2], axis=1) - y).max() < 1e-12
    assert np.abs(h2 - hf).max() < 1e-12


def test_one_state_one_channel_is_the_scalar_scan():
    rng = np.random.default_rng(10)
    Bt, L, H = 2, 40, 3
    x = rng.standard_normal((Bt, L, H, 1))
    B = rng.standard_normal((Bt, L, 1, 1))
    C = np.ones((Bt, L, 1, 1))
    dt = np.log1p(np.exp(rng.standard_normal((Bt, L, H)) - 2))
    A = -np.exp(rng.uniform(0, math.log(16), H))
    y, _ = ssd.ssd_loop(x, dt, A, B, C, None, None)
    for b in range(Bt):
        a_rows = np.exp(A[None, :] * dt[b]).T                     # [H, L]
        b_rows = (dt[b] * B[b, :, 0, 0][:, None] * x[b, :, :, 0]).T
        h = scan.scan_loop(a_rows, b_rows)
        assert np.abs(y[b, :, :, 0].T - h).max() < 1e-12


def test_group_mapping_is_contiguous_head_blocks():
    x, dt, A, B, C, D, h0 = rand_case(11, H=4, G=2)
    y, _ = ssd.ssd_loop(x, dt, A, B, C, D, h0)
    B2, C2 = B.copy(), C.copy()
    B2[:, :, 1] += 1.0
    C2[:, :, 1] -= 0.5
    y2, _ = ssd.ssd_loop(x, dt, A, B2, C2, D, h0)
    # heads 0,1 read group 0 and are unchanged; heads 2,3 read group 1
    assert np.abs(y2[:, :, :2] - y[:, :, :2]).max() == 0.0
    assert np.abs(y2[:, :, 2:] - y[:, :, 2:]).max() > 1e-3


def test_identical_heads_in_a_group_agree():
    x, dt, A, B, C, D, h0 = rand_case(12, H=4, G=1, h0=False)
    for h in range(1, 4):
        x[:, :, h] = x[:, :, 0]
        dt[:, :, h] = dt[:, :, 0]
    A[:] = A[0]
    D[:] = D[0]
    y, _ = ssd.ssd_loop(x, dt, A, B, C, D, None)
    for h in range(1, 4):
        assert np.array_equal(y[:, :, h], y[:, :, 0])


# ---- the decode step ---------------------------------------------------------

def test_step_hand_worked_token():
    """One head, P = S = 2, worked by hand: A = -ln 2 and dt = 1 give a decay of
    1/2 and b = dt B = (2, -1).  With h (rows p, columns s) = [[1, 2], [3, 4]]
    and x = (1, -2):
        h_new[0] = 0.5 (1, 2) + 1 (2, -1) = (2.5, 0.0)
        h_new[1] = 0.5 (3, 4) - 2 (2, -1) = (-2.5, 4.0)
    and with c = (1, 3), D = 0.5:  y[0] = 2.5 + 0 + 0.5 = 3.0,
    y[1] = -2.5 + 12 - 1 = 8.5."""
    h = np.array([[[[1.0, 2.0], [3.0, 4.0]]]])
    x = np.array([[[1.0, -2.0]]])
    dt = np.array([[1.0]])
    A = np.array([-math.log(2.0)])
    B = np.array([[[2.0, -1.0]]])
    C = np.array([[[1.0, 3.0]]])
    D = np.array([0.5])
    y, hn = ssd.ssd_step(h, x, dt, A, B, C, D)
    assert np.abs(hn[0, 0] - np.array([[2.5, 0.0], [-2.5, 4.0]])).max() < 1e-14
    assert np.abs(y[0, 0] - np.array([3.0, 8.5])).max() < 1e-14


def test_step_zero_timestep_keeps_state():
    x, dt, A, B, C, D, h0 = rand_case(31, L=1)
    y, hn = ssd.ssd_step(h0, x[:, 0], np.zeros_like(dt[:, 0]), A, B[:, 0], C[:, 0], D)
    assert np.array_equal(hn, h0)
    grp = np.arange(4) // 2
    expect = np.einsum("bhps,bhs->bhp", h0, C[:, 0][:, grp]) + D[None, :, None] * x[:, 0]
    assert np.abs(y - expect).max() < 1e-13


def test_step_full_decay_forgets_the_state():
    """A very negative A (decay exp(-inf-like) = 0): the new state is b x^T alone."""
    x, dt, A, B, C, D, h0 = rand_case(32, L=1)
    A = np.full_like(A, -1e6)
    y, hn = ssd.ssd_step(h0, x[:, 0], dt[:, 0], A, B[:, 0], C[:, 0], None)
    grp = np.arange(4) // 2
    b = dt[:, 0, :, None] * B[:, 0][:, grp]
    assert np.abs(hn - x[:, 0, :, :, None] * b[:, :, None, :]).max() < 1e-13


@pytest.mark.parametrize("chunk", [4, 16])
def test_step_rollout_matches_chunked(chunk):
    """Decode after prefill: running the step token by token from h0 gives the
    outputs and final state of the independent chunked formulation."""
    x, dt, A, B, C, D, h0 = rand_case(33, L=37)
    yc, hc = chunked.ssd_chunked(x, dt, A, B, C, D, h0, chunk=chunk)
    h = h0.copy()
    for t in range(x.shape[1]):
        y, h = ssd.ssd_step(h, x[:, t], dt[:, t], A, B[:, t], C[:, t], D)
        assert np.abs(y - yc[:, t]).max() < 1e-11
    assert np.abs(h - hc).max() < 1e-11


def test_step_previous_state_output_differs():
    """The literal h_{t-1} reading of the page's renamed form gives other
    outputs, so the reading the step takes is observable."""
    x, dt, A, B, C, D, h0 = rand_case(34, L=1)
    y, _ = ssd.ssd_step(h0, x[:, 0], dt[:, 0], A, B[:, 0], C[:, 0], D)
    yp, _ = ssd.ssd_loop(x, dt, A, B, C, D, h0, y_uses_previous_state=True)
    assert np.abs(y - yp[:, 0]).max() > 1e-3


def test_abs_terms_hand_value():
    """One token, P = S = 1: y = c (exp(a) h0 + dt b x) + D x.  With a = A dt =
    -ln 2 * 1 the decay is 1/2; x = -3, B = 2, C = -1, D = 0.5, h0 = -4, dt = 1:
    the terms of h are (1/2)(-4) = -2 and 1*2*(-3) = -6, so h = -8 and
    h_abs = 2 + 6 = 8; y = (-1)(-8) + 0.5(-3) = 6.5 and y_abs = 1*8 + 0.5*3 = 9.5."""
    x = np.array([[[[-3.0]]]])
    dt = np.array([[[1.0]]])
    A = np.array([-math.log(2.0)])
    B = np.array([[[[2.0]]]])
    C = np.array([[[[-1.0]]]])
    D = np.array([0.5])
    h0 = np.array([[[[-4.0]]]])
    y, h = ssd.ssd_loop(x, dt, A, B, C, D, h0)
    ya, ha = ssd.ssd_abs_terms(x, dt, A, B, C, D, h0)
    assert y[0, 0, 0, 0] == pytest.approx(6.5, abs=1e-14) and h[0, 0, 0, 0] == pytest.approx(-8.0, abs=1e-14)
    assert ya[0, 0, 0, 0] == pytest.approx(9.5, abs=1e-14) and ha[0, 0, 0, 0] == pytest.approx(8.0, abs=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_abs_terms_bound_the_outputs(seed):
    """Triangle inequality: |y| <= y_abs and |h| <= h_abs element by element,
    with equality when every input is nonnegative."""
    case = rand_case(100 + seed)
    y, h = ssd.ssd_loop(*case)
    ya, ha = ssd.ssd_abs_terms(*case)
    assert np.all(np.abs(y) <= ya * (1 + 1e-12)) and np.all(np.abs(h) <= ha * (1 + 1e-12))
    assert np.mean(ya) > 1.5 * np.mean(np.abs(y))  # random signs cancel: the scale is not |y|
    pos = [None if v is None else np.abs(v) for v in case]
    pos[1] = case[1]
    pos[2] = case[2]
    yp, hp = ssd.ssd_loop(*pos)
    yq, hq = ssd.ssd_abs_terms(*pos)
    np.testing.assert_allclose(yq, yp, rtol=1e-13)
    np.testing.assert_allclose(hq, hp, rtol=1e-13)
    with pytest.raises(ValueError):
        ssd.ssd_abs_terms(case[0], -case[1], *case[2:])
