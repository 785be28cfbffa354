"""Pins for the float64 scan oracle and the look-back protocol simulator (CPU).

The scan loop is tied to a hand-worked fixture, library routines (cumulative
sum), closed forms and row permutation; the simulator is tied to the loop
under many interleavings, and its swapped-combine mutant must fail.
"""
import json
import os

import numpy as np
import pytest

from oracle import lookback, scan


def test_hand_worked_fixture(golden_dir):
    with open(os.path.join(golden_dir, "scan_hand.json")) as f:
        g = json.load(f)
    h = scan.scan_loop(np.array(g["a"]), np.array(g["b"]))
    np.testing.assert_array_equal(h, np.array(g["h"]))
    c = g["combine"]
    assert list(scan.combine(c["first"], c["second"])) == c["first_then_second"]
    assert list(scan.combine(c["second"], c["first"])) == c["second_then_first"]


def test_unit_decay_is_cumsum():
    b = np.random.default_rng(0).standard_normal((3, 500))
    h = scan.scan_loop(np.ones_like(b), b)
    assert np.abs(h - np.cumsum(b, axis=1)).max() < 1e-11


def test_zero_decay_is_identity():
    b = np.random.default_rng(1).standard_normal((3, 100))
    np.testing.assert_array_equal(scan.scan_loop(np.zeros_like(b), b), b)


@pytest.mark.parametrize("c", [0.5, 0.9, 0.999999])
def test_constant_decay_geometric_series(c):
    L = 2000
    h = scan.scan_loop(np.full((1, L), c), np.ones((1, L)))
    t = np.arange(L)
    expect = (1.0 - c ** (t + 1)) / (1.0 - c)
    assert np.abs(h[0] - expect).max() < 1e-9 * expect.max()


def test_rows_are_independent():
    rng = np.random.default_rng(2)
    a = rng.uniform(0.9, 1.0, (5, 64))
    b = rng.standard_normal((5, 64))
    perm = rng.permutation(5)
    np.testing.assert_array_equal(scan.scan_loop(a, b)[perm], scan.scan_loop(a[perm], b[perm]))


def test_combine_is_associative_not_commutative():
    rng = np.random.default_rng(3)
    for _ in range(100):
        p, q, r = (tuple(rng.standard_normal(2)) for _ in range(3))
        lhs = scan.combine(scan.combine(p, q), r)
        rhs = scan.combine(p, scan.combine(q, r))
        assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    assert scan.combine((2.0, 3.0), (5.0, 7.0)) != scan.combine((5.0, 7.0), (2.0, 3.0))


def _pairs(a, b):
    return [(float(x), float(y)) for x, y in zip(a, b)]


@pytest.mark.parametrize("tile,window,resident,seed", [
    (1, 1, 4, 0), (1, 64, 16, 1), (3, 2, 8, 2), (8, 64, 3, 3), (5, 4, 32, 4), (16, 64, 64, 5),
])
def test_lookback_protocol_matches_loop(tile, window, resident, seed):
    rng = np.random.default_rng(seed)
    n = 301
    a = rng.uniform(0.5, 1.0, n)
    b = rng.standard_normal(n)
    ref = scan.scan_loop(a[None], b[None])[0]
    out = lookback.lookback_scan(_pairs(a, b), scan.combine, None, tile=tile,
                                 window=window, seed=seed, resident=resident)
    assert np.abs(np.array([v[1] for v in out]) - ref).max() < 1e-12


def test_lookback_swapped_combine_is_caught():
    rng = np.random.default_rng(6)
    n = 200
    a = rng.uniform(0.5, 1.0, n)
    b = rng.standard_normal(n)
    ref = scan.scan_loop(a[None], b[None])[0]
    out = lookback.lookback_scan(_pairs(a, b), scan.combine, None, tile=8, window=4,
                                 seed=1, resident=8, swap_combine=True)
    assert np.abs(np.array([v[1] for v in out]) - ref).max() > 1e-3


def test_lookback_stalled_predecessor_is_reported():
    pairs = [(0.9, 1.0)] * 64
    with pytest.raises(lookback.Deadlock):
        lookback.lookback_scan(pairs, scan.combine, None, tile=4, window=4, seed=0,
                               resident=4, max_steps=20_000, never_publish=3)


def test_lookback_matrix_payload_carries_chunk_states():
    """The inter-chunk state recurrence is the same scan over (alpha, S)
    pairs with S a matrix: (a1, S1) then (a2, S2) -> (a1 a2, a2 S1 + S2)."""
    rng = np.random.default_rng(7)
    n = 40
    alphas = rng.uniform(0.2, 1.0, n)
    mats = [rng.standard_normal((3, 4)) for _ in range(n)]
    h0 = rng.standard_normal((3, 4))
    elems = [(alphas[0], alphas[0] * h0 + mats[0])] + list(zip(alphas[1:], mats[1:]))
    ref = []
    h = h0
    for al, m in zip(alphas, mats):
        h = al * h + m
        ref.append(h)
    out = lookback.lookback_scan(elems, scan.combine, None, tile=3, window=4, seed=3, resident=6)
    assert max(np.abs(o[1] - r).max() for o, r in zip(out, ref)) < 1e-12


def test_error_scale_hand_values():
    """a = (0.5, -2, 1), b = (1, -1, 2): h_abs = scan(|a|, |b|) is 1, then
    2*1 + 1 = 3, then 1*3 + 2 = 5; the scale scan(|a|, h_abs) is 1, then
    2*1 + 3 = 5, then 1*5 + 5 = 10."""
    a = np.array([[0.5, -2.0, 1.0]])
    b = np.array([[1.0, -1.0, 2.0]])
    np.testing.assert_allclose(scan.scan_error_scale(a, b), [[1.0, 5.0, 10.0]], rtol=1e-15)


def test_error_scale_of_cumsum():
    """a = 1: h_abs is the running sum of |b| and the scale its running sum."""
    rng = np.random.default_rng(4)
    b = rng.standard_normal((3, 50))
    want = np.cumsum(np.cumsum(np.abs(b), axis=1), axis=1)
    np.testing.assert_allclose(scan.scan_error_scale(np.ones_like(b), b), want, rtol=1e-13)


@pytest.mark.parametrize("tile,window,resident", [(8, 4, 6), (3, 64, 16), (16, 2, 3)])
@pytest.mark.parametrize("seed", range(6))
def test_lookback_with_torn_halves_matches_loop(tile, window, resident, seed):
    """Status words written and read as two tagged halves at separate steps,
    with inclusive prefixes overwriting aggregates in place: a reader that
    accepts a word only when both halves carry the same tag gets the scan of
    the loop under every interleaving."""
    rng = np.random.default_rng(50 + seed)
    a = rng.uniform(0.5, 1.0, 150)
    b = rng.standard_normal(150)
    out = lookback.lookback_scan_halves(_pairs(a, b), scan.combine, tile=tile, window=window, seed=seed,
                                        resident=resident)
    ref = scan.scan_loop(a[None], b[None])[0]
    np.testing.assert_allclose([o[1] for o in out], ref, rtol=1e-12, atol=1e-12)


def test_lookback_trusting_one_half_is_caught():
    """The broken reader that trusts the first half's tag mixes two
    publications (or a published half with an unpublished one)."""
    rng = np.random.default_rng(7)
    a = rng.uniform(0.5, 1.0, 200)
    b = rng.standard_normal(200)
    ref = scan.scan_loop(a[None], b[None])[0]
    caught = 0
    for seed in range(10):
        try:
            out = lookback.lookback_scan_halves(_pairs(a, b), scan.combine, tile=8, window=4, seed=seed,
                                                resident=6, check_tags=False)
            caught += not np.allclose([o[1] for o in out], ref, rtol=1e-9, atol=1e-9)
        except TypeError:  # an unpublished half (None) reached the combine
            caught += 1
    assert caught >= 8


@pytest.mark.parametrize("tile,anchor,resident", [(4, 4, 6), (3, 8, 16), (2, 64, 64), (5, 1, 3)])
@pytest.mark.parametrize("seed", range(5))
def test_anchored_lookback_matches_loop(tile, anchor, resident, seed):
    """The anchored form (inclusive prefixes only at every anchor-th tile,
    aggregates elsewhere) is the scan under any interleaving, torn reads
    included."""
    rng = np.random.default_rng(100 + seed)
    n = 257
    a = rng.uniform(0.5, 1.0, n)
    b = rng.standard_normal(n)
    ref = scan.scan_loop(a[None], b[None])[0]
    out = lookback.lookback_scan_halves(_pairs(a, b), scan.combine, tile=tile, window=64, seed=seed,
                                        resident=resident, anchor=anchor)
    assert np.abs(np.array([v[1] for v in out]) - ref).max() < 1e-12


def _f32_combine(first, second):
    a1, b1 = first
    a2, b2 = second
    return (np.float32(a1 * a2), np.float32(np.float32(a2 * b1) + b2))


def test_anchored_lookback_is_bit_identical_across_interleavings():
    """fp32 arithmetic: with the nearest-prefix protocol the combine grouping
    follows which predecessors had published, so seeded interleavings give
    different last bits; the anchored form gives one answer for every
    interleaving."""
    rng = np.random.default_rng(9)
    n = 600
    pairs = [(np.float32(x), np.float32(y)) for x, y in zip(rng.uniform(0.9, 1.0, n), rng.standard_normal(n))]
    nearest = {tuple(float(v[1]) for v in lookback.lookback_scan_halves(pairs, _f32_combine, tile=5, window=64,
                                                                         seed=s, resident=16))
               for s in range(20)}
    anchored = {tuple(float(v[1]) for v in lookback.lookback_scan_halves(pairs, _f32_combine, tile=5, window=64,
                                                                          seed=s, resident=16, anchor=8))
                for s in range(20)}
    assert len(nearest) > 1
    assert len(anchored) == 1


def test_anchor_wider_than_window_is_rejected():
    with pytest.raises(ValueError):
        lookback.lookback_scan_halves([(1.0, 0.0)] * 8, scan.combine, tile=1, window=4, anchor=8)
