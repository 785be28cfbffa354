"""GPU parity tests for linear_scan_three_pass (block scan, spine scan, apply;
HIP path through the C ABI) against the float64 oracle, and its agreement with
the single-pass look-back kernel, which it cross-checks.  Tolerance: rel-L2
<= 1e-5 for fp32 inputs."""
import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
from oracle import compare, scan as oscan
import parity

pytestmark = pytest.mark.gpu

TOL = 1e-5


def inputs(seed, rows, L):
    g = torch.Generator().manual_seed(seed)
    a = 0.9 + 0.1 * torch.rand(rows, L, generator=g)
    b = torch.randn(rows, L, generator=g)
    return a, b


def check(a, b, label, elementwise=True):
    print(f"[scan3] {label} rows={a.shape[0]} L={a.shape[1]}", flush=True)
    got = cls.linear_scan_three_pass(a.cuda(), b.cuda())
    one = cls.linear_scan(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    got, one = got.cpu().numpy(), one.cpu().numpy()
    parity.check_scan(a, b, got, label=label, elementwise=elementwise)
    assert compare.rel_l2(got, one) <= 2 * TOL, label  # the two GPU paths agree


@pytest.mark.parametrize("rows,L", [(2, 1), (3, 2), (5, 7), (4, 8191), (4, 8192), (3, 8193), (2, 24580),
                                    (3, 24581), (7, 40000), (1, 1 << 20)])
def test_edge_lengths(rows, L):
    a, b = inputs(rows * 1000 + L % 997, rows, L)
    check(a, b, f"edge {rows}x{L}", elementwise=L < (1 << 20))


@pytest.mark.parametrize("name", ["scan", "scan_ragged"])
def test_full_workload(name):
    w = workloads.scan_workload(name)
    check(w["a"], w["b"], name)


def test_decay_one_is_cumsum_and_zero_is_identity():
    g = torch.Generator().manual_seed(3)
    b = torch.randn(3, 20000, generator=g)
    got = cls.linear_scan_three_pass(torch.ones_like(b).cuda(), b.cuda()).cpu().numpy()
    ref = np.cumsum(b.numpy().astype(np.float64), axis=1)
    assert compare.rel_l2(got, ref) <= TOL
    got0 = cls.linear_scan_three_pass(torch.zeros_like(b).cuda(), b.cuda()).cpu().numpy()
    assert np.array_equal(got0, b.numpy())


def test_deterministic_100_runs():
    a, b = inputs(9, 16, 70000)
    da, db = a.cuda(), b.cuda()
    h0 = cls.linear_scan_three_pass(da, db)
    for i in range(100):
        assert torch.equal(cls.linear_scan_three_pass(da, db), h0), i
