"""GPU parity tests for linear_scan (HIP path through the C ABI) against the
float64 oracle, at full workload sizes and at edge sizes, plus determinism and
workspace hygiene.  Whole outputs are compared (tests/parity.py): rel-L2 <=
1e-5 for fp32 inputs, per row and per 8192-element tile band within 10x of
that, and an element-wise bound against the oracle's error scale."""
import sys

import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
from oracle import compare, scan as oscan
import parity

pytestmark = pytest.mark.gpu

TOL = 1e-5


def run(a, b):
    h = cls.linear_scan(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    return h.cpu().numpy()


def check(a, b, label="", elementwise=True):
    print(f"[scan] {label} rows={a.shape[0]} L={a.shape[1]}", flush=True)
    sys.stdout.flush()
    got = run(a, b)
    return parity.check_scan(a, b, got, label=label, elementwise=elementwise)


@pytest.mark.parametrize("name", ["scan", "scan_ragged"])
def test_full_workload(name):
    w = workloads.scan_workload(name)
    got, ref = check(w["a"], w["b"], label=name)
    head, tail = compare.band_report(got, ref, 8192, axis=1)
    assert head <= TOL and tail <= TOL


@pytest.mark.parametrize("rows,L", [
    (1, 1), (3, 1), (5, 2), (7, 3), (2, 4), (4, 5), (3, 31), (3, 32), (3, 33), (1, 4089), (2, 4090),
    (2, 4091), (2, 4093), (2, 4096), (2, 4097), (3, 8185), (2, 8186), (2, 8187), (3, 8191), (3, 8192),
    (3, 8193), (2, 16383), (2, 16384), (2, 16385), (3, 24576), (3, 24580), (1, 65533),
    (5, 12345), (1000, 7), (257, 129), (5, 4096), (9, 2048), (3, 8184), (7, 1024), (33, 256), (5, 4), (17, 8),
    (4097, 4), (5, 4094), (7, 2730), (4, 4093), (3, 8186), (11, 2047), (50, 431), (39, 431)])
def test_edge_sizes(rows, L):
    w = workloads.make_scan_inputs(rows, L, seed=rows * 7919 + L)
    check(w["a"], w["b"], label="edge")


def test_very_long_row():
    L = 1 << 22
    w = workloads.make_scan_inputs(2, L, seed=11)
    check(w["a"], w["b"], label="2^22", elementwise=False)


def test_long_lookback_chain():
    # 1024 tiles in one row: the 64-lane window walks back many times
    L = 8192 * 1024
    a = torch.full((1, L), 0.999, dtype=torch.float32)
    b = torch.randn(1, L, generator=torch.Generator().manual_seed(3))
    check(a, b, label="chain", elementwise=False)


def test_special_cases():
    g = torch.Generator().manual_seed(5)
    b = torch.randn(4, 20000, generator=g)
    got = run(torch.zeros_like(b), b)
    assert np.array_equal(got, b.numpy())
    got = run(torch.ones(4, 3000), b[:, :3000].contiguous())
    ref = np.cumsum(b[:, :3000].numpy().astype(np.float64), axis=1)
    assert compare.rel_l2(got, ref) < TOL


def test_rows_do_not_leak_nonfinite_values():
    # short rows are packed into one tile: an overflow in row 0 must not reach row 1
    a = torch.full((3, 50), 10.0)
    a[1] = 0.5
    a[2] = 0.9
    b = torch.ones(3, 50)
    got = run(a, b)
    assert np.isinf(got[0, -1])
    ref = oscan.scan_loop(a[1:].numpy(), b[1:].numpy())
    assert compare.rel_l2(got[1:], ref) < TOL
    # long rows chain through the look-back: same check across rows
    a = torch.full((2, 9000), 1.5)
    a[1] = 0.95
    b = torch.ones(2, 9000)
    got = run(a, b)
    ref = oscan.scan_loop(a[1:].numpy(), b[1:].numpy())
    assert compare.rel_l2(got[1:], ref) < TOL


def test_deterministic_and_workspace_reuse():
    w = workloads.scan_workload("scan_ragged")
    a, b = w["a"].cuda(), w["b"].cuda()
    lib = cls.load_library()
    need = lib.linear_scan_workspace_size(*a.shape)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    first = cls.linear_scan(a, b, workspace=ws)
    for _ in range(100):
        again = cls.linear_scan(a, b, workspace=ws)
        assert torch.equal(again, first)
    torch.cuda.synchronize()
    ref = oscan.scan_loop(w["a"].numpy(), w["b"].numpy())
    assert compare.rel_l2(first.cpu().numpy(), ref) <= TOL
    err_word = int(ws[:4].view(torch.int32).item())
    assert err_word == 0, "a look-back wait gave up"


def test_workspace_reused_across_shapes():
    """One workspace, shapes whose tile layout changes from call to call (and
    back): stale status words from other layouts must never be taken as
    current."""
    lib = cls.load_library()
    shapes = [(384, 65536), (7, 100000), (1000, 33), (3, 9000), (384, 65533), (7, 100000),
              (384, 65536), (200, 4097)]
    need = max(lib.linear_scan_workspace_size(r, L) for r, L in shapes)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (r, L) in enumerate(shapes):
        w = workloads.make_scan_inputs(r, L, seed=100 + i)
        got = cls.linear_scan(w["a"].cuda(), w["b"].cuda(), workspace=ws).cpu().numpy()
        ref = oscan.scan_loop(w["a"].numpy(), w["b"].numpy())
        assert compare.rel_l2(got, ref) <= TOL, (r, L)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0


TYPED = [(torch.bfloat16, torch.float32), (torch.bfloat16, torch.bfloat16), (torch.float32, torch.bfloat16),
         (torch.float16, torch.float32), (torch.float16, torch.float16), (torch.float32, torch.float16),
         (torch.bfloat16, torch.float16)]


@pytest.mark.parametrize("din,dout", TYPED)
@pytest.mark.parametrize("rows,L", [(3, 1), (5, 7), (3, 33), (2, 4097), (3, 8186), (2, 8187), (3, 8193),
                                    (2, 16378), (2, 16379), (2, 16384), (2, 16385), (3, 32771), (1000, 7),
                                    (257, 129), (3, 5461), (5, 4096), (9, 2048), (33, 256), (4097, 4),
                                    (4, 65536), (1, 65533), (50, 431), (9, 2047), (5, 4094)])
def test_typed_scan_matches_oracle(din, dout, rows, L):
    """bf16 / fp16 / fp32 elements through linear_scan_typed.  The oracle runs
    on the exact float64 values of the (possibly 16-bit) inputs.  With an fp32
    h the scan is the fp32 scan (rel-L2 <= 1e-5); a 16-bit h is that fp32
    result rounded to nearest even once, so it equals the fp32-output run
    rounded on the host bit for bit, and stays within that rounding of the
    oracle."""
    print(f"[scan typed] {din} -> {dout} rows={rows} L={L}", flush=True)
    w = workloads.make_scan_inputs(rows, L, seed=rows * 31 + L)
    a, b = w["a"].to(din), w["b"].to(din)
    h = cls.linear_scan(a.cuda(), b.cuda(), out_dtype=dout)
    torch.cuda.synchronize()
    assert h.dtype == dout
    got = h.float().cpu().numpy()
    parity.check_scan(a, b, got, out_bf16=dout == torch.bfloat16, out_f16=dout == torch.float16,
                      label=f"{din}->{dout}")
    if dout != torch.float32:
        h32 = cls.linear_scan(a.cuda(), b.cuda(), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(h.cpu().view(torch.int16), h32.cpu().to(dout).view(torch.int16))


def test_typed_scan_full_workload_bf16_inputs():
    w = workloads.scan_workload("scan")
    a, b = w["a"].to(torch.bfloat16), w["b"].to(torch.bfloat16)
    print(f"[scan typed] full workload bf16 -> fp32 {tuple(a.shape)}", flush=True)
    h = cls.linear_scan(a.cuda(), b.cuda())
    torch.cuda.synchronize()
    parity.check_scan(a, b, h.cpu().numpy(), label="bf16 in, full workload")


@pytest.mark.parametrize("rows,L", [(12288, 2048), (6144, 4096)])
def test_page_table_row_lengths(rows, L):
    """Two of the row lengths of the page's table ("Selective-scan CUDA
    kernels", section "Results": 96 MiB per array), which run as whole rows
    packed several to a tile."""
    w = workloads.make_scan_inputs(rows, L, seed=rows + L)
    check(w["a"], w["b"], label=f"page table L={L}")


@pytest.mark.parametrize("rows,L", [(1, 1), (3, 5), (2, 255), (2, 256), (3, 257), (5, 4096), (3, 8186), (2, 8187),
                                    (3, 8193), (2, 20000), (1000, 7), (257, 129), (4097, 4), (11, 2047)])
def test_hillis_steele_matches_oracle_and_single_pass(rows, L):
    """The register-resident Hillis-Steele kernel: whole-output parity with
    the oracle, on long rows (look-back across tiles) and packed short rows
    (row starts carried through the Hillis-Steele rounds), and agreement with
    the work-efficient kernel to fp32 rounding."""
    w = workloads.make_scan_inputs(rows, L, seed=rows * 13 + L)
    a, b = w["a"].cuda(), w["b"].cuda()
    print(f"[scan hs] rows={rows} L={L}", flush=True)
    hs = cls.linear_scan_hillis_steele(a, b)
    one = cls.linear_scan(a, b)
    torch.cuda.synchronize()
    got = hs.cpu().numpy()
    parity.check_scan(w["a"], w["b"], got, label=f"hillis-steele {rows}x{L}")
    assert compare.rel_l2(got, one.cpu().numpy()) <= 2 * TOL


@pytest.mark.parametrize("name", ["scan", "scan_ragged"])
def test_hillis_steele_full_workload(name):
    w = workloads.scan_workload(name)
    print(f"[scan hs] {name}", flush=True)
    got = cls.linear_scan_hillis_steele(w["a"].cuda(), w["b"].cuda()).cpu().numpy()
    parity.check_scan(w["a"], w["b"], got, label=f"hillis-steele {name}")


def test_hillis_steele_special_cases_and_determinism():
    g = torch.Generator().manual_seed(6)
    b = torch.randn(3, 30000, generator=g).cuda()
    assert torch.equal(cls.linear_scan_hillis_steele(torch.zeros_like(b), b), b)  # a = 0: h = b exactly
    got = cls.linear_scan_hillis_steele(torch.ones_like(b), b).cpu().numpy()
    ref = np.cumsum(b.cpu().numpy().astype(np.float64), axis=1)
    assert compare.rel_l2(got, ref) < TOL
    w = workloads.make_scan_inputs(16, 70000, seed=9)
    a, bb = w["a"].cuda(), w["b"].cuda()
    first = cls.linear_scan_hillis_steele(a, bb)
    for i in range(100):
        assert torch.equal(cls.linear_scan_hillis_steele(a, bb), first), i


@pytest.mark.parametrize("vec,nt,grid", [(1, 1, 0), (2, 0, 0), (4, 1, 0), (8, 1, 0), (8, 0, 0), (4, 1, 7),
                                         (8, 0, 300)])
def test_stream_kernel_is_an_exact_product(vec, nt, grid):
    """The streaming ceiling kernel computes h = a * b (one fp32 rounding, the
    same as torch's product) over every element, ragged tails included."""
    print(f"[stream] vec={vec} nt={nt} grid={grid}", flush=True)
    g = torch.Generator().manual_seed(vec * 10 + nt + grid)
    for n in (4, 1020, 256 * 4 * vec + 12, 1 << 20):
        a = torch.randn(n, generator=g).cuda()
        b = torch.randn(n, generator=g).cuda()
        h = torch.full_like(a, float("nan"))
        cls.stream_mul(a, b, out=h, vec=vec, nt=bool(nt), grid_blocks=grid)
        torch.cuda.synchronize()
        assert torch.equal(h, a * b), n
