"""GPU parity tests for ssd_fwd (HIP path through the C ABI) against the
float64 oracle.

Tolerances: rel-L2 <= 1e-5 for fp32 inputs and <= 2e-2 for bf16 inputs (fp32
state), for y and for the final state.  Small shapes are compared element by
element in full; the full-size workloads are compared on sampled
(batch, head) sequences, which the oracle runs exactly (a head's outputs
depend only on its own inputs and its group's B/C).
"""
import math
import sys

import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
from oracle import compare, ssd as ossd

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def to_dev(inp):
    out = {}
    for k, v in inp.items():
        out[k] = v.cuda() if isinstance(v, torch.Tensor) else v
    return out


def gpu_run(inp, chunk=None, want_final=True):
    d = to_dev(inp)
    y, hf = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"), d.get("h0"),
                        chunk=chunk or inp["chunk"], want_final_state=want_final)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), (None if hf is None else hf.cpu().numpy())


def np64(t):
    return None if t is None else t.to(torch.float64).numpy()


def oracle_run(inp, batches=None, heads=None):
    """Oracle on a subset of (batch, head); each chosen head gets its own group."""
    x, dt, A, B, C, D, h0 = (inp[k] for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    H, G = x.shape[2], B.shape[2]
    bsel = list(range(x.shape[0])) if batches is None else list(batches)
    hsel = list(range(H)) if heads is None else list(heads)
    if heads is None:
        sub = dict(x=x[bsel], dt=dt[bsel], A=A, B=B[bsel], C=C[bsel], D=D,
                   h0=None if h0 is None else h0[bsel])
    else:
        grp = [h // (H // G) for h in hsel]
        sub = dict(x=x[bsel][:, :, hsel], dt=dt[bsel][:, :, hsel], A=A[hsel],
                   B=B[bsel][:, :, grp], C=C[bsel][:, :, grp], D=None if D is None else D[hsel],
                   h0=None if h0 is None else h0[bsel][:, hsel])
    y, hf = ossd.ssd_loop(*(np64(sub[k]) for k in ("x", "dt", "A", "B", "C", "D", "h0")))
    return y, hf, bsel, hsel


def assert_close(got, ref, tol, label):
    err = compare.rel_l2(got, ref)
    mm = compare.first_mismatch(got, ref, rtol=50 * tol, atol=50 * tol)
    print(f"  {label}: rel-L2 {err:.3e}", flush=True)
    assert err <= tol, (label, err, mm)
    return err


def small_case(seed, Bt, L, H, P, S, G, dtype, h0=True, D=True, dt_shift=-2.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(Bt, L, H, P, generator=g).to(dtype)
    B = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    C = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    dt = torch.nn.functional.softplus(torch.randn(Bt, L, H, generator=g) + dt_shift)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    Dv = torch.randn(H, generator=g) if D else None
    hv = 0.3 * torch.randn(Bt, H, P, S, generator=g) if h0 else None
    return {"x": x, "dt": dt, "A": A, "B": B, "C": C, "D": Dv, "h0": hv, "chunk": 32}


def test_tiny_fp32_workload():
    inp = workloads.ssd_workload("ssd_tiny")
    print("[ssd] ssd_tiny fp32", flush=True)
    y, hf = gpu_run(inp)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_F32, "y")
    assert_close(hf, rh, TOL_F32, "h_final")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_fp32_chunk_sizes_and_ragged(chunk):
    inp = small_case(1, 2, 300, 4, 16, 16, 2, torch.float32)
    print(f"[ssd] fp32 chunk={chunk}", flush=True)
    y, hf = gpu_run(inp, chunk=chunk)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_F32, "y")
    assert_close(hf, rh, TOL_F32, "h_final")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("P,S", [(16, 32), (64, 128), (32, 64), (128, 64)])
def test_bf16_shapes_chunks_ragged(P, S, chunk):
    if not cls.load_library().ssd_fwd_workspace_size(2, 301, 4, P, S, 2, chunk, cls.SSD_BF16):
        pytest.skip("shape not supported by the bf16 kernels at this chunk")
    inp = small_case(2, 2, 301, 4, P, S, 2, torch.bfloat16)
    print(f"[ssd] bf16 P={P} S={S} chunk={chunk}", flush=True)
    y, hf = gpu_run(inp, chunk=chunk)
    ry, rh, _, _ = oracle_run(inp)
    e = assert_close(y, ry, TOL_BF16, "y")
    assert_close(hf, rh, TOL_BF16, "h_final")
    assert e < 1e-2  # bf16 operand rounding alone stays well under the bound
    head, tail = compare.band_report(y, ry, chunk, axis=1)
    assert head <= TOL_BF16 and tail <= TOL_BF16


def test_bf16_edge_lengths():
    for L in (1, 2, 31, 32, 33, 255, 257):
        inp = small_case(3 + L, 1, L, 2, 64, 128, 1, torch.bfloat16)
        print(f"[ssd] bf16 L={L}", flush=True)
        y, hf = gpu_run(inp, chunk=256)
        ry, rh, _, _ = oracle_run(inp)
        assert_close(y, ry, TOL_BF16, f"y L={L}")
        assert_close(hf, rh, TOL_BF16, f"h L={L}")


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
def test_whole_chains_many_chunks(chunk):
    """Every (batch, head) chain in one workgroup (segments forced to 1), so a
    workgroup walks tens of (sub-)chunks: the loaders' register sets, the
    double-buffered LDS halves and the staged outputs all rotate many times,
    with a ragged last chunk."""
    ct = __import__("ctypes")
    lib = cls.load_library()
    lib.cls_ssd_set_segments.argtypes = [ct.c_int]
    print(f"[ssd] whole chains, chunk={chunk}", flush=True)
    inp = small_case(90 + chunk, 1, 64 * 40 + 17, 2, 64, 128, 1, torch.bfloat16, dt_shift=-3.0)
    lib.cls_ssd_set_segments(1)
    try:
        y, hf = gpu_run(inp, chunk=chunk)
    finally:
        lib.cls_ssd_set_segments(0)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, f"y chunk={chunk}")
    assert_close(hf, rh, TOL_BF16, f"h chunk={chunk}")


def test_optional_arguments():
    inp = small_case(4, 1, 200, 2, 64, 128, 1, torch.bfloat16, h0=False, D=False)
    y, hf = gpu_run(inp, chunk=64, want_final=False)
    assert hf is None
    ry, _, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, "y (no D, no h0)")


def test_decay_free_and_zero_timestep():
    inp = small_case(5, 1, 160, 2, 64, 128, 1, torch.bfloat16)
    inp["A"] = torch.zeros_like(inp["A"])  # linear attention
    y, hf = gpu_run(inp, chunk=64)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, "y a=0")
    inp = small_case(6, 1, 160, 2, 64, 128, 1, torch.bfloat16)
    inp["dt"] = torch.zeros_like(inp["dt"])  # state stays h0
    y, hf = gpu_run(inp, chunk=64)
    assert np.abs(hf - inp["h0"].numpy()).max() == 0.0
    ry, _, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, "y dt=0")


def test_chained_calls_carry_state():
    inp = small_case(7, 2, 512, 4, 64, 128, 2, torch.bfloat16)
    d = to_dev(inp)
    y_full, h_full = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=128)
    L1 = 256
    sl = lambda t, a, b: t[:, a:b].contiguous()
    y1, h1 = cls.ssd_fwd(sl(d["x"], 0, L1), sl(d["dt"], 0, L1), d["A"], sl(d["B"], 0, L1),
                         sl(d["C"], 0, L1), d["D"], d["h0"], chunk=128)
    y2, h2 = cls.ssd_fwd(sl(d["x"], L1, 512), sl(d["dt"], L1, 512), d["A"], sl(d["B"], L1, 512),
                         sl(d["C"], L1, 512), d["D"], h1, chunk=128)
    torch.cuda.synchronize()
    # the chunk boundaries coincide, so the split run performs the same arithmetic
    assert torch.equal(torch.cat([y1, y2], dim=1), y_full)
    assert torch.equal(h2, h_full)


def test_one_state_one_channel_matches_linear_scan():
    """S = P = 1 embedded in a 4 x 4 fp32 problem (other channels zero, C = 1
    on the live channel): y equals the scalar scan of (exp(A dt), dt B x)."""
    g = torch.Generator().manual_seed(8)
    Bt, L, H = 2, 777, 3
    x = torch.zeros(Bt, L, H, 4)
    B = torch.zeros(Bt, L, 1, 4)
    C = torch.zeros(Bt, L, 1, 4)
    x[..., 0] = torch.randn(Bt, L, H, generator=g)
    B[..., 0] = torch.randn(Bt, L, 1, generator=g)
    C[..., 0] = 1.0
    dt = torch.nn.functional.softplus(torch.randn(Bt, L, H, generator=g) - 2)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    inp = {"x": x, "dt": dt, "A": A, "B": B, "C": C, "D": None, "h0": None, "chunk": 64}
    y, _ = gpu_run(inp)
    a_rows = torch.exp(A[None, None, :] * dt).permute(0, 2, 1).reshape(Bt * H, L).contiguous()
    b_rows = (dt * B[..., 0, 0][:, :, None] * x[..., 0]).permute(0, 2, 1).reshape(Bt * H, L).contiguous()
    h = cls.linear_scan(a_rows.cuda(), b_rows.cuda()).cpu().numpy()
    ys = y[..., 0].transpose(0, 2, 1).reshape(Bt * H, L)
    assert compare.rel_l2(ys, h) < 1e-5


def test_deterministic():
    inp = small_case(9, 2, 1024, 8, 64, 128, 2, torch.bfloat16)
    d = to_dev(inp)
    y0, h0 = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=256)
    for _ in range(20):
        y1, h1 = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=256)
        assert torch.equal(y0, y1) and torch.equal(h0, h1)


FULL = [("ssd_small", [0, 7], [0, 13, 23]), ("ssd_large", [0, 3], [0, 41, 79]),
        ("ssd_long", [0], [0, 9, 18, 63])]


@pytest.mark.parametrize("name,bsel,hsel", FULL)
def test_full_workloads_sampled(name, bsel, hsel):
    print(f"[ssd] {name} full size, sampled b={bsel} h={hsel}", flush=True)
    inp = workloads.ssd_workload(name)
    y, hf = gpu_run(inp)
    ry, rh, _, _ = oracle_run(inp, batches=bsel, heads=hsel)
    gy = y[bsel][:, :, hsel]
    gh = hf[bsel][:, hsel]
    assert_close(gy, ry, TOL_BF16, f"{name} y")
    assert_close(gh, rh, TOL_BF16, f"{name} h_final")
    # every sampled sequence on its own, and its last chunk
    for bi in range(len(bsel)):
        for hi in range(len(hsel)):
            assert compare.rel_l2(gy[bi, :, hi], ry[bi, :, hi]) <= TOL_BF16
            T = inp["chunk"]
            assert compare.rel_l2(gy[bi, -T:, hi], ry[bi, -T:, hi]) <= TOL_BF16
    assert np.isfinite(y).all()


@pytest.mark.parametrize("nsegs", [1, 2, 3, 7, 64])
def test_segment_lookback_forced(nsegs):
    """The fused path splits each sequence into segments whose start states
    come from the aggregate launch's pieces, folded in order; force the segment
    count so the fold runs with one-chunk segments, uneven segments and many
    segments."""
    lib = cls.load_library()
    lib.cls_ssd_set_segments.argtypes = [__import__("ctypes").c_int]
    inp = small_case(20 + nsegs, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    lib.cls_ssd_set_segments(nsegs)
    try:
        y, hf = gpu_run(inp, chunk=32)
    finally:
        lib.cls_ssd_set_segments(0)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, f"y nsegs={nsegs}")
    assert_close(hf, rh, TOL_BF16, f"h nsegs={nsegs}")


@pytest.mark.parametrize("nsegs,nsplit,chunk", [(2, 1, 128), (5, 4, 128), (4, 5, 32), (3, 2, 64)])
def test_segment_mixed_whole_and_split(nsegs, nsplit, chunk):
    """Plans that run some (batch, head) chains whole and split the last
    `nsplit` chains into segments (the shape of the plan that fills the CUs
    left idle by a partial last round): both kinds of tile in one launch."""
    ct = __import__("ctypes")
    lib = cls.load_library()
    lib.cls_ssd_set_segments.argtypes = [ct.c_int]
    lib.cls_ssd_set_split.argtypes = [ct.c_int]
    print(f"[ssd] mixed plan nsegs={nsegs} nsplit={nsplit} chunk={chunk}", flush=True)
    inp = small_case(60 + nsegs, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    lib.cls_ssd_set_segments(nsegs)
    lib.cls_ssd_set_split(nsplit)
    try:
        y, hf = gpu_run(inp, chunk=chunk)
    finally:
        lib.cls_ssd_set_segments(0)
        lib.cls_ssd_set_split(0)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, f"y nsegs={nsegs} nsplit={nsplit}")
    assert_close(hf, rh, TOL_BF16, f"h nsegs={nsegs} nsplit={nsplit}")


@pytest.mark.parametrize("nsegs,pieces,chunk", [(3, 1, 64), (3, 5, 64), (4, 16, 32), (2, 40, 64), (5, 3, 128)])
def test_aggregate_pieces_forced(nsegs, pieces, chunk):
    """The aggregate launch cuts each segment but the last into `pieces`
    pieces (the autotuner searches this count); the output launch folds them
    in order.  Counts from one piece per segment to one chunk per piece (the
    count is capped at the segment's chunks), uneven last pieces included."""
    ct = __import__("ctypes")
    lib = cls.load_library()
    lib.cls_ssd_set_segments.argtypes = [ct.c_int]
    lib.cls_ssd_set_agg_pieces.argtypes = [ct.c_int]
    print(f"[ssd] aggregate pieces nsegs={nsegs} pieces={pieces} chunk={chunk}", flush=True)
    inp = small_case(80 + pieces, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    lib.cls_ssd_set_segments(nsegs)
    lib.cls_ssd_set_agg_pieces(pieces)
    try:
        y, hf = gpu_run(inp, chunk=chunk)
    finally:
        lib.cls_ssd_set_segments(0)
        lib.cls_ssd_set_agg_pieces(0)
    ry, rh, _, _ = oracle_run(inp)
    assert_close(y, ry, TOL_BF16, f"y nsegs={nsegs} pieces={pieces}")
    assert_close(hf, rh, TOL_BF16, f"h nsegs={nsegs} pieces={pieces}")
