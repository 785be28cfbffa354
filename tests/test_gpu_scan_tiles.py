"""GPU tests of the linear scan's tile sizes and its autotuner through the C
ABI (linear_scan_planned, linear_scan_autotune, linear_scan_plan,
linear_scan_autotune_reset).

Every fp32 tile instance (4096, 8192, 16384 elements) must match the float64
oracle to the scan's tolerances (tests/parity.py: rel-L2 <= 1e-5 per row and
band, element-wise against the oracle's error scale) at shapes around each
instance's packed-rows threshold (rows of at most tile - 6 elements are packed
whole into tiles) and ragged tails.  The tuner's choice is kept per shape and
is deterministic: later linear_scan, linear_scan_typed (fp32) and
linear_scan_noalloc calls return the tuner's own output bit for bit."""
import ctypes

import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
import parity

pytestmark = pytest.mark.gpu

TILES = (4096, 8192, 16384)


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("rows,L", [(2, 4089), (2, 4090), (2, 4091), (3, 4096), (2, 8186), (2, 8187), (3, 8192),
                                    (2, 16378), (2, 16379), (3, 16384), (3, 16385), (2, 24580), (1, 65533),
                                    (1000, 7), (5, 100), (7, 40000), (2, 49152)])
def test_every_tile_matches_the_oracle(tile, rows, L):
    print(f"[scan tile] tile={tile} rows={rows} L={L}", flush=True)
    w = workloads.make_scan_inputs(rows, L, seed=tile + rows * 131 + L)
    h = cls.linear_scan_planned(w["a"].cuda(), w["b"].cuda(), tile=tile)
    torch.cuda.synchronize()
    parity.check_scan(w["a"], w["b"], h.cpu().numpy(), label=f"tile {tile}")


@pytest.mark.parametrize("tile", (4096, 16384))
@pytest.mark.parametrize("name", ["scan", "scan_ragged"])
def test_tiles_on_the_full_workload(tile, name):
    print(f"[scan tile] tile={tile} workload={name}", flush=True)
    w = workloads.scan_workload(name)
    h = cls.linear_scan_planned(w["a"].cuda(), w["b"].cuda(), tile=tile)
    torch.cuda.synchronize()
    parity.check_scan(w["a"], w["b"], h.cpu().numpy(), label=f"{name} tile {tile}")


def test_planned_tile_zero_is_linear_scan():
    w = workloads.make_scan_inputs(9, 30000, seed=4)
    a, b = w["a"].cuda(), w["b"].cuda()
    assert torch.equal(cls.linear_scan_planned(a, b, tile=0), cls.linear_scan(a, b))


@pytest.mark.parametrize("rows,L", [(384, 65536), (384, 65533), (64, 20000)])
def test_autotune_result_plan_and_later_calls(rows, L):
    print(f"[scan tune] rows={rows} L={L}", flush=True)
    cls.linear_scan_autotune_reset()
    try:
        assert cls.linear_scan_plan(rows, L) == {"tile": 8192, "source": "built-in"}
        w = workloads.make_scan_inputs(rows, L, seed=rows + L)
        a, b = w["a"].cuda(), w["b"].cuda()
        h, info = cls.linear_scan_autotune(a, b, reps=5)
        torch.cuda.synchronize()
        assert info["tile"] in TILES and info["ms_per_call"] > 0.0
        assert cls.linear_scan_plan(rows, L) == {"tile": info["tile"], "source": "tuned"}
        later = cls.linear_scan(a, b)
        typed = torch.empty_like(a)
        lib = cls.load_library()
        ws = torch.zeros(lib.linear_scan_workspace_size(rows, L), dtype=torch.uint8, device="cuda")
        assert lib.linear_scan_typed(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                     ctypes.c_void_p(typed.data_ptr()), rows, L, cls.SSD_F32, cls.SSD_F32,
                                     ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
        noalloc = torch.empty_like(a)
        lib.linear_scan_noalloc.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
        lib.linear_scan_noalloc.restype = ctypes.c_int
        if lib.linear_scan_workspace_size(rows, L) <= (1 << 20):
            assert lib.linear_scan_noalloc(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                           ctypes.c_void_p(noalloc.data_ptr()), rows, L,
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == 0
        else:
            noalloc = h
        torch.cuda.synchronize()
        assert torch.equal(later, h) and torch.equal(typed, h) and torch.equal(noalloc, h)
        # the tuned tile is the one the planned call runs when asked for it
        assert torch.equal(cls.linear_scan_planned(a, b, tile=info["tile"]), h)
        parity.check_scan(w["a"], w["b"], h.cpu().numpy(), label=f"tuned {rows}x{L}")
    finally:
        cls.linear_scan_autotune_reset()
    assert cls.linear_scan_plan(rows, L)["source"] == "built-in"


@pytest.mark.parametrize("seed", [1, 77, 4099])
@pytest.mark.parametrize("tile,rows,L", [(8192, 384, 65536), (8192, 7, 100003), (4096, 3, 300000),
                                         (16384, 2, 200000), (8192, 1, 8192 * 200), (8192, 1000, 7)])
def test_lookback_stress_gives_the_same_bits(seed, tile, rows, L):
    """Look-back stress ("Selective-scan CUDA kernels", section "Correctness"):
    a quarter of the tiles, picked by a hash of the seed, wait up to ~100 us
    before they publish, so tiles publish and look back out of order.  The
    anchored look-back folds in an order fixed by the tile index, so the
    output equals the unperturbed call bit for bit, and the oracle within the
    scan's bounds.  1 x 8192·200 runs three anchors deep."""
    print(f"[scan stress] seed={seed} tile={tile} rows={rows} L={L}", flush=True)
    w = workloads.make_scan_inputs(rows, L, seed=seed + rows + L)
    a, b = w["a"].cuda(), w["b"].cuda()
    ref = cls.linear_scan_planned(a, b, tile=tile)
    got = cls.linear_scan_planned(a, b, tile=tile, stress_seed=seed)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    if rows * L <= 4_000_000:
        parity.check_scan(w["a"], w["b"], got.cpu().numpy(), label=f"stress {seed}", elementwise=rows * L < 1_000_000)
