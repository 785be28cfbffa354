"""GPU test of linear_scan_noalloc (the linear scan for callers that cannot
allocate) through the C ABI: its output equals linear_scan's bit for bit (same
kernels, same plan) on two calls in a row, the second smaller than the first,
so the second call runs on what the first left in the shared array; shapes
past the fixed array's size are rejected with nothing enqueued."""
import ctypes

import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
import parity

pytestmark = pytest.mark.gpu


def noalloc(lib, a, b, h):
    rows, L = a.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.linear_scan_noalloc(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(b.data_ptr()),
                                   ctypes.c_void_p(h.data_ptr()), rows, L, stream)


def setup_lib():
    lib = cls.load_library()
    lib.linear_scan_noalloc.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    lib.linear_scan_noalloc.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("first,second", [((384, 65536), (7, 100000)), ((300, 20000), (1000, 33)),
                                          ((5, 8193), (3, 8192))])
def test_noalloc_matches_linear_scan_twice(first, second):
    lib = setup_lib()
    for k, (rows, L) in enumerate((first, second)):
        print(f"[noalloc] call {k}: rows={rows} L={L}", flush=True)
        w = workloads.make_scan_inputs(rows, L, seed=500 + 7 * k + rows)
        a, b = w["a"].cuda(), w["b"].cuda()
        h = torch.empty_like(a)
        assert noalloc(lib, a, b, h) == 0
        ref = cls.linear_scan(a, b)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), ref.view(torch.int32)), (rows, L)
        if rows * L <= 3_000_000:
            parity.check_scan(w["a"], w["b"], h.cpu().numpy(), label=f"noalloc {rows}x{L}")


def test_noalloc_rejects_shapes_past_its_array():
    lib = setup_lib()
    need = lib.linear_scan_workspace_size(20000, 65536)
    assert need > (1 << 20)
    a = torch.empty(16, device="cuda")
    # validation runs before anything is launched; the pointers are not read
    st = lib.linear_scan_noalloc(ctypes.c_void_p(a.data_ptr()), ctypes.c_void_p(a.data_ptr()),
                                 ctypes.c_void_p(a.data_ptr()), 20000, 65536, None)
    assert st == -6
