"""C-ABI tests that need no GPU: the library loads, exports every function the
public header declares, and rejects bad arguments on the host before any
launch (validation runs before any HIP call)."""
import ctypes
import os
import re

import pytest

import chunked_linear_scan_amd as cls

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chunked_linear_scan.h")

pytestmark = pytest.mark.skipif(not os.path.exists(cls.LIB_PATH),
                                reason="library not built (run __graft_entry__.build())")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    skip = {"if", "sizeof", "defined"}
    return sorted({n for n in names if n not in skip})


def test_header_lists_expected_entry_points():
    assert set(header_functions()) == {
        "ssd_fwd_workspace_size", "ssd_fwd", "ssd_fwd_autotune", "ssd_fwd_plan", "ssd_fwd_autotune_reset",
        "linear_scan_workspace_size", "linear_scan", "linear_scan_typed", "linear_scan_noalloc", "linear_scan_hillis_steele", "ssd_step", "linear_scan_three_pass_workspace_size", "linear_scan_three_pass", "ssd_strerror",
        "linear_scan_autotune", "linear_scan_plan", "linear_scan_autotune_reset"}


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(cls.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_strerror_covers_every_status():
    for st in range(0, -9, -1):
        txt = cls.strerror(st)
        assert txt and txt != "unknown status"
    assert cls.strerror(-99) == "unknown status"


FAKE = ctypes.c_void_p(0x10000)  # 16-byte aligned, never dereferenced on error paths


def test_linear_scan_rejects_bad_arguments():
    lib = cls.load_library()
    ws = lib.linear_scan_workspace_size(4, 100)
    assert ws > 0
    assert lib.linear_scan(None, FAKE, FAKE, 4, 100, FAKE, ws, None) == -1
    assert lib.linear_scan(FAKE, FAKE, FAKE, 0, 100, FAKE, ws, None) == -2
    assert lib.linear_scan(FAKE, FAKE, FAKE, 4, -1, FAKE, ws, None) == -2
    assert lib.linear_scan(FAKE, ctypes.c_void_p(0x10004), FAKE, 4, 100, FAKE, ws, None) == -5
    assert lib.linear_scan(FAKE, FAKE, FAKE, 4, 100, FAKE, 0, None) == -6
    assert lib.linear_scan(FAKE, FAKE, FAKE, 4, 100, None, ws, None) == -1


def test_linear_scan_workspace_size_is_monotone_and_row_scaled():
    lib = cls.load_library()
    assert lib.linear_scan_workspace_size(0, 10) == 0
    short = lib.linear_scan_workspace_size(1000, 100)      # packed rows: header only
    long1 = lib.linear_scan_workspace_size(1, 65536)
    long384 = lib.linear_scan_workspace_size(384, 65536)
    assert short > 0 and long1 > 0
    assert long384 > long1
    assert long384 >= 384 * 8 * 16  # one 16-byte status word per 8192-element tile


def test_scan_workspace_covers_every_tile_size():
    """The size covers the smallest candidate tile (4096 elements): rows past
    4090 elements need status words even where 8192-element tiles pack them."""
    lib = cls.load_library()
    assert lib.linear_scan_workspace_size(5, 4090) == 256      # every tile size packs these rows
    assert lib.linear_scan_workspace_size(2, 8000) == 256 + 256 + 256 + 2 * 2 * 16
    # a row's tiles cover it from the 16-byte boundary at or before its start
    tiles = (65536 + 3 + 4095) // 4096
    assert lib.linear_scan_workspace_size(384, 65536) == 256 + 2 * 1536 + 384 * tiles * 16


def test_scan_plan_and_tuner_validate_on_host():
    lib = cls.load_library()
    lib.linear_scan_autotune_reset()
    tile = ctypes.c_int64()
    assert lib.linear_scan_plan(4, 100, ctypes.byref(tile)) == 0 and tile.value == 8192
    assert lib.linear_scan_plan(0, 100, ctypes.byref(tile)) == -2
    assert lib.linear_scan_plan(4, 100, None) == -1
    ws = lib.linear_scan_workspace_size(4, 100)
    for bad in (1000, 8193, -1, 32768):
        assert lib.linear_scan_planned(FAKE, FAKE, FAKE, 4, 100, bad, 0, FAKE, ws, None) == -2, bad
    assert lib.linear_scan_planned(None, FAKE, FAKE, 4, 100, 4096, 0, FAKE, ws, None) == -1
    ms = ctypes.c_float()
    assert lib.linear_scan_autotune(FAKE, FAKE, FAKE, 4, 100, FAKE, ws, None, 5, None, ctypes.byref(ms)) == -1
    assert lib.linear_scan_autotune(FAKE, FAKE, FAKE, 4, 100, FAKE, ws, None, 0, ctypes.byref(tile),
                                    ctypes.byref(ms)) == -2
    assert lib.linear_scan_autotune(FAKE, FAKE, FAKE, 4, 100, FAKE, ws - 16, None, 5, ctypes.byref(tile),
                                    ctypes.byref(ms)) in (-6, -2)
    assert lib.linear_scan_autotune(FAKE, FAKE, FAKE, 0, 100, FAKE, ws, None, 5, ctypes.byref(tile),
                                    ctypes.byref(ms)) == -2


def test_ssd_rejects_bad_arguments():
    lib = cls.load_library()
    args_ok = dict(Bt=1, L=64, H=2, P=16, S=32, G=1, T=32, dt=cls.SSD_BF16)

    def call(x=FAKE, dtp=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, ws=FAKE, ws_bytes=1 << 30, **kw):
        a = dict(args_ok)
        a.update(kw)
        return lib.ssd_fwd(x, dtp, A, B, C, None, None, a["Bt"], a["L"], a["H"], a["P"], a["S"],
                           a["G"], a["T"], a["dt"], y, None, ws, ws_bytes, None)

    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(Bt=0) == -2
    assert call(L=0) == -2  # an empty sequence is rejected, not run
    assert call(L=-5) == -2
    assert call(H=0) == -2
    assert call(P=0) == -2
    assert call(H=3, G=2) == -2
    assert call(dt=7) == -3
    assert call(T=48) == -4
    assert call(T=512) == -4
    assert call(B=ctypes.c_void_p(0x10008)) == -5
    assert call(ws_bytes=0) in (-6, -8)
    assert call(P=24) in (-8, -2)


def test_fp32_workspace_holds_segment_states_only_when_chains_are_cut():
    """The fp32 path needs no workspace for whole chains; cut into segments,
    it holds per chain and segment but the last a [P][S] fp32 state and a
    decay, after the 1 KB header."""
    lib = cls.load_library()
    up = lambda v: (v + 255) // 256 * 256
    # 2 chains of 8 chunks: no segments (at least 8 chunks each)
    assert lib.ssd_fwd_workspace_size(1, 256, 2, 16, 16, 1, 32, cls.SSD_F32) == 0
    # 64 chains of 64 chunks, P = S = 16: 8 segments of 8 chunks
    assert lib.ssd_fwd_workspace_size(2, 4096, 32, 16, 16, 2, 64, cls.SSD_F32) == \
        1024 + up(64 * 7 * 16 * 16 * 4) + 64 * 7 * 4
    # a plan request of 3 segments on the first shape
    three = cls.plan_request(nsegs=3)
    assert lib.ssd_fwd_planned_workspace_size(1, 256, 2, 16, 16, 1, 32, cls.SSD_F32, ctypes.byref(three)) == \
        1024 + up(2 * 2 * 16 * 16 * 4) + 2 * 2 * 4


def test_ssd_plan_request_c_source_is_validated():
    """c_source takes SSD_CSRC_AUTO, _COPY or _ROWS; any other value is
    refused before anything is sized or launched."""
    lib = cls.load_library()
    shape = (1, 1000, 8, 64, 128, 1, 128, cls.SSD_BF16)
    base = lib.ssd_fwd_workspace_size(*shape)
    for src in ("auto", "copy", "rows"):
        assert lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(cls.plan_request(c_source=src))) >= base > 0
    for bad_value in (-1, 3):
        bad = cls.plan_request()
        bad.c_source = bad_value
        assert lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(bad)) == 0


def test_ssd_workspace_size_zero_for_invalid_shapes():
    lib = cls.load_library()
    assert lib.ssd_fwd_workspace_size(1, 64, 3, 16, 32, 2, 32, 1) == 0
    assert lib.ssd_fwd_workspace_size(1, 64, 2, 16, 32, 1, 33, 1) == 0


def test_head_dim_128_takes_the_fused_path():
    """Head dim 128 with dstate 64 or 128 runs the fused kernels (a head as
    two chains of head dim 64) at every chunk length."""
    for S in (64, 128):
        for chunk in (16, 32, 64, 128, 256):
            p = cls.ssd_fwd_plan(2, 1000, 4, 128, S, 2, chunk)
            assert p["source"] == "heuristic" and p["nsegs"] >= 1
    assert cls.ssd_fwd_plan(2, 1000, 4, 128, 256, 2, 64)["source"] == "none"


def test_every_head_dim_and_state_size_of_the_set_is_supported():
    """bf16: every head dim in {16, 32, 64, 128} and state size in {32, 64,
    128, 256} runs at every chunk length, on the fused kernels or on the
    per-(batch, head) kernel (which runs a chunk whose tiles would overflow LDS
    as sub-chunks); a forced per-(batch, head) plan runs too.  Outside the set
    the shape is rejected before anything runs."""
    lib = cls.load_library()
    chunk_path = cls.plan_request(path="chunk")
    for P in (16, 32, 64, 128):
        for S in (32, 64, 128, 256):
            for chunk in (16, 32, 64, 128, 256):
                shape = (2, 1000, 4, P, S, 2, chunk, cls.SSD_BF16)
                assert lib.ssd_fwd_workspace_size(*shape) > 0, shape
                assert lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(chunk_path)) > 0, shape
    # the per-(batch, head) kernel's workspace is C B^T per (batch, sub-chunk,
    # group): 256-token chunks run as 128-token sub-chunks, and as 64-token
    # ones where the 128-token tiles overflow LDS (P = 128, S = 256).  Chains
    # cut into segments add, per chain and segment but the last, the segment's
    # fp32 state (a multiple of 4 state tiles of 16 x 16, one per wave) and its
    # decay.
    up = lambda v: (v + 255) // 256 * 256
    assert lib.ssd_fwd_workspace_size(2, 1000, 4, 32, 64, 2, 256, cls.SSD_BF16) == 2 * 8 * 2 * 128 * 128 * 2 + 1024
    # head dim 128 runs as 16 chains of head dim 64 (8 heads x 2), 16 sub-chunks
    # of 64 tokens in 2 segments: 16 aggregates of 4 x 4 tiles
    cb = 2 * 16 * 2 * 64 * 64 * 2
    assert lib.ssd_fwd_workspace_size(2, 1000, 4, 128, 256, 2, 256, cls.SSD_BF16) == \
        1024 + up(cb) + up(16 * 16 * 256 * 16) + 16 * 4
    # 8 chains of head dim 16, 63 sub-chunks of 16 tokens in 7 segments of 9:
    # 48 aggregates of 1 x 1 tiles
    cb = 2 * 63 * 2 * 32 * 32 * 2
    assert lib.ssd_fwd_workspace_size(2, 1000, 4, 16, 32, 2, 16, cls.SSD_BF16) == \
        1024 + up(cb) + up(48 * 1 * 256 * 16) + 48 * 4
    # a plan request of whole chains needs no more than ssd_fwd's workspace
    one = cls.plan_request(path="chunk", nsegs=1)
    assert lib.ssd_fwd_planned_workspace_size(2, 1000, 4, 16, 32, 2, 16, cls.SSD_BF16, ctypes.byref(one)) == \
        lib.ssd_fwd_workspace_size(2, 1000, 4, 16, 32, 2, 16, cls.SSD_BF16)
    for P, S in ((48, 64), (64, 96), (256, 64)):
        shape = (2, 1000, 4, P, S, 2, 64, cls.SSD_BF16)
        assert lib.ssd_fwd_workspace_size(*shape) == 0
        assert lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(chunk_path)) == 0
        st = lib.ssd_fwd_planned(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, *shape, FAKE, None, FAKE, 1 << 34, None,
                                 ctypes.byref(chunk_path), None)
        assert st == -8


def test_ssd_step_rejects_bad_arguments():
    lib = cls.load_library()
    args_ok = dict(Bt=2, H=4, P=64, S=128, G=2, dt=cls.SSD_BF16)

    def call(h=FAKE, x=FAKE, dtp=FAKE, A=FAKE, B=FAKE, C=FAKE, y=FAKE, **kw):
        a = dict(args_ok)
        a.update(kw)
        return lib.ssd_step(h, x, dtp, A, B, C, None, a["Bt"], a["H"], a["P"], a["S"], a["G"], a["dt"], y,
                            None)

    assert call(h=None) == -1
    assert call(y=None) == -1
    assert call(C=None) == -1
    assert call(dt=5) == -3
    assert call(Bt=0) == -2
    assert call(P=-1) == -2
    assert call(H=3, G=2) == -2
    assert call(S=96) == -8
    assert call(S=512) == -8
    assert call(S=2) == -8
    assert call(h=ctypes.c_void_p(0x10008)) == -5
    assert call(x=ctypes.c_void_p(0x10001)) == -5


def test_linear_scan_three_pass_rejects_bad_arguments():
    lib = cls.load_library()
    ws = lib.linear_scan_three_pass_workspace_size(4, 100)
    assert ws >= 4 * 100 * 4
    assert lib.linear_scan_three_pass_workspace_size(0, 100) == 0
    assert lib.linear_scan_three_pass(None, FAKE, FAKE, 4, 100, FAKE, ws, None) == -1
    assert lib.linear_scan_three_pass(FAKE, FAKE, FAKE, 4, 0, FAKE, ws, None) == -2
    assert lib.linear_scan_three_pass(FAKE, FAKE, ctypes.c_void_p(0x10004), 4, 100, FAKE, ws, None) == -5
    assert lib.linear_scan_three_pass(FAKE, FAKE, FAKE, 4, 100, FAKE, ws - 1, None) == -6


def test_ssd_autotune_rejects_bad_arguments():
    """Validation happens on the host before any launch: missing outputs of
    the tuner, a repetition count out of range, and ssd_fwd's own checks."""
    lib = cls.load_library()
    n1, n2, n3, n4, ms = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_float()
    s3, pol = ctypes.c_int(), ctypes.c_int()

    def call(x=FAKE, y=FAKE, reps=3, out=True, Bt=1, T=32, ws_bytes=1 << 30):
        outs = (ctypes.byref(n1), ctypes.byref(n2), ctypes.byref(n3), ctypes.byref(n4), ctypes.byref(s3),
                ctypes.byref(pol), ctypes.byref(ms)) if out else (None,) * 7
        return lib.ssd_fwd_autotune(x, FAKE, FAKE, FAKE, FAKE, None, None, Bt, 64, 2, 16, 32, 1, T, cls.SSD_BF16,
                                    y, None, FAKE, ws_bytes, None, reps, *outs)

    assert call(out=False) == -1
    assert call(reps=0) == -2
    assert call(reps=1001) == -2
    assert call(x=None) == -1
    assert call(y=None) == -1
    assert call(Bt=0) == -2
    assert call(T=48) == -4
    assert call(ws_bytes=0) in (-6, -8)


def test_ssd_plan_query_on_host():
    """The plan ssd_fwd uses is host logic: the built-in heuristic splits the
    chains left over after whole rounds of 256 CUs when that shortens the
    last round; fp32 shapes and non-fused shapes report no plan; a forgotten
    table leaves the heuristic."""
    import torch
    cls.ssd_fwd_autotune_reset()
    # 4 x 80 chains: 64 left over after one round, cut into 4 segments
    # (192 pieces of 3 segments fit 512 aggregate slots twice: 2 pieces per segment);
    # a 256-token chunk runs as 128-token sub-chunks
    # (whole chains walk 64 sub-chunks: non-temporal x and y)
    assert cls.ssd_fwd_plan(4, 8192, 80, 64, 128, 1, 256) == {"nsegs": 4, "nsplit": 64, "agg_pieces": 2,
                                                              "sub_chunk": 128, "s3": "reduce",
                                                              "cache_policy": "nontemporal",
                                                              "source": "heuristic"}
    # 64 chains of 512 chunks: every chain cut into 4 (segments of 128 sub-chunks)
    assert cls.ssd_fwd_plan(1, 65536, 64, 64, 128, 8, 128) == {"nsegs": 4, "nsplit": 64, "agg_pieces": 2,
                                                               "sub_chunk": 128, "s3": "reduce",
                                                               "cache_policy": "nontemporal",
                                                               "source": "heuristic"}
    # 192 chains of 16 chunks: a split would not pay, whole chains, default policy
    assert cls.ssd_fwd_plan(8, 2048, 24, 64, 128, 1, 256) == {"nsegs": 1, "nsplit": 0, "agg_pieces": 0,
                                                              "sub_chunk": 128, "s3": None,
                                                              "cache_policy": "default",
                                                              "source": "heuristic"}
    # non-temporal instances exist for 128-token sub-chunks only
    assert cls.ssd_fwd_plan(1, 8192, 4, 64, 128, 1, 64)["cache_policy"] == "default"
    assert cls.ssd_fwd_plan(1, 1000, 4, 64, 128, 1, 32)["sub_chunk"] == 32
    assert cls.ssd_fwd_plan(1, 256, 2, 16, 16, 1, 32, torch.float32)["source"] == "none"
    assert cls.ssd_fwd_plan(1, 256, 2, 32, 32, 1, 32)["source"] == "none"  # head dim 32: per-head kernel
    with pytest.raises(cls.SSDError):
        cls.ssd_fwd_plan(1, 256, 3, 64, 128, 2, 32)
    lib = cls.load_library()
    n1, n2, n3, n4, s3 = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    pol = ctypes.c_int()
    assert lib.ssd_fwd_plan(1, 256, 2, 64, 128, 1, 32, 1, None, ctypes.byref(n1), ctypes.byref(n2),
                            ctypes.byref(n3), ctypes.byref(s3), ctypes.byref(pol)) == -1
    assert lib.ssd_fwd_plan(1, 256, 2, 64, 128, 1, 32, 1, ctypes.byref(n1), ctypes.byref(n2), ctypes.byref(n3),
                            ctypes.byref(n4), None, ctypes.byref(pol)) == -1
    assert lib.ssd_fwd_plan(1, 256, 2, 64, 128, 1, 32, 1, ctypes.byref(n1), ctypes.byref(n2), ctypes.byref(n3),
                            ctypes.byref(n4), ctypes.byref(s3), None) == -1


def test_linear_scan_typed_rejects_bad_arguments():
    lib = cls.load_library()

    def call(a=FAKE, h=FAKE, rows=2, L=100, din=cls.SSD_BF16, dout=cls.SSD_F32, ws=FAKE, ws_bytes=1 << 20):
        return lib.linear_scan_typed(a, FAKE, h, rows, L, din, dout, ws, ws_bytes, None)

    assert call(din=3) == -3
    assert call(dout=-1) == -3
    assert call(a=None) == -1
    assert call(h=None) == -1
    assert call(ws=None) == -1
    assert call(rows=0) == -2
    assert call(L=-1) == -2
    assert call(h=ctypes.c_void_p(0x10008)) == -5
    assert call(ws_bytes=0) == -6


TESTING_HEADER = os.path.join(ROOT, "include", "chunked_linear_scan_testing.h")


def test_testing_header_entry_points_are_exported():
    text = re.sub(r"/\*.*?\*/", "", open(TESTING_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof", "defined"})
    assert names == ["linear_scan_planned", "ssd_fwd_planned", "ssd_fwd_planned_workspace_size", "stream_mul_f32"]
    lib = ctypes.CDLL(cls.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_stream_kernel_rejects_bad_arguments():
    lib = cls.load_library()

    def call(a=FAKE, b=FAKE, h=FAKE, n=1024, vec=4, nt=1, grid=0):
        return lib.stream_mul_f32(a, b, h, n, vec, nt, grid, None)

    assert call(a=None) == -1
    assert call(h=ctypes.c_void_p(0x10004)) == -5
    for bad in (dict(n=0), dict(n=1022), dict(n=-4), dict(vec=3), dict(vec=16), dict(nt=2), dict(grid=-1),
                dict(grid=(1 << 23) + 1), dict(n=1 << 41)):
        assert call(**bad) == -2, bad


def test_no_process_wide_override_hooks():
    """Plans are passed per call (ssd_fwd_planned): the library exports no
    setter that would change what every later call does."""
    lib = ctypes.CDLL(cls.LIB_PATH)
    for name in ("cls_ssd_set_segments", "cls_ssd_set_split", "cls_ssd_set_agg_pieces", "cls_ssd_set_xcds",
                 "cls_ssd_force_path", "cls_ssd_profile", "cls_ssd_profile_read"):
        assert not hasattr(lib, name), name


def test_planned_call_validates_the_plan_on_host():
    lib = cls.load_library()
    shape = (1, 65536, 8, 64, 128, 1, 128, cls.SSD_BF16)

    def call(plan, events=None, ws_bytes=1 << 34):
        return lib.ssd_fwd_planned(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, *shape, FAKE, None, FAKE, ws_bytes,
                                   None, ctypes.byref(plan) if plan is not None else None, events)

    for bad in (cls.plan_request(nsegs=65), cls.PlanRequest(3, 0, 0, 0, 0, 0, 0), cls.PlanRequest(0, 3, 0, 0, 0, 0, 0),
                cls.PlanRequest(0, 0, -1, 0, 0, 0, 0), cls.PlanRequest(0, 0, 2, -1, 0, 0, 0),
                cls.PlanRequest(0, 0, 0, 0, 0, 65, 0), cls.PlanRequest(0, 0, 0, 0, 0, 0, 7),
                cls.PlanRequest(0, 0, 0, 0, 0, 0, 0, 0, 3), cls.PlanRequest(0, 0, 0, 0, 0, 0, 0, 0, -1),
                cls.PlanRequest(0, 0, 0, 0, 0, 0, 0, 0, 0, 3), cls.PlanRequest(0, 0, 0, 0, 0, 0, 0, 0, 0, -1)):
        assert call(bad) == -2
        assert lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(bad)) == 0
    # a forced plan's workspace: at least ssd_fwd's, more when it splits finer than the tuner would
    base = lib.ssd_fwd_workspace_size(*shape)
    fine = lib.ssd_fwd_planned_workspace_size(*shape, ctypes.byref(cls.plan_request(nsegs=64, agg_pieces=1000)))
    assert base > 0 and fine > base
    assert call(cls.plan_request(nsegs=64, agg_pieces=1000), ws_bytes=base) == -6
    # four events or none
    ev = (ctypes.c_void_p * 4)(0x10, 0x20, None, 0x40)
    assert call(cls.plan_request(), events=ev) == -1


def test_workspace_cache_is_keyed_by_device_and_stream():
    """Two streams of one device get two workspaces (calls sharing one must be
    stream-ordered); growing one stream's buffer leaves the other's alone."""
    import torch
    made = []

    def alloc(device, size):
        made.append((device, size))
        return torch.zeros(size, dtype=torch.uint8)

    c = cls._Workspace(alloc)
    a1 = c.get("cuda:0", 111, 5000)
    assert c.get("cuda:0", 111, 100) is a1          # same stream, fits: reused
    b1 = c.get("cuda:0", 222, 5000)
    assert b1 is not a1                              # another stream: its own buffer
    d1 = c.get("cuda:1", 111, 5000)
    assert d1 is not a1                              # another device: its own buffer
    a2 = c.get("cuda:0", 111, 9000)
    assert a2 is not a1 and a2.numel() == 9000       # grows
    assert c.get("cuda:0", 222, 10) is b1            # the other stream's buffer is untouched
    assert len(made) == 4
    # the error-word reader sums and clears the words of the given buffers
    a2[:4].view(torch.int32).fill_(3)
    b1[:4].view(torch.int32).fill_(2)
    assert cls.workspace_errors([a2, b1]) == 5
    assert cls.workspace_errors([a2, b1]) == 0
