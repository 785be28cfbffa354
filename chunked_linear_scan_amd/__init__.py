"""Python binding of the gfx950 ``libchunked_linear_scan.so`` C ABI.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs and the workspace are allocated with torch on the device,
and the C entry points of ``include/chunked_linear_scan.h`` are called with
raw pointers on torch's current stream.  Every step of the computation runs in
the library's HIP kernels; there is no fallback path.  If the shared library
has not been built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libchunked_linear_scan.so")

SSD_OK = 0
SSD_F32 = 0
SSD_BF16 = 1
SSD_F16 = 2
_DTYPE_CODE = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}           # SSD operands
_SCAN_CODE = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16, torch.float16: SSD_F16}  # scan elements

_lib = None
_lib_lock = threading.Lock()


class PlanRequest(ctypes.Structure):
    """``ssd_plan_request`` of include/chunked_linear_scan_testing.h."""
    _fields_ = [("path", ctypes.c_int32), ("s3", ctypes.c_int32), ("nsegs", ctypes.c_int64),
                ("nsplit", ctypes.c_int64), ("agg_pieces", ctypes.c_int64), ("xcds", ctypes.c_int32),
                ("sub_chunk", ctypes.c_int32), ("stress_seed", ctypes.c_uint32), ("cache_policy", ctypes.c_int32),
                ("c_source", ctypes.c_int32)]


PATH = {"auto": 0, "chunk": 1, "fused": 2}
S3 = {"auto": 0, "reduce": 1, "lookback": 2}
_S3_NAME = {0: None, 1: "reduce", 2: "lookback"}
CACHE = {"auto": 0, "default": 1, "nontemporal": 2}
_CACHE_NAME = {0: None, 1: "default", 2: "nontemporal"}
CSRC = {"auto": 0, "copy": 1, "rows": 2}  # where the fused state term reads C


class SSDError(RuntimeError):
    """A negative status returned by the library."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({strerror(status)})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and return the shared library; raise if it is missing."""
    global _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                " (there is no non-HIP fallback)")
        lib = ctypes.CDLL(path)
        i64, sz, vp, fp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p
        lib.ssd_strerror.argtypes = [ctypes.c_int]
        lib.ssd_strerror.restype = ctypes.c_char_p
        lib.linear_scan_workspace_size.argtypes = [i64, i64]
        lib.linear_scan_workspace_size.restype = sz
        lib.linear_scan.argtypes = [fp, fp, fp, i64, i64, vp, sz, vp]
        lib.linear_scan.restype = ctypes.c_int
        lib.linear_scan_typed.argtypes = [vp, vp, vp, i64, i64, ctypes.c_int, ctypes.c_int, vp, sz, vp]
        lib.linear_scan_typed.restype = ctypes.c_int
        lib.linear_scan_hillis_steele.argtypes = [fp, fp, fp, i64, i64, vp, sz, vp]
        lib.linear_scan_hillis_steele.restype = ctypes.c_int
        lib.ssd_fwd_workspace_size.argtypes = [i64] * 7 + [ctypes.c_int]
        lib.ssd_fwd_workspace_size.restype = sz
        lib.ssd_fwd.argtypes = [vp, fp, fp, vp, vp, fp, fp] + [i64] * 7 + [ctypes.c_int, vp, fp, vp, sz, vp]
        lib.ssd_fwd.restype = ctypes.c_int
        lib.linear_scan_three_pass_workspace_size.argtypes = [i64, i64]
        lib.linear_scan_three_pass_workspace_size.restype = sz
        lib.linear_scan_three_pass.argtypes = [fp, fp, fp, i64, i64, vp, sz, vp]
        lib.linear_scan_three_pass.restype = ctypes.c_int
        lib.ssd_step.argtypes = [fp, vp, fp, fp, vp, vp, fp] + [i64] * 5 + [ctypes.c_int, vp, vp]
        lib.ssd_step.restype = ctypes.c_int
        pi64 = ctypes.POINTER(ctypes.c_int64)
        pint = ctypes.POINTER(ctypes.c_int)
        lib.ssd_fwd_autotune.argtypes = lib.ssd_fwd.argtypes + [ctypes.c_int, pi64, pi64, pi64, pi64, pint, pint,
                                                                ctypes.POINTER(ctypes.c_float)]
        lib.ssd_fwd_autotune.restype = ctypes.c_int
        lib.ssd_fwd_plan.argtypes = [i64] * 7 + [ctypes.c_int, pi64, pi64, pi64, pi64, pint, pint]
        lib.ssd_fwd_plan.restype = ctypes.c_int
        lib.ssd_fwd_autotune_reset.argtypes = []
        lib.ssd_fwd_autotune_reset.restype = None
        lib.ssd_fwd_planned.argtypes = lib.ssd_fwd.argtypes + [ctypes.POINTER(PlanRequest), vp]
        lib.ssd_fwd_planned.restype = ctypes.c_int
        lib.ssd_fwd_planned_workspace_size.argtypes = [i64] * 7 + [ctypes.c_int, ctypes.POINTER(PlanRequest)]
        lib.ssd_fwd_planned_workspace_size.restype = sz
        lib.stream_mul_f32.argtypes = [fp, fp, fp, i64, ctypes.c_int, ctypes.c_int, i64, vp]
        lib.stream_mul_f32.restype = ctypes.c_int
        lib.linear_scan_planned.argtypes = [fp, fp, fp, i64, i64, i64, ctypes.c_uint32, vp, sz, vp]
        lib.linear_scan_planned.restype = ctypes.c_int
        lib.linear_scan_autotune.argtypes = [fp, fp, fp, i64, i64, vp, sz, vp, ctypes.c_int, pi64,
                                             ctypes.POINTER(ctypes.c_float)]
        lib.linear_scan_autotune.restype = ctypes.c_int
        lib.linear_scan_plan.argtypes = [i64, i64, pi64]
        lib.linear_scan_plan.restype = ctypes.c_int
        lib.linear_scan_autotune_reset.argtypes = []
        lib.linear_scan_autotune_reset.restype = None
        _lib = lib
        return lib


def strerror(status: int) -> str:
    try:
        return load_library().ssd_strerror(int(status)).decode()
    except RuntimeError:
        return "library not loaded"


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _stream_key(device: torch.device) -> int:
    return int(torch.cuda.current_stream(device).cuda_stream)


def workspace_errors(workspaces=None, reset: bool = True) -> int:
    """Sum of the error words of the given workspaces (default: every
    workspace the binding has cached), after waiting for their devices.

    The kernels' bounded waits (the scans' look-back, the SSD kernels'
    hand-offs between wave roles) never hang: when one gives up it adds 1 to
    the 32-bit word at the start of its workspace and carries on, so its
    outputs are then wrong.  Nonzero means such a call happened since the
    word was last cleared; ``reset`` clears it."""
    if workspaces is None:
        workspaces = [b for _, b in _scan_ws.buffers()] + [b for _, b in _ssd_ws.buffers()]
    total = 0
    for ws in workspaces:
        if ws.device.type == "cuda":
            torch.cuda.synchronize(ws.device)
        word = ws[:4].view(torch.int32)
        v = int(word.item())
        if v and reset:
            word.zero_()
        total += v
    return total


class _Workspace:
    """Workspaces cached per (device, stream).  Calls that share a workspace
    must be ordered on one stream (the library's contract), so each stream of
    each device gets its own; it is allocated while that stream is current,
    so torch's allocator orders its reuse after the work queued on it.  It is
    zero-filled when (re)allocated; the kernels leave their flags and
    counters at zero, so it is reused as is."""

    def __init__(self, alloc=None):
        self._buf = {}
        self._lock = threading.Lock()
        self._alloc = alloc or (lambda device, size: torch.zeros(size, dtype=torch.uint8, device=device))

    def get(self, device, stream_key, nbytes: int) -> torch.Tensor:
        key = (str(device), stream_key)
        with self._lock:
            buf = self._buf.get(key)
            if buf is None or buf.numel() < nbytes:
                buf = self._alloc(device, max(nbytes, 4096))
                self._buf[key] = buf
            return buf

    def buffers(self):
        with self._lock:
            return list(self._buf.items())


_scan_ws = _Workspace()
_ssd_ws = _Workspace()


def _check_cuda(name, t, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def linear_scan(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None, out_dtype: torch.dtype | None = None) -> torch.Tensor:
    """h[r, t] = a[r, t] h[r, t-1] + b[r, t] with h[r, -1] = 0, [rows, L].

    a and b are both fp32, both bf16 or both fp16; h is fp32 unless out (or
    out_dtype) is bf16 or fp16.  The scan runs in fp32 either way."""
    lib = load_library()
    if a.dtype not in _SCAN_CODE:
        raise TypeError("a must be float32, bfloat16 or float16")
    _check_cuda("a", a, a.dtype)
    if a.dim() != 2:
        raise ValueError("a must be [rows, L]")
    _check_cuda("b", b, a.dtype, a.shape)
    rows, length = a.shape
    if out is None:
        h = torch.empty(a.shape, dtype=out_dtype or torch.float32, device=a.device)
    else:
        h = out
    if h.dtype not in _SCAN_CODE:
        raise TypeError("out must be float32, bfloat16 or float16")
    _check_cuda("out", h, h.dtype, a.shape)
    need = lib.linear_scan_workspace_size(rows, length)
    if need == 0:
        raise SSDError(-2, "linear_scan_workspace_size")
    ws = _scan_ws.get(a.device, _stream_key(a.device), need) if workspace is None else workspace
    if a.dtype == torch.float32 and h.dtype == torch.float32:
        st = lib.linear_scan(_ptr(a), _ptr(b), _ptr(h), rows, length, _ptr(ws), ws.numel(),
                             _stream_handle(a.device))
    else:
        st = lib.linear_scan_typed(_ptr(a), _ptr(b), _ptr(h), rows, length, _SCAN_CODE[a.dtype],
                                   _SCAN_CODE[h.dtype], _ptr(ws), ws.numel(), _stream_handle(a.device))
    if st != SSD_OK:
        raise SSDError(st, "linear_scan")
    return h


def _scan_f32_args(lib, a, b, out, workspace):
    _check_cuda("a", a, torch.float32)
    if a.dim() != 2:
        raise ValueError("a must be [rows, L]")
    _check_cuda("b", b, torch.float32, a.shape)
    rows, length = a.shape
    h = torch.empty_like(a) if out is None else out
    _check_cuda("out", h, torch.float32, a.shape)
    need = lib.linear_scan_workspace_size(rows, length)
    if need == 0:
        raise SSDError(-2, "linear_scan_workspace_size")
    ws = _scan_ws.get(a.device, _stream_key(a.device), need) if workspace is None else workspace
    return rows, length, h, ws


def linear_scan_planned(a: torch.Tensor, b: torch.Tensor, tile: int = 0, out: torch.Tensor | None = None,
                        workspace: torch.Tensor | None = None, stress_seed: int = 0) -> torch.Tensor:
    """fp32 linear_scan with an explicit tile size (4096, 8192 or 16384
    elements; 0: what linear_scan runs) and an optional look-back stress
    seed, ``linear_scan_planned`` of the testing header."""
    lib = load_library()
    rows, length, h, ws = _scan_f32_args(lib, a, b, out, workspace)
    st = lib.linear_scan_planned(_ptr(a), _ptr(b), _ptr(h), rows, length, int(tile), int(stress_seed), _ptr(ws),
                                 ws.numel(), _stream_handle(a.device))
    if st != SSD_OK:
        raise SSDError(st, "linear_scan_planned")
    return h


def linear_scan_autotune(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, reps: int = 10,
                         workspace: torch.Tensor | None = None):
    """Times the fp32 scan's tile sizes on these arguments and keeps the
    fastest for the shape (the built-in 8192 unless another is faster by more
    than the noise).  Returns (h, {"tile", "ms_per_call"}); h is what a later
    linear_scan of the shape returns."""
    lib = load_library()
    rows, length, h, ws = _scan_f32_args(lib, a, b, out, workspace)
    tile, ms = ctypes.c_int64(), ctypes.c_float()
    st = lib.linear_scan_autotune(_ptr(a), _ptr(b), _ptr(h), rows, length, _ptr(ws), ws.numel(),
                                  _stream_handle(a.device), int(reps), ctypes.byref(tile), ctypes.byref(ms))
    if st != SSD_OK:
        raise SSDError(st, "linear_scan_autotune")
    return h, {"tile": tile.value, "ms_per_call": ms.value}


def linear_scan_plan(rows: int, length: int) -> dict:
    """The tile an fp32 linear_scan of this shape runs on the current device:
    {"tile", "source": "tuned" | "built-in"}.  Launches nothing."""
    lib = load_library()
    tile = ctypes.c_int64()
    st = lib.linear_scan_plan(int(rows), int(length), ctypes.byref(tile))
    if st < 0:
        raise SSDError(st, "linear_scan_plan")
    return {"tile": tile.value, "source": "tuned" if st == 1 else "built-in"}


def linear_scan_autotune_reset():
    """Forgets every tuned scan tile."""
    load_library().linear_scan_autotune_reset()


def _ssd_fwd_args(lib, x, dt, A, B, C, D, h0, chunk, want_final_state, out, workspace, plan=None):
    """Checks ssd_fwd's tensors and returns the C call's argument list."""
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16")
    _check_cuda("x", x, x.dtype)
    if x.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim]")
    Bt, L, H, P = x.shape
    _check_cuda("B", B, x.dtype)
    if B.dim() != 4 or B.shape[0] != Bt or B.shape[1] != L:
        raise ValueError("B must be [batch, seqlen, ngroups, dstate]")
    G, S = B.shape[2], B.shape[3]
    _check_cuda("C", C, x.dtype, B.shape)
    _check_cuda("dt", dt, torch.float32, (Bt, L, H))
    _check_cuda("A", A, torch.float32, (H,))
    if D is not None:
        _check_cuda("D", D, torch.float32, (H,))
    if h0 is not None:
        _check_cuda("h0", h0, torch.float32, (Bt, H, P, S))
    y = torch.empty_like(x) if out is None else out
    _check_cuda("out", y, x.dtype, x.shape)
    hf = torch.empty((Bt, H, P, S), dtype=torch.float32, device=x.device) if want_final_state else None
    code = _DTYPE_CODE[x.dtype]
    if plan is None:
        need = lib.ssd_fwd_workspace_size(Bt, L, H, P, S, G, chunk, code)
    else:
        need = lib.ssd_fwd_planned_workspace_size(Bt, L, H, P, S, G, chunk, code, ctypes.byref(plan))
    ws = workspace
    if ws is None:
        ws = _ssd_ws.get(x.device, _stream_key(x.device), max(need, 1))
    args = [_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(h0), Bt, L, H, P, S, G, int(chunk), code,
            _ptr(y), _ptr(hf), _ptr(ws), ws.numel(), _stream_handle(x.device)]
    return args, y, hf


def ssd_fwd(x, dt, A, B, C, D=None, h0=None, chunk: int = 256, want_final_state: bool = True,
            out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Mamba-2 SSD chunked forward pass.  Returns (y, h_final or None).

    x [Bt,L,H,P] and B, C [Bt,L,G,S] in fp32 or bf16 (same dtype); dt
    [Bt,L,H], A [H], D [H] (optional) and h0 [Bt,H,P,S] (optional) in fp32.
    """
    lib = load_library()
    args, y, hf = _ssd_fwd_args(lib, x, dt, A, B, C, D, h0, chunk, want_final_state, out, workspace)
    st = lib.ssd_fwd(*args)
    if st != SSD_OK:
        raise SSDError(st, "ssd_fwd")
    return y, hf


def plan_request(path="auto", s3="auto", nsegs=0, nsplit=0, agg_pieces=0, xcds=0, sub_chunk=0,
                 stress_seed=0, cache_policy="auto", c_source="auto") -> PlanRequest:
    """An explicit plan for ``ssd_fwd_planned`` (see the testing header)."""
    return PlanRequest(PATH[path], S3[s3 or "auto"], int(nsegs), int(nsplit), int(agg_pieces), int(xcds),
                       int(sub_chunk), int(stress_seed), CACHE[cache_policy or "auto"],
                       CSRC[c_source or "auto"])


def ssd_fwd_planned(x, dt, A, B, C, D=None, h0=None, chunk: int = 256, plan: PlanRequest | None = None,
                    events=None, want_final_state: bool = True, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None):
    """``ssd_fwd`` with an explicit plan (tests and measurement).  ``events``:
    None, or four torch.cuda.Event(enable_timing=True) recorded on the current
    stream before the first launch, after the CB pass, after the aggregate
    launch and after the output launch."""
    lib = load_library()
    plan = plan if plan is not None else plan_request()
    args, y, hf = _ssd_fwd_args(lib, x, dt, A, B, C, D, h0, chunk, want_final_state, out, workspace, plan)
    evp = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events must be four torch.cuda.Event")
        stream = torch.cuda.current_stream(x.device)
        for e in events:
            if e.cuda_event == 0:  # torch creates the event at its first record
                e.record(stream)
        evp = (ctypes.c_void_p * 4)(*[e.cuda_event for e in events])
    st = lib.ssd_fwd_planned(*args, ctypes.byref(plan), evp)
    if st != SSD_OK:
        raise SSDError(st, "ssd_fwd_planned")
    return y, hf


def ssd_fwd_autotune(x, dt, A, B, C, D=None, h0=None, chunk: int = 256, reps: int = 5,
                     want_final_state: bool = True, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None):
    """Times ssd_fwd's candidate plans on these inputs against the built-in
    heuristic's and keeps the fastest for this shape (later ssd_fwd calls use
    it).  Blocks until done.  Returns (y, h_final or None, {"nsegs", "nsplit",
    "agg_pieces", "sub_chunk", "s3", "cache_policy", "ms_per_call"}); y and
    h_final are the chosen plan's result.  nsegs == 0: nothing to tune."""
    lib = load_library()
    args, y, hf = _ssd_fwd_args(lib, x, dt, A, B, C, D, h0, chunk, want_final_state, out, workspace)
    nsegs, nsplit, pieces, sub, ms = (ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(),
                                      ctypes.c_float())
    s3, pol = ctypes.c_int(), ctypes.c_int()
    st = lib.ssd_fwd_autotune(*args, int(reps), ctypes.byref(nsegs), ctypes.byref(nsplit), ctypes.byref(pieces),
                              ctypes.byref(sub), ctypes.byref(s3), ctypes.byref(pol), ctypes.byref(ms))
    if st != SSD_OK:
        raise SSDError(st, "ssd_fwd_autotune")
    return y, hf, {"nsegs": nsegs.value, "nsplit": nsplit.value, "agg_pieces": pieces.value,
                   "sub_chunk": sub.value, "s3": _S3_NAME[s3.value], "cache_policy": _CACHE_NAME[pol.value],
                   "ms_per_call": ms.value}


def ssd_fwd_plan(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype=torch.bfloat16):
    """The plan ssd_fwd uses for a shape: {"nsegs", "nsplit", "agg_pieces",
    "sub_chunk", "s3", "cache_policy", "source": "tuned" | "heuristic" |
    "none"}.  Launches nothing."""
    lib = load_library()
    nsegs, nsplit, pieces, sub = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    s3, pol = ctypes.c_int(), ctypes.c_int()
    st = lib.ssd_fwd_plan(batch, seqlen, nheads, headdim, dstate, ngroups, int(chunk), _DTYPE_CODE[dtype],
                          ctypes.byref(nsegs), ctypes.byref(nsplit), ctypes.byref(pieces), ctypes.byref(sub),
                          ctypes.byref(s3), ctypes.byref(pol))
    if st < 0:
        raise SSDError(st, "ssd_fwd_plan")
    return {"nsegs": nsegs.value, "nsplit": nsplit.value, "agg_pieces": pieces.value, "sub_chunk": sub.value,
            "s3": _S3_NAME[s3.value], "cache_policy": _CACHE_NAME[pol.value],
            "source": {0: "heuristic", 1: "tuned", 2: "none"}[st]}


def ssd_fwd_autotune_reset():
    """Forget every tuned plan (ssd_fwd falls back to its built-in heuristic)."""
    load_library().ssd_fwd_autotune_reset()


def linear_scan_hillis_steele(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The same scan (fp32) with a register-resident Hillis-Steele scan inside
    each tile (the work-inefficient comparison kernel)."""
    lib = load_library()
    _check_cuda("a", a, torch.float32)
    if a.dim() != 2:
        raise ValueError("a must be [rows, L]")
    _check_cuda("b", b, torch.float32, a.shape)
    rows, length = a.shape
    h = torch.empty_like(a) if out is None else out
    _check_cuda("out", h, torch.float32, a.shape)
    need = lib.linear_scan_workspace_size(rows, length)
    if need == 0:
        raise SSDError(-2, "linear_scan_workspace_size")
    ws = _scan_ws.get(a.device, _stream_key(a.device), need) if workspace is None else workspace
    st = lib.linear_scan_hillis_steele(_ptr(a), _ptr(b), _ptr(h), rows, length, _ptr(ws), ws.numel(),
                                       _stream_handle(a.device))
    if st != SSD_OK:
        raise SSDError(st, "linear_scan_hillis_steele")
    return h


def stream_mul(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, vec: int = 4, nt: bool = True,
               grid_blocks: int = 0) -> torch.Tensor:
    """h = a * b elementwise over contiguous fp32 tensors (``stream_mul_f32``
    of the testing header): the linear scan's traffic without the scan, the
    measured ceiling of a three-stream kernel."""
    lib = load_library()
    _check_cuda("a", a, torch.float32)
    _check_cuda("b", b, torch.float32, a.shape)
    h = torch.empty_like(a) if out is None else out
    _check_cuda("out", h, torch.float32, a.shape)
    st = lib.stream_mul_f32(_ptr(a), _ptr(b), _ptr(h), a.numel(), int(vec), 1 if nt else 0, int(grid_blocks),
                            _stream_handle(a.device))
    if st != SSD_OK:
        raise SSDError(st, "stream_mul_f32")
    return h


def linear_scan_three_pass(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """h[r, t] = a[r, t] h[r, t-1] + b[r, t] by the three-pass (block scan, spine,
    apply) kernels: the independent cross-check of ``linear_scan``."""
    lib = load_library()
    _check_cuda("a", a, torch.float32)
    if a.dim() != 2:
        raise ValueError("a must be [rows, length]")
    _check_cuda("b", b, torch.float32, a.shape)
    rows, L = a.shape
    h = torch.empty_like(a) if out is None else out
    _check_cuda("out", h, torch.float32, a.shape)
    need = lib.linear_scan_three_pass_workspace_size(rows, L)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=a.device)
    st = lib.linear_scan_three_pass(_ptr(a), _ptr(b), _ptr(h), rows, L, _ptr(ws), ws.numel(),
                                    _stream_handle(a.device))
    if st != SSD_OK:
        raise SSDError(st, "linear_scan_three_pass")
    return h


def ssd_step(h, x, dt, A, B, C, D=None, out: torch.Tensor | None = None):
    """One decode token: updates the state h [Bt,H,P,S] (fp32) in place and
    returns y [Bt,H,P].

    x [Bt,H,P] and B, C [Bt,G,S] in fp32 or bf16 (same dtype); dt [Bt,H],
    A [H] and D [H] (optional) in fp32.
    """
    lib = load_library()
    if x.dtype not in _DTYPE_CODE:
        raise TypeError("x must be float32 or bfloat16")
    _check_cuda("x", x, x.dtype)
    if x.dim() != 3:
        raise ValueError("x must be [batch, nheads, headdim]")
    Bt, H, P = x.shape
    _check_cuda("B", B, x.dtype)
    if B.dim() != 3 or B.shape[0] != Bt:
        raise ValueError("B must be [batch, ngroups, dstate]")
    G, S = B.shape[1], B.shape[2]
    _check_cuda("C", C, x.dtype, B.shape)
    _check_cuda("h", h, torch.float32, (Bt, H, P, S))
    _check_cuda("dt", dt, torch.float32, (Bt, H))
    _check_cuda("A", A, torch.float32, (H,))
    if D is not None:
        _check_cuda("D", D, torch.float32, (H,))
    y = torch.empty_like(x) if out is None else out
    _check_cuda("out", y, x.dtype, x.shape)
    st = lib.ssd_step(_ptr(h), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), Bt, H, P, S, G,
                      _DTYPE_CODE[x.dtype], _ptr(y), _stream_handle(x.device))
    if st != SSD_OK:
        raise SSDError(st, "ssd_step")
    return y


__all__ = ["linear_scan", "linear_scan_hillis_steele", "linear_scan_three_pass", "ssd_fwd", "ssd_fwd_autotune", "ssd_fwd_plan",
           "ssd_fwd_autotune_reset", "ssd_fwd_planned", "plan_request", "ssd_step", "load_library", "strerror",
           "workspace_errors", "SSDError", "LIB_PATH", "SSD_F32", "SSD_BF16", "SSD_F16"]
