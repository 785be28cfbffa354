"""Throughput benchmark of the SSD forward pass and the linear scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ssd_large]

One step is one ``ssd_fwd`` call over one batch of the named workload, with
inputs already resident in HBM: the CB pass (C B^T per (batch, chunk, group)
and the token-contiguous copy of B) and the fused kernel (segment sums,
intra-chunk products, chunk states, the inter-chunk recurrence and outputs).
K steps are timed with HIP events on the launch stream, bracketed by device
synchronisation; during the same steps the library records events around
each of its two kernels, which gives the fused kernel's own time for the
roofline.  Input and output buffers rotate over enough copies that the
footprint exceeds 1 GiB, so the 256 MB Infinity Cache cannot serve repeated
steps.  The linear scan (one kernel) is timed the same way in its own loop and
reported in the ``linear_scan`` object of the same JSON line (with its bf16
forms and a plain elementwise kernel of the same traffic beside it), and so are
the three-pass scan (``linear_scan_three_pass``) and one decode token
(``ssd_step``).  The ``autotune`` object compares the plan ssd_fwd_autotune
keeps for the workload with the built-in heuristic's, timed back to back.

Other modes: ``--scan-ceiling-sweep`` (linear_scan against torch.mul over row
lengths), ``--copy-probe`` / ``--record-traffic`` (the HBM traffic counters),
``--no-autotune`` (counter and trace runs), ``--no-scan``, ``--workload``.

The CPU baseline is the float64 oracle, unmodified, run on a bounded sample
of the same workload (a few whole (batch, head) sequences, one per worker
process) and scaled to the metric's unit.

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
FP32_PEAK_TFLOPS = 157.3
METRIC = "SSD fwd tokens/sec (B·L) + % of HBM/MFMA roofline; linear-scan GB/s"


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def ssd_alg_bytes(inp, shape):
    """Compulsory HBM bytes of one forward pass: every input read once and
    every output written once (x, dt, A, B, C, D, optional h0, y, h_final)."""
    b = sum(_nbytes(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "h0"))
    b += _nbytes(inp["x"])                                            # y
    b += shape.batch * shape.nheads * shape.headdim * shape.dstate * 4  # h_final
    return b


def ssd_alg_flops(shape):
    """Causal-triangle MFMA flops: C B^T once per (batch, chunk, group) plus,
    per (batch, chunk, head), the masked product, the chunk state and C h^T."""
    T = shape.chunk
    nc = shape.nchunks
    cb = shape.batch * nc * shape.ngroups * T * (T + 1) * shape.dstate
    per_head = T * (T + 1) * shape.headdim + 4 * T * shape.dstate * shape.headdim
    return cb + shape.batch * nc * shape.nheads * per_head


def code_text(src):
    """Source text without comments and with whitespace runs collapsed: what
    the compiler sees, so an edit to a comment keeps a kernel's digest."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_digest(names, read=None):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunked_linear_scan_amd", "csrc")
    for n in sorted(names):
        if read is None:
            with open(os.path.join(csrc, n), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(n)
        h.update(n.encode())
        h.update(code_text(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, sources, launches_per_step=1):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, only if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            db = json.load(f)
    except (OSError, ValueError):
        return None
    rec = db.get(kernel_key)
    if not rec or rec.get("source_digest") != source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


SSD_SOURCES = ["ssd_fused.hpp", "ssd_fused.hip", "common.hpp", "ssd_kernels.hpp"]
SCAN_SOURCES = ["linear_scan.hip", "common.hpp"]
STEP_SOURCES = ["ssd_step.hip", "common.hpp"]


def record_traffic(fetch_csv, write_csv, workload):
    """Write profiles/traffic.json from two rocprofv3 --pmc runs of this script
    with --copy-probe (one with FETCH_SIZE, one with WRITE_SIZE).  Each counter
    is scaled by what it reads for the 1 GiB device copies of --copy-probe
    (copyBuffer dispatches of 131072 workgroups), per dispatch of each kernel."""
    import csv
    import statistics

    def read(path, name):
        d = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == name:
                    d.setdefault((r["Kernel_Name"], r["Grid_Size"]), []).append(float(r["Counter_Value"]))
        return d

    fe, wr = read(fetch_csv, "FETCH_SIZE"), read(write_csv, "WRITE_SIZE")
    copy_f = [v for (k, g), vs in fe.items() if "copyBuffer" in k and g == "131072" for v in vs]
    copy_w = [v for (k, g), vs in wr.items() if "copyBuffer" in k and g == "131072" for v in vs]
    if not copy_f or not copy_w:
        raise SystemExit("no 1 GiB copy dispatches in the counter files (run bench.py with --copy-probe)")
    sf = 1048576.0 / statistics.mean(copy_f)  # counters read KiB
    sw = 1048576.0 / statistics.mean(copy_w)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = {}
    if os.path.exists(path):
        with open(path) as f:
            db = json.load(f)
    for key, srcs, pat in [("ssd_fused_kernel:" + workload, SSD_SOURCES, "ssd_fused_kernel<"),
                           ("ssd_fused_agg_kernel:" + workload, SSD_SOURCES, "ssd_fused_agg_kernel<"),
                           ("linear_scan:scan", SCAN_SOURCES, "linear_scan_kernel<false, float, float>"),
                           ("ssd_step:decode_large", STEP_SOURCES, "ssd_step_kernel")]:
        f = [v for (k, g), vs in fe.items() if pat in k for v in vs]
        w = [v for (k, g), vs in wr.items() if pat in k for v in vs]
        if not f or not w:
            continue
        fb = statistics.mean(f) * sf * 1024
        wb = statistics.mean(w) * sw * 1024
        db[key] = {"source_digest": source_digest(srcs), "hbm_bytes_per_launch": round(fb + wb),
                   "fetch_bytes": round(fb), "write_bytes": round(wb), "dispatches": len(f),
                   "scale_fetch": round(sf, 4), "scale_write": round(sw, 4)}
        print(key, db[key])
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)


def time_loop(fn, nsets, steps, warmup, stream, before_timed=None):
    import torch
    for i in range(warmup):
        fn(i % nsets)
    torch.cuda.synchronize()
    if before_timed is not None:
        before_timed()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i % nsets)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3 / steps  # seconds per step


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample, one (batch, head) per process
# ---------------------------------------------------------------------------
def _oracle_ssd_job(args):
    import numpy as np
    from oracle import ssd as ossd
    x, dt, A, B, C, D, h0 = args
    t0 = time.perf_counter()
    ossd.ssd_loop(x, dt, A, B, C, D, h0)
    return time.perf_counter() - t0


def cpu_baseline_ssd(inp, shape, budget_s=15.0):
    """Oracle wall time on as many whole (batch, head) sequences as fit the
    budget (all of them when they do), one sequence per job, one job per core."""
    import multiprocessing as mp
    import torch
    cores = len(os.sched_getaffinity(0))
    H, G = shape.nheads, shape.ngroups
    np64 = lambda t: None if t is None else t.to(dtype=torch.float64).numpy()

    def job(bb, h, n=None):
        g = h // (H // G)
        sl = slice(None) if n is None else slice(0, n)
        return (np64(inp["x"][bb:bb + 1, sl, h:h + 1]), np64(inp["dt"][bb:bb + 1, sl, h:h + 1]),
                np64(inp["A"][h:h + 1]), np64(inp["B"][bb:bb + 1, sl, g:g + 1]),
                np64(inp["C"][bb:bb + 1, sl, g:g + 1]), np64(inp["D"][h:h + 1]),
                None if inp["h0"] is None else np64(inp["h0"][bb:bb + 1, h:h + 1]))

    L = shape.seqlen
    probe = min(L, 1024)
    t_job = _oracle_ssd_job(job(0, 0, probe)) * L / probe
    total = shape.batch * H
    njobs = max(1, min(total, int(budget_s * cores / max(t_job, 1e-6))))
    # spread the sampled sequences over batches and heads
    pairs = [(k % shape.batch, (k * 7919) % H) for k in range(total)][:njobs] if njobs < total \
        else [(bb, h) for bb in range(shape.batch) for h in range(H)]
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    jobs = [job(bb, h) for bb, h in pairs]
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(cores) as pool:
        pool.map(_oracle_ssd_job, jobs, chunksize=1)
    wall = time.perf_counter() - t0
    tok_equiv = L * len(jobs) / H  # a token counts once all H heads of its row are done
    return {"value": tok_equiv / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(jobs)} of {total} whole (batch, head) sequences of {L} tokens, "
                      f"one per job on {cores} processes, wall {wall:.1f}s"}


def cpu_baseline_scan(inp):
    from oracle import scan as oscan
    t0 = time.perf_counter()
    oscan.scan_loop(inp["a"].numpy(), inp["b"].numpy())
    wall = time.perf_counter() - t0
    nbytes = 12 * inp["a"].numel()
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload ({tuple(inp['a'].shape)}), wall {wall:.2f}s"}


def bench_scan3(name, steps, warmup, scan_us):
    """The three-pass scan (block scan, spine, apply) on the same workload, and
    the traffic model it tests: seven arrays of traffic against the single
    pass's three, so at equal bus efficiency 7/3 of its time."""
    import torch
    import chunked_linear_scan_amd as cls
    from chunked_linear_scan_amd import workloads
    inp = workloads.scan_workload(name)
    rows, L = inp["a"].shape
    nbytes = 12 * rows * L
    nsets = max(1, math.ceil((1 << 30) / nbytes))
    dev = torch.device("cuda:0")
    lib = cls.load_library()
    sets = [(inp["a"].to(dev), inp["b"].to(dev), torch.empty(rows, L, device=dev)) for _ in range(nsets)]
    ws = torch.empty(lib.linear_scan_three_pass_workspace_size(rows, L), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        a, b, h = sets[i]
        st = lib.linear_scan_three_pass(cls._ptr(a), cls._ptr(b), cls._ptr(h), rows, L, cls._ptr(ws), ws.numel(),
                                        cls._stream_handle(dev))
        if st != 0:
            raise RuntimeError(cls.strerror(st))

    t = time_loop(step, nsets, steps, warmup, stream)
    moved = 28 * rows * L
    return {"workload": f"{name}: {rows} rows x {L} fp32", "value": round(nbytes / t / 1e9, 1), "unit": "GB/s",
            "us_per_call": round(t * 1e6, 2), "moved_bytes": moved, "moved_gbs": round(moved / t / 1e9, 1),
            "moved_frac_of_peak": round(moved / t / 1e9 / HBM_PEAK_GBS, 4),
            "time_ratio_to_single_pass": round(t * 1e6 / scan_us, 3), "traffic_model_ratio": round(7 / 3, 3)}


def cpu_baseline_step(inp, nbytes):
    from oracle import ssd as ossd
    arrs = [inp[k].to(torch_f64()).numpy() for k in ("h", "x", "dt", "A", "B", "C", "D")]
    t0 = time.perf_counter()
    ossd.ssd_step(*arrs)
    wall = time.perf_counter() - t0
    return {"value": nbytes / wall / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload (one token, {tuple(inp['h'].shape)} state), wall {wall:.2f}s"}


def torch_f64():
    import torch
    return torch.float64


def bench_step(name, steps, warmup, want_cpu):
    """One decode token per call (ssd_step) over the named workload; the state
    is updated in place, so repeated calls keep decoding."""
    import torch
    import chunked_linear_scan_amd as cls
    from chunked_linear_scan_amd import workloads
    shape, _ = workloads.STEP_WORKLOADS[name]
    inp = workloads.step_workload(name)
    Bt, H, P, S, G = shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    esz = 2 if shape.dtype == "bf16" else 4
    nbytes = (2 * Bt * H * P * S * 4 + 2 * Bt * H * P * esz + Bt * H * 4 + 2 * Bt * G * S * esz + 2 * H * 4)
    nsets = max(1, math.ceil((1 << 30) / nbytes))
    dev = torch.device("cuda:0")
    sets = []
    for _ in range(nsets):
        d = {k: v.to(dev) for k, v in inp.items()}
        d["y"] = torch.empty_like(d["x"])
        sets.append(d)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i]
        cls.ssd_step(d["h"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], out=d["y"])

    t = time_loop(step, nsets, steps, warmup, stream)
    gbs = nbytes / t / 1e9
    res = {"workload": f"{name}: one decode token, batch {Bt}, {H} heads, P={P}, S={S}, {G} group(s), "
                       f"{shape.dtype}",
           "value": round(gbs, 1), "unit": "GB/s", "us_per_call": round(t * 1e6, 2), "nsets": nsets,
           "tokens_per_s": round(Bt / t, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes": nbytes,
                        "traffic": measured_traffic("ssd_step:" + name, STEP_SOURCES)}}
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline_step(inp, nbytes)
    return res


# ---------------------------------------------------------------------------
def bench_ssd(name, steps, warmup, want_cpu, want_autotune=True):
    import torch
    import chunked_linear_scan_amd as cls
    from chunked_linear_scan_amd import workloads
    shape, seed = workloads.SSD_WORKLOADS[name]
    inp = workloads.make_ssd_inputs(shape, seed)
    alg_bytes = ssd_alg_bytes(inp, shape)
    nsets = max(1, math.ceil((1 << 30) / alg_bytes))
    dev = torch.device("cuda:0")
    sets = []
    for _ in range(nsets):
        d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
        d["y"] = torch.empty_like(d["x"])
        d["hf"] = torch.empty(shape.batch, shape.nheads, shape.headdim, shape.dstate,
                              dtype=torch.float32, device=dev)
        sets.append(d)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        d = sets[i]
        cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=shape.chunk,
                    out=d["y"])

    lib = cls.load_library()
    import ctypes
    lib.cls_ssd_profile.argtypes = [ctypes.c_int]
    lib.cls_ssd_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double)] * 3 + [ctypes.POINTER(ctypes.c_int)]
    if lib.cls_ssd_profile(1) != 0:  # creates the events
        raise RuntimeError("could not create the profiling events")
    lib.cls_ssd_profile(0)
    # the timed steps run without the library's events (recording them costs a
    # few microseconds per call); a second, shorter loop records them for the
    # per-launch breakdown
    t = time_loop(step, nsets, steps, warmup, stream)
    time_loop(step, nsets, max(10, steps // 4), 2, stream, before_timed=lambda: lib.cls_ssd_profile(1))
    cb_ms, agg_ms, fu_ms, ncalls = ctypes.c_double(), ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    if lib.cls_ssd_profile_read(ctypes.byref(cb_ms), ctypes.byref(agg_ms), ctypes.byref(fu_ms),
                                ctypes.byref(ncalls)) != 0:
        raise RuntimeError("reading the profiling events failed")
    lib.cls_ssd_profile(0)
    n = max(ncalls.value, 1)
    t_fused = fu_ms.value / 1e3 / n if ncalls.value else None
    t_cb = cb_ms.value / 1e3 / n if ncalls.value else None
    t_agg = agg_ms.value / 1e3 / n if ncalls.value else None
    tokens = shape.batch * shape.seqlen
    flops = ssd_alg_flops(shape)
    t_kernel = t_fused if t_fused else t
    gbs = alg_bytes / t_kernel / 1e9
    tflops = flops / t_kernel / 1e12
    t_roof = max(alg_bytes / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    srcs = SSD_SOURCES
    res = {
        "t": t, "tokens_per_s": tokens / t, "alg_bytes": alg_bytes, "alg_flops": flops,
        "gbs": gbs, "tflops": tflops, "nsets": nsets,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("ssd_fused_kernel:" + name, srcs),
                     "aggregate_pass_traffic": measured_traffic("ssd_fused_agg_kernel:" + name, srcs),
                     "kernel": "ssd_fused_kernel (output launch)" if t_fused else "whole ssd_fwd call",
                     "kernel_us": round(t_kernel * 1e6, 2),
                     "cb_pass_us": None if t_cb is None else round(t_cb * 1e6, 2),
                     "aggregate_pass_us": None if t_agg is None else round(t_agg * 1e6, 2),
                     "fused_launches_frac": None if t_agg is None else
                     round(alg_bytes / (t_agg + t_kernel) / 1e9 / HBM_PEAK_GBS, 4),
                     "call_us": round(t * 1e6, 2),
                     "alg_bytes": alg_bytes, "alg_flops": flops,
                     "mfma_tflops": round(tflops, 1), "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                     "call_frac_of_roofline": round(t_roof / t, 4)},
        "shape": shape,
    }
    # The autotuner (ssd_fwd_autotune) on the same inputs: the plan it keeps
    # and ssd_fwd's time on that plan, beside the built-in heuristic's, which
    # is what the timed steps above ran.  The table is cleared afterwards.
    if want_autotune:
        heur = cls.ssd_fwd_plan(shape.batch, shape.seqlen, shape.nheads, shape.headdim, shape.dstate,
                                shape.ngroups, shape.chunk, inp["x"].dtype)
        d0 = sets[0]
        _, _, info = cls.ssd_fwd_autotune(d0["x"], d0["dt"], d0["A"], d0["B"], d0["C"], d0["D"], d0["h0"],
                                          chunk=shape.chunk, reps=10, out=d0["y"])
        t_tuned = time_loop(step, nsets, steps, warmup, stream)
        cls.ssd_fwd_autotune_reset()
        # the heuristic again, right after, so that both loops run in the same
        # state of the GPU (a later loop tends to run a little faster)
        t_heur = time_loop(step, nsets, steps, warmup, stream)
        res["autotune"] = {"plan": {"nsegs": info["nsegs"], "nsplit": info["nsplit"],
                                    "agg_pieces": info["agg_pieces"]},
                           "heuristic_plan": {"nsegs": heur["nsegs"], "nsplit": heur["nsplit"],
                                              "agg_pieces": heur["agg_pieces"]},
                           "us_per_call_tuned": round(t_tuned * 1e6, 2),
                           "us_per_call_heuristic": round(t_heur * 1e6, 2),
                           "speedup": round(t_heur / t_tuned, 3)}
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline_ssd(inp, shape)
    return res


def bench_scan(name, steps, warmup, want_cpu):
    import torch
    import chunked_linear_scan_amd as cls
    from chunked_linear_scan_amd import workloads
    inp = workloads.scan_workload(name)
    rows, L = inp["a"].shape
    nbytes = 12 * rows * L
    nsets = max(1, math.ceil((1 << 30) / nbytes))
    dev = torch.device("cuda:0")
    sets = [(inp["a"].to(dev), inp["b"].to(dev), torch.empty(rows, L, device=dev)) for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)
    ws = torch.zeros(cls.load_library().linear_scan_workspace_size(rows, L), dtype=torch.uint8, device=dev)

    def step(i):
        a, b, h = sets[i]
        cls.linear_scan(a, b, out=h, workspace=ws)

    t = time_loop(step, nsets, steps, warmup, stream)
    gbs = nbytes / t / 1e9
    res = {"workload": f"{name}: {rows} rows x {L} fp32", "value": round(gbs, 1), "unit": "GB/s",
           "us_per_call": round(t * 1e6, 2), "nsets": nsets,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic("linear_scan:" + name, SCAN_SOURCES)}}

    # A plain elementwise kernel with the same traffic (read two arrays, write
    # one) on the same buffers: the practical streaming ceiling for this
    # access pattern, reported beside the scan (not part of the scan).
    def mul_step(i):
        a, b, h = sets[i]
        torch.mul(a, b, out=h)

    tm = time_loop(mul_step, nsets, steps, warmup, stream)
    res["elementwise_ceiling"] = {"kernel": "torch.mul(a, b, out=h)", "us_per_call": round(tm * 1e6, 2),
                                  "GB/s": round(nbytes / tm / 1e9, 1), "scan_over_ceiling": round(tm / t, 3)}
    # bf16 elements (linear_scan_typed): the same rows, a and b rounded to bf16
    res["bf16"] = {}
    for dout, tag in [(torch.float32, "bf16_in_f32_out"), (torch.bfloat16, "bf16_in_bf16_out")]:
        a16, b16 = inp["a"].to(torch.bfloat16), inp["b"].to(torch.bfloat16)
        nb16 = (4 + (4 if dout == torch.float32 else 2)) * rows * L
        ns16 = max(1, math.ceil((1 << 30) / nb16))
        sets16 = [(a16.to(dev), b16.to(dev), torch.empty(rows, L, dtype=dout, device=dev)) for _ in range(ns16)]

        def step16(i, sets16=sets16):
            a, b, h = sets16[i]
            cls.linear_scan(a, b, out=h, workspace=ws)

        t16 = time_loop(step16, ns16, steps, warmup, stream)
        res["bf16"][tag] = {"us_per_call": round(t16 * 1e6, 2), "bytes_per_elem": nb16 // (rows * L),
                            "GB/s": round(nb16 / t16 / 1e9, 1), "frac": round(nb16 / t16 / 1e9 / HBM_PEAK_GBS, 4)}
        del sets16
    if want_cpu:
        res["cpu_baseline"] = cpu_baseline_scan(inp)
    return res


def scan_ceiling_sweep(steps, warmup):
    """linear_scan against torch.mul(a, b, out=h), which moves the same bytes:
    the row lengths of the page's table ("Selective-scan CUDA kernels",
    section "Results": 96 MiB per array, L = 2048 ... 65536), then twice and
    half that size at L = 65536, packed rows of 8186 and longer rows."""
    import torch
    import chunked_linear_scan_amd as cls
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev).manual_seed(1)
    # the page's table: 96 MiB per array at L = 2048 ... 65536; then other sizes
    for rows, L in [(12288, 2048), (6144, 4096), (3072, 8192), (1536, 16384), (768, 32768), (384, 65536),
                    (768, 65536), (192, 65536), (3072, 8186), (96, 262144), (24, 1048576)]:
        nsets = 3
        sets = [(0.9 + 0.1 * torch.rand(rows, L, device=dev, generator=g),
                 torch.randn(rows, L, device=dev, generator=g), torch.empty(rows, L, device=dev))
                for _ in range(nsets)]
        ws = torch.zeros(cls.load_library().linear_scan_workspace_size(rows, L), dtype=torch.uint8, device=dev)
        ts = time_loop(lambda i: cls.linear_scan(sets[i][0], sets[i][1], out=sets[i][2], workspace=ws), nsets,
                       steps, warmup, stream)
        tm = time_loop(lambda i: torch.mul(sets[i][0], sets[i][1], out=sets[i][2]), nsets, steps, warmup, stream)
        nb = 12 * rows * L
        print(json.dumps({"rows": rows, "L": L, "scan_us": round(ts * 1e6, 2), "scan_GBs": round(nb / ts / 1e9, 1),
                          "mul_us": round(tm * 1e6, 2), "mul_GBs": round(nb / tm / 1e9, 1),
                          "mul_over_scan": round(tm / ts, 3)}), flush=True)
        del sets, ws


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="ssd_large",
                    choices=["ssd_small", "ssd_large", "ssd_long", "ssd_tiny"])
    ap.add_argument("--scan-workload", default="scan", choices=["scan", "scan_ragged"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-scan", action="store_true")
    ap.add_argument("--no-autotune", action="store_true",
                    help="skip the autotuner comparison (counter runs: its candidate plans would mix into "
                         "the per-launch figures)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run three plain 1 GiB device copies (the known-size reference that "
                         "scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    ap.add_argument("--scan-ceiling-sweep", action="store_true",
                    help="time linear_scan and torch.mul (same traffic) over a sweep of row lengths, "
                         "print one JSON line per shape, then exit")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter files of "
                         "--copy-probe runs (FETCH_SIZE, WRITE_SIZE) for --workload, then exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic[0], args.record_traffic[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); run it with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.scan_ceiling_sweep:
        scan_ceiling_sweep(args.steps, args.warmup)
        return
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    want_cpu = not args.no_cpu_baseline
    ssd = bench_ssd(args.workload, args.steps, args.warmup, want_cpu, not args.no_autotune)
    shape = ssd["shape"]
    line = {
        "metric": METRIC,
        "value": round(ssd["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ssd["t"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if shape.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; shapes and distributions of the named workload)",
        "config": {"workload": f"{args.workload}: batch {shape.batch}, L={shape.seqlen}, "
                               f"{shape.nheads} heads, P={shape.headdim}, S={shape.dstate}, "
                               f"{shape.ngroups} group(s), chunk {shape.chunk}, {shape.dtype}",
                   "global_batch": shape.batch, "seq_len": shape.seqlen, "parallelism": "single GPU",
                   "buffer_sets": ssd["nsets"]},
        "roofline": ssd["roofline"],
        "autotune": ssd.get("autotune"),
    }
    if "cpu_baseline" in ssd:
        line["cpu_baseline"] = ssd["cpu_baseline"]
    if not args.no_scan:
        line["linear_scan"] = bench_scan(args.scan_workload, args.steps, args.warmup, want_cpu)
        line["linear_scan_three_pass"] = bench_scan3(args.scan_workload, args.steps, args.warmup,
                                                     line["linear_scan"]["us_per_call"])
        line["ssd_step"] = bench_step("decode_large", args.steps, args.warmup, want_cpu)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
