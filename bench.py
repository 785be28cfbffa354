"""Throughput benchmark of the SSD forward pass and the linear scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload ssd_long]

One step is one ``ssd_fwd`` call (every launch of the call: the CB pass, the
aggregate launch when chains are split, the output launch) over one batch of
the named workload, with inputs already resident in HBM.  The headline
workload is the long-context prefill (batch 1, L = 65536, 64 heads, P = 64,
S = 128, 8 groups, chunk 128, nonzero initial state), the largest of the
workloads.

Timing protocol ("Selective-scan CUDA kernels", section "Results": median of
15 interleaved samples, repetitions inside the timed window; section "Two real
bugs the tests caught": kernels too short for the GPU to boost):

* every workload is warmed up with W steps and then until at least 50 ms of
  its own GPU time has run, and each of its timed windows is preceded by
  about 1 ms of its own untimed calls (the clocks settle after a
  latency-bound workload such as the tiny fp32 one);
* the K timed steps of the headline run as 15 windows, each bracketed by HIP
  events on the launch stream; the other workloads (the small- and
  large-model layer shapes, the large layer in heads of dim 128, the large
  layer forced onto the per-(batch, head) kernel, a long context at state
  size 256 (the per-(batch, head) kernel in segments), the tiny fp32 one,
  the scans, the decode step) run their own
  windows of at least 5 ms, interleaved with the headline's: window w of
  every workload runs before window w + 1 of any;
* inputs and outputs rotate over enough buffer copies that each workload's
  footprint exceeds 1 GiB, so the 256 MB Infinity Cache cannot serve repeats;
* ``value`` is tokens / (mean time per step over the K timed steps); the
  median and IQR of the 15 windows are reported beside it;
* GPU clocks and power (amd-smi, else rocm-smi) are recorded before and after.

``roofline`` is for the whole ssd_fwd call: algorithmic bytes (every input
read once, every output written once) over the mean call time, against
8 TB/s; the MFMA side (causal-triangle flops over 2.5 PFLOP/s) is reported
beside it, and ``per_launch`` splits the call into its launches (a separate
loop that records events between them through ssd_fwd_planned).

The CPU baseline is the float64 oracle, unmodified, over a process pool on the
host's cores (one whole (batch, head) sequence or row block per job), scaled
to the metric's unit.

Other modes: ``--scan-ceiling-sweep``, ``--copy-probe`` / ``--record-traffic``
(HBM traffic counters), ``--no-autotune``, ``--no-cpu-baseline``,
``--only-headline`` (the headline workload alone, for counter runs),
``--no-side-ssd`` (the headline, the scans and the decode step: a counter run
that holds one SSD shape), ``--path chunk`` (the headline workload on the
per-(batch, head) kernel), ``--s3-ab`` (the two inter-segment schemes).

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "SSD fwd tokens/sec (B·L) + % of HBM/MFMA roofline; linear-scan GB/s"
NWIN = 15                      # timed windows per workload
MIN_WINDOW_S = 5e-3            # each window of a side workload lasts at least this long
LEAD_S = 1e-3                  # untimed calls of a workload right before each of its windows
WARM_S = 50e-3                 # GPU time each workload runs before its first window


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


# ---------------------------------------------------------------------------
# traffic counters (rocprofv3 --pmc) committed under profiles/
# ---------------------------------------------------------------------------
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


SSD_SOURCES = ["ssd_fused.hpp", "ssd_fused.hip", "common.hpp", "ssd_kernels.hpp", "ssd_dispatch.cpp"]
# the per-(batch, head) kernel at 128-token sub-chunks (the CB pass and the chunk kernel)
CHUNK_SOURCES = ["ssd_bf16.hpp", "ssd_bf16_t128.hip", "common.hpp", "ssd_kernels.hpp", "ssd_dispatch.cpp"]
SCAN_SOURCES = ["linear_scan.hip", "common.hpp"]
STEP_SOURCES = ["ssd_step.hip", "common.hpp"]


def measured_traffic(key, sources):
    """HBM bytes per call from profiles/traffic.json, only if they were taken
    on the current kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            db = json.load(f)
    except (OSError, ValueError):
        return None
    rec = db.get(key)
    if not rec or rec.get("source_digest") != source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_call")


def record_traffic(fetch_csv, write_csv, workload):
    """Write profiles/traffic.json from two rocprofv3 --pmc runs of this script
    with --copy-probe (one with FETCH_SIZE, one with WRITE_SIZE).  Each counter
    is scaled by what it reads for the 1 GiB device copies of --copy-probe
    (copyBuffer dispatches of 131072 workgroups).  An SSD call's bytes are the
    sum over its kernels (per-dispatch means)."""
    import csv

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

    def per_kernel(pat):
        # pat: a substring of the kernel name, or "a|b": both substrings
        pats = pat.split("|")
        f = [v for (k, g), vs in fe.items() if all(q in k for q in pats) for v in vs]
        w = [v for (k, g), vs in wr.items() if all(q in k for q in pats) for v in vs]
        if not f or not w:
            return None
        return statistics.mean(f) * sf * 1024, statistics.mean(w) * sw * 1024, len(f)

    groups = [("ssd_fwd:" + workload, SSD_SOURCES, ["ssd_cbt_kernel<", "ssd_fused_agg_kernel<", "ssd_fused_kernel<"]),
              ("ssd_fwd_chunk_kernel:" + workload, CHUNK_SOURCES,
               ["ssd_cb_kernel<", "ssd_chunk_kernel<|false>", "ssd_chunk_kernel<|true>"]),
              ("linear_scan:scan", SCAN_SOURCES, ["linear_scan_kernel<false, float, float, false, 2048>"]),
              ("ssd_step:decode_large", STEP_SOURCES, ["ssd_step_kernel"])]
    for key, srcs, pats in groups:
        names = {"ssd_chunk_kernel<|false>": "ssd_chunk_kernel", "ssd_chunk_kernel<|true>": "ssd_chunk_kernel (aggregate)"}
        parts = {names.get(p, p.rstrip("<")): per_kernel(p) for p in pats}
        parts = {k: v for k, v in parts.items() if v is not None}
        if not parts:
            continue
        fb = sum(v[0] for v in parts.values())
        wb = sum(v[1] for v in parts.values())
        db[key] = {"source_digest": source_digest(srcs), "hbm_bytes_per_call": round(fb + wb),
                   "fetch_bytes": round(fb), "write_bytes": round(wb),
                   "per_kernel": {k: {"fetch_bytes": round(v[0]), "write_bytes": round(v[1]), "dispatches": v[2]}
                                  for k, v in parts.items()},
                   "scale_fetch": round(sf, 4), "scale_write": round(sw, 4)}
        print(key, db[key])
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)


# ---------------------------------------------------------------------------
# clocks and power
# ---------------------------------------------------------------------------
def gpu_state():
    """GPU clocks and power as amd-smi (else rocm-smi) reports them, as text
    trimmed to the lines that carry them; None when neither tool answers."""
    for cmd in (["amd-smi", "metric", "-g", "0", "-c", "-p"], ["rocm-smi", "--showclocks", "--showpower"]):
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=20)
        except (OSError, subprocess.SubprocessError):
            continue
        if r.returncode != 0 or not r.stdout.strip():
            continue
        keep = [ln.strip() for ln in r.stdout.splitlines()
                if any(k in ln.upper() for k in ("CLK", "CLOCK", "POWER", "MHZ", " W"))]
        return {"tool": cmd[0], "lines": keep[:40]}
    return None


# ---------------------------------------------------------------------------
# workloads as runners: step(i) enqueues one call on buffer set i
# ---------------------------------------------------------------------------
class Runner:
    name = ""
    nsets = 1

    def step(self, i):
        raise NotImplementedError


def _dev():
    import torch
    return torch.device("cuda:0")


class SsdRunner(Runner):
    """One ssd_fwd call per step.  path "chunk": the call forced onto the
    per-(batch, head) kernel through ssd_fwd_planned."""

    def __init__(self, name, path="auto"):
        import torch
        import chunked_linear_scan_amd as cls
        from chunked_linear_scan_amd import workloads
        self.cls = cls
        self.workload = name
        self.path = path
        self.name = name + ("" if path == "auto" else ":chunk_kernel")
        self.plan = cls.plan_request(path=path) if path != "auto" else None
        self.shape, _ = workloads.SSD_WORKLOADS[name]
        # the call runs the per-(batch, head) kernel: forced, or a shape outside the fused set
        self.chunk_path = self.plan is not None or not (
            self.shape.dtype == "bf16" and self.shape.headdim in (64, 128) and self.shape.dstate in (64, 128))
        self.inp = workloads.ssd_workload(name)
        self.alg_bytes = ssd_alg_bytes(self.inp, self.shape)
        self.flops = ssd_alg_flops(self.shape)
        self.tokens = self.shape.batch * self.shape.seqlen
        self.nsets = max(1, math.ceil((1 << 30) / self.alg_bytes))
        dev = _dev()
        s = self.shape
        self.sets = []
        for _ in range(self.nsets):
            d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in self.inp.items()}
            d["y"] = torch.empty_like(d["x"])
            self.sets.append(d)
        self.hf = torch.empty(s.batch, s.nheads, s.headdim, s.dstate, dtype=torch.float32, device=dev)

    def step(self, i):
        d = self.sets[i % self.nsets]
        if self.plan is None:
            self.cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=self.shape.chunk,
                             out=d["y"])
        else:
            self.cls.ssd_fwd_planned(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                     chunk=self.shape.chunk, plan=self.plan, out=d["y"])

    def describe(self):
        s = self.shape
        return (f"{self.workload}: batch {s.batch}, L={s.seqlen}, {s.nheads} heads, P={s.headdim}, S={s.dstate}, "
                f"{s.ngroups} group(s), chunk {s.chunk}, {s.dtype}"
                + (f", h0 ~ N(0, {s.h0_std}^2)" if s.h0_std > 0 else "")
                + ("" if self.plan is None else ", forced onto the per-(batch, head) kernel"))

    def traffic_key(self):
        return (("ssd_fwd_chunk_kernel:" if self.chunk_path else "ssd_fwd:") + self.workload,
                CHUNK_SOURCES if self.chunk_path else SSD_SOURCES)

    def per_launch(self, calls=20):
        """Mean time of each launch of a call: events between the launches
        (ssd_fwd_planned with the default plan), on their own loop."""
        import torch
        cls = self.cls
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(calls)]
        for k in range(calls):
            d = self.sets[k % self.nsets]
            cls.ssd_fwd_planned(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=self.shape.chunk,
                                plan=self.plan, out=d["y"], events=evs[k])
        torch.cuda.synchronize()
        t = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / calls * 1e3 for j in range(3)]
        if self.chunk_path:  # the CB pass and the chunk kernel's launches, timed as one
            return {"cb_pass_and_chunk_kernel_us": round(t[2], 2),
                    "grid": "one workgroup per (batch, head) chain, or per segment of a chain where the "
                            "chains fill at most half of the CUs (then after an aggregate launch)"}
        plan = cls.ssd_fwd_plan(self.shape.batch, self.shape.seqlen, self.shape.nheads, self.shape.headdim,
                                self.shape.dstate, self.shape.ngroups, self.shape.chunk, self.inp["x"].dtype)
        return {"cb_pass_us": round(t[0], 2), "aggregate_launch_us": round(t[1], 2),
                "output_launch_us": round(t[2], 2), "sum_us": round(sum(t), 2), "plan": plan}


class ScanRunner(Runner):
    def __init__(self, name, dtype_in="f32", dtype_out="f32"):
        import torch
        import chunked_linear_scan_amd as cls
        from chunked_linear_scan_amd import workloads
        self.cls = cls
        self.name = name + ("" if (dtype_in, dtype_out) == ("f32", "f32") else f":{dtype_in}->{dtype_out}")
        self.inp = workloads.scan_workload(name)
        rows, L = self.inp["a"].shape
        self.rows, self.L = rows, L
        tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
        tin, tout = tdt[dtype_in], tdt[dtype_out]
        self.bytes_per_elem = 2 * (4 if dtype_in == "f32" else 2) + (4 if dtype_out == "f32" else 2)
        self.alg_bytes = self.bytes_per_elem * rows * L
        self.nsets = max(1, math.ceil((1 << 30) / self.alg_bytes))
        dev = _dev()
        self.sets = [(self.inp["a"].to(tin).to(dev), self.inp["b"].to(tin).to(dev),
                      torch.empty(rows, L, dtype=tout, device=dev)) for _ in range(self.nsets)]
        self.ws = torch.zeros(cls.load_library().linear_scan_workspace_size(rows, L), dtype=torch.uint8, device=dev)

    def step(self, i):
        a, b, h = self.sets[i % self.nsets]
        self.cls.linear_scan(a, b, out=h, workspace=self.ws)


class HillisSteeleRunner(ScanRunner):
    """linear_scan_hillis_steele: the register-resident Hillis-Steele in-tile
    scan, the page's fair comparison for the work-efficient kernel."""

    def __init__(self, name):
        super().__init__(name)
        self.name = name + ":hillis_steele"

    def step(self, i):
        a, b, h = self.sets[i % self.nsets]
        self.cls.linear_scan_hillis_steele(a, b, out=h, workspace=self.ws)


class Scan3Runner(ScanRunner):
    def __init__(self, name):
        super().__init__(name)
        self.name = name + ":three_pass"

    def step(self, i):
        a, b, h = self.sets[i % self.nsets]
        self.cls.linear_scan_three_pass(a, b, out=h)


class MulRunner(ScanRunner):
    """torch.mul(a, b, out=h): a plain elementwise kernel with the scan's
    traffic (read two arrays, write one), as context for the scan."""

    def __init__(self, name):
        super().__init__(name)
        self.name = name + ":torch.mul"

    def step(self, i):
        import torch
        a, b, h = self.sets[i % self.nsets]
        torch.mul(a, b, out=h)


class StreamRunner(ScanRunner):
    """stream_mul_f32: a hand-written kernel that moves the scan's exact bytes
    (h = a * b), one configuration of its vector width and cache policy."""

    def __init__(self, name, vec, nt):
        super().__init__(name)
        self.vec, self.nt = vec, nt
        self.name = f"{name}:stream_v{vec}_{'nt' if nt else 'default'}"

    def step(self, i):
        a, b, h = self.sets[i % self.nsets]
        self.cls.stream_mul(a, b, out=h, vec=self.vec, nt=self.nt)


class TiledScanRunner(ScanRunner):
    """fp32 linear_scan with an explicit tile size (linear_scan_planned)."""

    def __init__(self, base, name, tile):
        self.__dict__.update(base.__dict__)
        self.name, self.tile = name, tile

    def step(self, i):
        a, b, h = self.sets[i % self.nsets]
        self.cls.linear_scan_planned(a, b, tile=self.tile, out=h, workspace=self.ws)


class StepRunner(Runner):
    def __init__(self, name):
        import torch
        import chunked_linear_scan_amd as cls
        from chunked_linear_scan_amd import workloads
        self.cls = cls
        self.name = name
        self.shape, _ = workloads.STEP_WORKLOADS[name]
        self.inp = workloads.step_workload(name)
        s = self.shape
        esz = 2 if s.dtype == "bf16" else 4
        Bt, H, P, S, G = s.batch, s.nheads, s.headdim, s.dstate, s.ngroups
        self.alg_bytes = (2 * Bt * H * P * S * 4 + 2 * Bt * H * P * esz + Bt * H * 4 + 2 * Bt * G * S * esz
                          + 2 * H * 4)
        self.nsets = max(1, math.ceil((1 << 30) / self.alg_bytes))
        dev = _dev()
        self.sets = []
        for _ in range(self.nsets):
            d = {k: v.to(dev) for k, v in self.inp.items()}
            d["y"] = torch.empty_like(d["x"])
            self.sets.append(d)

    def step(self, i):
        d = self.sets[i % self.nsets]
        self.cls.ssd_step(d["h"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], out=d["y"])


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------
def warm(runner, warmup_steps):
    """W steps, then more until >= 50 ms of this workload's GPU time has run.
    Returns (warm-up GPU seconds, seconds per step estimate)."""
    import torch
    stream = torch.cuda.current_stream()
    for i in range(warmup_steps):
        runner.step(i)
    torch.cuda.synchronize()
    total, n, est = 0.0, 4, None
    while total < WARM_S:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            runner.step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) / 1e3
        total += dt
        est = dt / n
        n = min(4 * n, 1024)
    return total, est


def split_steps(k, nwin):
    base, extra = divmod(k, nwin)
    return [base + (1 if w < extra else 0) for w in range(nwin)]


def timed_windows(runners, plan, lead=None):
    """Interleaved windows: window w of every runner before window w + 1 of
    any.  plan[name] = steps per window (list of NWIN); lead[name] = untimed
    steps right before each of its windows (the clocks settle on this
    workload after the one before it).  Returns per runner the seconds of
    each window."""
    import torch
    stream = torch.cuda.current_stream()
    out = {r.name: [] for r in runners}
    offs = {r.name: 0 for r in runners}
    lead = lead or {}
    torch.cuda.synchronize()
    for w in range(NWIN):
        for r in runners:
            n = plan[r.name][w]
            if n == 0:
                out[r.name].append(0.0)
                continue
            for i in range(lead.get(r.name, 0)):
                r.step(offs[r.name] + i)
            offs[r.name] += lead.get(r.name, 0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                r.step(offs[r.name] + i)
            e1.record(stream)
            offs[r.name] += n
            out[r.name].append((e0, e1))
    torch.cuda.synchronize()
    res = {}
    for r in runners:
        res[r.name] = [(x[0].elapsed_time(x[1]) / 1e3 if isinstance(x, tuple) else 0.0) for x in out[r.name]]
    return res


def summarize(window_s, steps):
    """Mean over all steps, and median / quartiles of the per-step time of
    the windows (seconds)."""
    per = sorted(t / n for t, n in zip(window_s, steps) if n > 0)
    q = statistics.quantiles(per, n=4) if len(per) >= 2 else [per[0]] * 3
    return {"mean": sum(window_s) / sum(steps), "median": statistics.median(per), "q1": q[0], "q3": q[2],
            "min": per[0], "max": per[-1]}


def _us(s):
    return round(s * 1e6, 2)


def timing_block(st, steps):
    return {"windows": NWIN, "steps_per_window": steps, "mean_us": _us(st["mean"]), "median_us": _us(st["median"]),
            "q1_us": _us(st["q1"]), "q3_us": _us(st["q3"]), "iqr_us": _us(st["q3"] - st["q1"]),
            "min_us": _us(st["min"]), "max_us": _us(st["max"])}


# ---------------------------------------------------------------------------
# CPU baselines: the oracle over a process pool on the host's cores
# ---------------------------------------------------------------------------
def _cores():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return max(1, min(n, 64))


def _pool_run(fn, jobs, cores):
    import multiprocessing as mp
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    t0 = time.perf_counter()
    with mp.get_context("spawn").Pool(cores) as pool:
        pool.map(fn, jobs, chunksize=1)
    return time.perf_counter() - t0


def _oracle_ssd_job(args):
    from oracle import ssd as ossd
    ossd.ssd_loop(*args)


def _oracle_scan_job(args):
    from oracle import scan as oscan
    oscan.scan_loop(*args)


def _oracle_step_job(args):
    from oracle import ssd as ossd
    ossd.ssd_step(*args)


def cpu_baseline_ssd(runner, budget_s=15.0):
    """Oracle wall time on as many whole (batch, head) sequences as fit the
    budget (all of them when they do), one sequence per job."""
    import torch
    inp, shape = runner.inp, runner.shape
    cores = _cores()
    H, G, L = shape.nheads, shape.ngroups, shape.seqlen
    np64 = lambda t: None if t is None else t.to(dtype=torch.float64).numpy()

    def job(bb, h, n=None):
        g = h // (H // G)
        sl = slice(None) if n is None else slice(0, n)
        return (np64(inp["x"][bb:bb + 1, sl, h:h + 1]), np64(inp["dt"][bb:bb + 1, sl, h:h + 1]),
                np64(inp["A"][h:h + 1]), np64(inp["B"][bb:bb + 1, sl, g:g + 1]),
                np64(inp["C"][bb:bb + 1, sl, g:g + 1]), np64(inp["D"][h:h + 1]),
                None if inp["h0"] is None else np64(inp["h0"][bb:bb + 1, h:h + 1]))

    probe = min(L, 1024)
    t0 = time.perf_counter()
    _oracle_ssd_job(job(0, 0, probe))
    t_job = (time.perf_counter() - t0) * L / probe
    total = shape.batch * H
    njobs = max(1, min(total, int(budget_s * cores / max(t_job, 1e-6))))
    pairs = [(bb, h) for bb in range(shape.batch) for h in range(H)]
    if njobs < total:
        pairs = [(k % shape.batch, (k * 7919) % H) for k in range(njobs)]
    wall = _pool_run(_oracle_ssd_job, [job(bb, h) for bb, h in pairs], cores)
    tok_equiv = L * len(pairs) / H  # a token counts once all H heads of its row are done
    return {"value": tok_equiv / wall, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(pairs)} of {total} whole (batch, head) sequences of {L} tokens, one per job on "
                      f"{cores} processes, wall {wall:.1f}s"}


def cpu_baseline_scan(runner):
    """The whole workload, its rows split into one block per core."""
    a, b = runner.inp["a"].numpy(), runner.inp["b"].numpy()
    cores = _cores()
    blk = max(1, math.ceil(a.shape[0] / cores))
    jobs = [(a[r:r + blk], b[r:r + blk]) for r in range(0, a.shape[0], blk)]
    wall = _pool_run(_oracle_scan_job, jobs, min(cores, len(jobs)))
    return {"value": runner.alg_bytes / wall / 1e9, "unit": "GB/s", "cores": min(cores, len(jobs)),
            "kind": "oracle", "sample": f"whole workload {tuple(a.shape)}, rows in {len(jobs)} blocks, "
                                        f"one per process, wall {wall:.2f}s"}


def cpu_baseline_step(runner):
    """One decode token of the whole batch, batch rows split over the cores."""
    import torch
    arrs = [runner.inp[k].to(torch.float64).numpy() for k in ("h", "x", "dt", "A", "B", "C", "D")]
    Bt = arrs[0].shape[0]
    cores = _cores()
    blk = max(1, math.ceil(Bt / cores))
    jobs = []
    for r in range(0, Bt, blk):
        jobs.append(tuple(v[r:r + blk] if k not in (3, 6) else v for k, v in enumerate(arrs)))
    wall = _pool_run(_oracle_step_job, jobs, min(cores, len(jobs)))
    return {"value": runner.alg_bytes / wall / 1e9, "unit": "GB/s", "cores": min(cores, len(jobs)),
            "kind": "oracle", "sample": f"whole workload (one token, state {tuple(arrs[0].shape)}), batch rows in "
                                        f"{len(jobs)} blocks, one per process, wall {wall:.2f}s"}


# ---------------------------------------------------------------------------
def ssd_result(r, st, steps):
    t = st["mean"]
    gbs = r.alg_bytes / t / 1e9
    tflops = r.flops / t / 1e12
    res = {"workload": r.describe(), "value": round(r.tokens / t, 1), "unit": "tokens/s",
           "us_per_call": _us(t), "timing": timing_block(st, steps), "buffer_sets": r.nsets,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": measured_traffic(*r.traffic_key()),
                        "kernel": "whole ssd_fwd call", "alg_bytes": r.alg_bytes,
                        "frac_at_median": round(r.alg_bytes / st["median"] / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma": {"alg_flops": r.flops, "achieved_tflops": round(tflops, 1),
                                 "peak_tflops": BF16_PEAK_TFLOPS, "frac": round(tflops / BF16_PEAK_TFLOPS, 4)}}}
    return res


def scan_result(r, st, steps):
    t = st["mean"]
    gbs = r.alg_bytes / t / 1e9
    return {"workload": f"{r.name}: {r.rows} rows x {r.L}", "value": round(gbs, 1), "unit": "GB/s",
            "us_per_call": _us(t), "timing": timing_block(st, steps), "buffer_sets": r.nsets,
            "bytes_per_elem": r.bytes_per_elem,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def step_result(r, st, steps):
    t = st["mean"]
    gbs = r.alg_bytes / t / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "us_per_call": _us(t), "timing": timing_block(st, steps),
            "buffer_sets": r.nsets,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "alg_bytes": r.alg_bytes}}


def autotune_compare(r, steps, warmup):
    """The plan ssd_fwd_autotune keeps for the workload against the built-in
    heuristic, each timed in interleaved windows right after tuning."""
    cls = r.cls
    s = r.shape
    heur = cls.ssd_fwd_plan(s.batch, s.seqlen, s.nheads, s.headdim, s.dstate, s.ngroups, s.chunk, r.inp["x"].dtype)
    d0 = r.sets[0]
    _, _, info = cls.ssd_fwd_autotune(d0["x"], d0["dt"], d0["A"], d0["B"], d0["C"], d0["D"], d0["h0"],
                                      chunk=s.chunk, reps=10, out=d0["y"])
    base = min(s.chunk, 128)
    tuned = cls.plan_request(nsegs=info["nsegs"], nsplit=info["nsplit"], agg_pieces=info["agg_pieces"],
                             s3=info["s3"], sub_chunk=0 if info["sub_chunk"] == base else info["sub_chunk"],
                             cache_policy=info["cache_policy"]) \
        if info["nsegs"] > 0 else None
    cls.ssd_fwd_autotune_reset()

    class Planned(Runner):
        def __init__(self, name, plan):
            self.name, self.plan, self.nsets = name, plan, r.nsets

        def step(self, i):
            d = r.sets[i % r.nsets]
            if self.plan is None:
                cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=s.chunk, out=d["y"])
            else:
                cls.ssd_fwd_planned(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=s.chunk,
                                    out=d["y"], plan=self.plan)

    a, b = Planned("tuned", tuned), Planned("heuristic", None)
    for x in (a, b):
        warm(x, warmup)
    n = split_steps(steps, NWIN)
    ws = timed_windows([a, b], {"tuned": n, "heuristic": n})
    ta, tb = summarize(ws["tuned"], n), summarize(ws["heuristic"], n)
    keys = ("nsegs", "nsplit", "agg_pieces", "sub_chunk", "s3", "cache_policy")
    return {"plan": {k: info[k] for k in keys}, "heuristic_plan": {k: heur[k] for k in keys},
            "tuner_ms_per_call": round(info["ms_per_call"], 4),
            "us_per_call_tuned": _us(ta["median"]), "us_per_call_heuristic": _us(tb["median"]),
            "speedup": round(tb["median"] / ta["median"], 3)}


def scan_autotune_compare(runners, steps, warmup):
    """The tile linear_scan_autotune keeps for each scan workload against the
    built-in 8192-element tile, timed in interleaved windows after tuning."""
    out = {}
    for r in runners:
        cls = r.cls
        cls.linear_scan_autotune_reset()
        a, b, h = r.sets[0]
        _, info = cls.linear_scan_autotune(a, b, out=h, reps=20, workspace=r.ws)
        cls.linear_scan_autotune_reset()
        tuned, builtin = TiledScanRunner(r, "tuned", info["tile"]), TiledScanRunner(r, "built-in", 8192)
        for x in (tuned, builtin):
            warm(x, warmup)
        n = [max(1, min(2000, math.ceil(MIN_WINDOW_S / 50e-6)))] * NWIN
        ws = timed_windows([tuned, builtin], {"tuned": n, "built-in": n})
        ta, tb = summarize(ws["tuned"], n), summarize(ws["built-in"], n)
        out[r.name] = {"tile": info["tile"], "built_in_tile": 8192, "tuner_ms_per_call": round(info["ms_per_call"], 4),
                       "us_per_call_tuned": _us(ta["median"]), "us_per_call_built_in": _us(tb["median"]),
                       "speedup": round(tb["median"] / ta["median"], 3)}
    return out


def s3_ab(steps, warmup, names=("ssd_large", "ssd_long")):
    """The two inter-segment schemes of split chains timed against each other
    on the workloads whose plans split chains: reduce-then-fold (aggregate
    launch, then a fold at each segment start) and the single-pass look-back
    (segments publish aggregates and look back), each at the built-in segment
    count and at other counts, in interleaved windows.  One JSON line per
    workload."""
    import chunked_linear_scan_amd as cls

    class Planned(Runner):
        def __init__(self, base, name, plan):
            self.base, self.name, self.plan, self.nsets = base, name, plan, base.nsets

        def step(self, i):
            d = self.base.sets[i % self.base.nsets]
            cls.ssd_fwd_planned(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"],
                                chunk=self.base.shape.chunk, out=d["y"], plan=self.plan)

    for name in names:
        base = SsdRunner(name)
        runners = []
        for nsegs in (0, 2, 4, 8, 16):
            for s3 in ("reduce", "lookback"):
                runners.append(Planned(base, f"{s3}:nsegs={nsegs or 'heuristic'}",
                                       cls.plan_request(nsegs=nsegs, s3=s3)))
        for r in runners:
            warm(r, warmup)
        n = split_steps(max(steps, NWIN), NWIN)
        win = timed_windows(runners, {r.name: n for r in runners})
        out = {r.name: _us(summarize(win[r.name], n)["median"]) for r in runners}
        print(json.dumps({"workload": base.describe(), "median_us_per_call": out}), flush=True)
        del base, runners


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ssd_long",
                    choices=["ssd_small", "ssd_large", "ssd_long", "ssd_tiny", "ssd_large_p128", "ssd_long_s256"])
    ap.add_argument("--path", default="auto", choices=["auto", "chunk"],
                    help="SSD path of --workload: auto (what ssd_fwd runs) or chunk (forced onto the "
                         "per-(batch, head) kernel; counter and trace runs of that kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-autotune", action="store_true",
                    help="skip the autotuner comparison (counter runs: its candidate plans would mix into "
                         "the per-kernel figures)")
    ap.add_argument("--only-headline", action="store_true",
                    help="time the headline workload alone (counter and trace runs)")
    ap.add_argument("--no-clocks", action="store_true",
                    help="do not run amd-smi for the clock lines (for runs under a profiler, whose preloaded "
                         "library would start the GPU in that child too)")
    ap.add_argument("--no-side-ssd", action="store_true",
                    help="run no SSD workload but the headline (scans and the decode step still run): "
                         "counter runs then hold one SSD shape's kernels")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run three plain 1 GiB device copies (the known-size reference that "
                         "scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    ap.add_argument("--scan-ceiling-sweep", action="store_true",
                    help="time linear_scan and torch.mul (same traffic) over a sweep of row lengths, "
                         "print one JSON line per shape, then exit")
    ap.add_argument("--s3-ab", action="store_true",
                    help="time reduce-then-fold against the single-pass look-back for split chains "
                         "(ssd_large, ssd_long), print one JSON line per workload, then exit")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc counter files of "
                         "--copy-probe runs (FETCH_SIZE, WRITE_SIZE) for --workload, then exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.record_traffic[0], args.record_traffic[1], args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the kernels run on a single GPU; "
              f"run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.steps < NWIN:
        print(f"--steps must be at least {NWIN} (one per timed window)", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.scan_ceiling_sweep:
        scan_ceiling_sweep(args.steps, args.warmup)
        return
    if args.s3_ab:
        s3_ab(args.steps, args.warmup)
        return
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    want_cpu = not args.no_cpu_baseline

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    clocks_before = None if args.no_clocks else gpu_state()
    head = SsdRunner(args.workload, args.path)
    log(f"headline {head.describe()}, {head.nsets} buffer set(s)")
    side = []
    if not args.only_headline:
        if not args.no_side_ssd:
            for name, path in (("ssd_large", "auto"), ("ssd_large_p128", "auto"), ("ssd_small", "auto"),
                               ("ssd_large", "chunk"), ("ssd_long_s256", "auto"), ("ssd_tiny", "auto")):
                if (name, path) != (args.workload, args.path):
                    side.append(SsdRunner(name, path))
        side += [ScanRunner("scan"), ScanRunner("scan_ragged"), ScanRunner("scan", "bf16", "f32"),
                 ScanRunner("scan", "bf16", "bf16"), ScanRunner("scan", "f16", "f32"), ScanRunner("scan", "f16", "f16"),
                 HillisSteeleRunner("scan"), Scan3Runner("scan"), MulRunner("scan"), StreamRunner("scan", 2, True),
                 StreamRunner("scan", 4, True), StreamRunner("scan", 2, False), StepRunner("decode_large")]
    runners = [head] + side
    plan = {head.name: split_steps(args.steps, NWIN)}
    lead = {}
    warm_s = {}
    for r in runners:
        warm_s[r.name], est = warm(r, args.warmup)
        lead[r.name] = max(1, min(200, math.ceil(LEAD_S / max(est, 1e-7))))
        if r is not head:
            n = max(1, min(2000, math.ceil(MIN_WINDOW_S / max(est, 1e-7))))
            plan[r.name] = [n] * NWIN
        log(f"warmed {r.name}: {warm_s[r.name] * 1e3:.1f} ms, ~{est * 1e6:.1f} us/step")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    win = timed_windows(runners, plan, lead)
    t_wall = time.perf_counter() - t_wall
    stats = {r.name: summarize(win[r.name], plan[r.name]) for r in runners}
    clocks_after = None if args.no_clocks else gpu_state()
    log(f"timed {sum(sum(v) for v in win.values()) * 1e3:.1f} ms of GPU time in {t_wall:.2f} s")

    hs = stats[head.name]
    res = ssd_result(head, hs, plan[head.name])
    res["roofline"]["per_launch"] = head.per_launch()
    line = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(hs["mean"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.shape.dtype,
        "data": "synthetic (seeded; shapes and value distributions of the named workload)",
        "config": {"workload": head.describe(), "global_batch": head.shape.batch, "seq_len": head.shape.seqlen,
                   "parallelism": "single GPU", "buffer_sets": head.nsets},
        "timing": dict(res["timing"], warmup_gpu_ms=round(warm_s[head.name] * 1e3, 1),
                       untimed_lead_steps_per_window=lead[head.name]),
        "roofline": res["roofline"],
        "clocks": {"before": clocks_before, "after": clocks_after},
    }
    others = {}
    for r in side:
        st = stats[r.name]
        if isinstance(r, SsdRunner):
            o = ssd_result(r, st, plan[r.name])
            o["roofline"]["per_launch"] = r.per_launch()
        elif isinstance(r, StepRunner):
            o = step_result(r, st, plan[r.name])
        else:
            o = scan_result(r, st, plan[r.name])
        o["timing"]["untimed_lead_steps_per_window"] = lead[r.name]
        others[r.name] = o
    if others:
        line["workloads"] = {k: v for k, v in others.items() if k.startswith("ssd_") and k != "decode_large"}
        sc = others["scan"]
        sc["three_pass"] = others["scan:three_pass"]
        sc["three_pass"]["time_ratio_to_single_pass"] = round(
            stats["scan:three_pass"]["mean"] / stats["scan"]["mean"], 3)
        sc["three_pass"]["traffic_model_ratio"] = round(7 / 3, 3)
        sc["elementwise_ceiling"] = dict(others["scan:torch.mul"], kernel="torch.mul(a, b, out=h)",
                                         scan_over_ceiling=round(stats["scan:torch.mul"]["mean"]
                                                                 / stats["scan"]["mean"], 3))
        streams = [r for r in side if isinstance(r, StreamRunner)]
        best = min(streams, key=lambda r: stats[r.name]["median"])
        sc["stream_ceiling"] = dict(
            others[best.name], kernel=f"stream_mul_f32 (h = a * b), vec={best.vec}, nt={int(best.nt)}: the fastest of "
                                      + ", ".join(f"{r.name.split(':')[1]} {_us(stats[r.name]['median'])} us"
                                                  for r in streams),
            scan_over_ceiling=round(stats[best.name]["median"] / stats["scan"]["median"], 3))
        sc["bf16"] = {"bf16_in_f32_out": others["scan:bf16->f32"], "bf16_in_bf16_out": others["scan:bf16->bf16"]}
        sc["f16"] = {"f16_in_f32_out": others["scan:f16->f32"], "f16_in_f16_out": others["scan:f16->f16"]}
        sc["hillis_steele"] = dict(others["scan:hillis_steele"], time_ratio_to_single_pass=round(
            stats["scan:hillis_steele"]["mean"] / stats["scan"]["mean"], 3))
        sc["ragged"] = others["scan_ragged"]
        sc["roofline"]["traffic"] = measured_traffic("linear_scan:scan", SCAN_SOURCES)
        line["linear_scan"] = sc
        step = next(r for r in side if isinstance(r, StepRunner))
        so = others[step.name]
        so["workload"] = (f"{step.name}: one decode token, batch {step.shape.batch}, {step.shape.nheads} heads, "
                          f"P={step.shape.headdim}, S={step.shape.dstate}, {step.shape.ngroups} group(s), "
                          f"{step.shape.dtype}")
        so["tokens_per_s"] = round(step.shape.batch / stats[step.name]["mean"], 1)
        so["roofline"]["traffic"] = measured_traffic("ssd_step:" + step.name, STEP_SOURCES)
        line["ssd_step"] = so
    if not args.no_autotune and args.path == "auto":
        log("autotune comparison")
        line["autotune"] = autotune_compare(head, max(args.steps // 2, NWIN), args.warmup)
        if others:
            log("scan autotune comparison")
            line["linear_scan"]["autotune"] = scan_autotune_compare(
                [r for r in side if type(r) is ScanRunner and r.name in ("scan", "scan_ragged")], args.steps,
                args.warmup)
    if want_cpu:
        log("cpu baselines")
        line["cpu_baseline"] = cpu_baseline_ssd(head)
        if others:
            line["linear_scan"]["cpu_baseline"] = cpu_baseline_scan(next(r for r in side if r.name == "scan"))
            line["ssd_step"]["cpu_baseline"] = cpu_baseline_step(next(r for r in side if isinstance(r, StepRunner)))
    print(json.dumps(line), flush=True)


def scan_ceiling_sweep(steps, warmup):
    """linear_scan against torch.mul(a, b, out=h), which moves the same bytes:
    the row lengths of the page's table ("Selective-scan CUDA kernels",
    section "Results": 96 MiB per array, L = 2048 ... 65536), then twice and
    half that size at L = 65536, packed rows of 8186 and longer rows."""
    import torch
    import chunked_linear_scan_amd as cls
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(1)
    for rows, L in [(12288, 2048), (6144, 4096), (3072, 8192), (1536, 16384), (768, 32768), (384, 65536),
                    (768, 65536), (192, 65536), (3072, 8186), (96, 262144), (24, 1048576)]:
        sets = [(0.9 + 0.1 * torch.rand(rows, L, device=dev, generator=g),
                 torch.randn(rows, L, device=dev, generator=g), torch.empty(rows, L, device=dev))
                for _ in range(3)]
        ws = torch.zeros(cls.load_library().linear_scan_workspace_size(rows, L), dtype=torch.uint8, device=dev)

        class S(Runner):
            name, nsets = "scan", 3

            def step(self, i):
                a, b, h = sets[i % 3]
                cls.linear_scan(a, b, out=h, workspace=ws)

        class M(Runner):
            name, nsets = "mul", 3

            def step(self, i):
                a, b, h = sets[i % 3]
                torch.mul(a, b, out=h)

        class K(Runner):
            name, nsets = "stream", 3

            def step(self, i):
                a, b, h = sets[i % 3]
                cls.stream_mul(a, b, out=h, vec=2, nt=True)

        rs = [S(), M(), K()]
        for r in rs:
            warm(r, warmup)
        n = split_steps(max(steps, NWIN), NWIN)
        win = timed_windows(rs, {"scan": n, "mul": n, "stream": n})
        ts, tm = summarize(win["scan"], n)["median"], summarize(win["mul"], n)["median"]
        tk = summarize(win["stream"], n)["median"]
        nb = 12 * rows * L
        print(json.dumps({"rows": rows, "L": L, "scan_us": _us(ts), "scan_GBs": round(nb / ts / 1e9, 1),
                          "mul_us": _us(tm), "mul_GBs": round(nb / tm / 1e9, 1),
                          "mul_over_scan": round(tm / ts, 3), "stream_us": _us(tk),
                          "stream_GBs": round(nb / tk / 1e9, 1), "stream_over_scan": round(tk / ts, 3)}), flush=True)
        del sets, ws


if __name__ == "__main__":
    main()
