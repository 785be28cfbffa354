"""GPU parity tests for ssd_fwd (HIP path through the C ABI) against the
float64 oracle.

Every test compares whole outputs (tests/parity.py): the global rel-L2
against the method's tolerance (1e-5 for fp32 inputs, 2e-2 for bf16 inputs
with fp32 state) for y and for the final state, the rel-L2 of every
chunk-long band of the sequence, and an element-wise bound derived from the
roundings of each path.  The full-size workloads are compared whole too, with
the oracle spread over a process pool.  Forced plans go through
ssd_fwd_planned (include/chunked_linear_scan_testing.h), which takes the plan
per call.
"""
import math

import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from chunked_linear_scan_amd import workloads
from oracle import compare
import parity

pytestmark = pytest.mark.gpu


def to_dev(inp):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_run(inp, chunk=None, want_final=True, plan=None, workspace=None):
    d = to_dev(inp)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"), d.get("h0"))
    if plan is None:
        y, hf = cls.ssd_fwd(*args, chunk=chunk or inp["chunk"], want_final_state=want_final, workspace=workspace)
    else:
        y, hf = cls.ssd_fwd_planned(*args, chunk=chunk or inp["chunk"], plan=plan, want_final_state=want_final,
                                    workspace=workspace)
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), (None if hf is None else hf.cpu().numpy())


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


def run_and_check(inp, chunk, label, plan=None, want_final=True):
    print(f"[ssd] {label}", flush=True)
    y, hf = gpu_run(inp, chunk=chunk, plan=plan, want_final=want_final)
    parity.check_ssd(inp, y, hf, chunk, label)
    return y, hf


def test_tiny_fp32_workload():
    inp = workloads.ssd_workload("ssd_tiny")
    run_and_check(inp, inp["chunk"], "ssd_tiny fp32")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
def test_fp32_chunk_sizes_and_ragged(chunk):
    inp = small_case(1, 2, 300, 4, 16, 16, 2, torch.float32)
    run_and_check(inp, chunk, f"fp32 chunk={chunk}")


@pytest.mark.parametrize("P,S,chunk", [(32, 32, 64), (48, 20, 32), (4, 8, 128), (64, 64, 64), (16, 16, 256)])
def test_fp32_staged_and_unstaged_chunks(P, S, chunk):
    """The fp32 kernel stages whole chunks in LDS (the next one loaded while
    the current one is computed) where two fit, and reads global memory per
    phase elsewhere (here the last two shapes); both match the oracle,
    including widths that are not powers of two and a ragged last chunk."""
    inp = small_case(21, 2, 333, 4, P, S, 2, torch.float32)
    run_and_check(inp, chunk, f"fp32 P={P} S={S} chunk={chunk}")


@pytest.mark.parametrize("P,S,chunk,nsegs,h0", [(16, 16, 32, 3, True), (32, 32, 64, 6, True), (64, 64, 64, 2, True),
                                                (16, 16, 16, 64, False), (48, 20, 32, 4, False)])
def test_fp32_segments(P, S, chunk, nsegs, h0):
    """The fp32 kernel with its chains cut into segments (an aggregate
    launch, then each segment folds its predecessors' states into its start
    state), staged and unstaged chunks, with and without h0; against the
    oracle at the fp32 tolerance, and equal on 20 reruns."""
    print(f"[ssd fp32 segments] P={P} S={S} chunk={chunk} nsegs={nsegs} h0={h0}", flush=True)
    inp = small_case(41, 2, 777, 3, P, S, 1, torch.float32, h0=h0)
    plan = cls.plan_request(nsegs=nsegs)
    y, hf = run_and_check(inp, chunk, f"fp32, {nsegs} segments", plan=plan)
    for _ in range(20):
        y2, h2 = gpu_run(inp, chunk=chunk, plan=plan)
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))
        assert np.array_equal(hf.view(np.uint32), h2.view(np.uint32))


@pytest.mark.parametrize("chunk", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("P", [16, 32, 64, 128])
@pytest.mark.parametrize("S", [32, 64, 128, 256])
def test_bf16_shapes_chunks_ragged(P, S, chunk):
    """Every head dim and state size of the bf16 set at every chunk length, on
    a ragged length (fused kernels for P in {64, 128} with S in {64, 128}, the
    per-(batch, head) kernel otherwise)."""
    assert cls.load_library().ssd_fwd_workspace_size(2, 301, 4, P, S, 2, chunk, cls.SSD_BF16) > 0
    inp = small_case(2, 2, 301, 4, P, S, 2, torch.bfloat16)
    y, _ = run_and_check(inp, chunk, f"bf16 P={P} S={S} chunk={chunk}")


@pytest.mark.parametrize("chunk", [32, 128, 256])
def test_bf16_chunk_kernel_on_fused_shapes(chunk):
    """The per-(batch, head) chunk kernel forced on a head-dim-64 shape that
    the fused kernels would otherwise take."""
    inp = small_case(12 + chunk, 2, 700, 4, 64, 128, 2, torch.bfloat16)
    run_and_check(inp, chunk, f"chunk kernel forced, chunk={chunk}", plan=cls.plan_request(path="chunk"))


def test_bf16_edge_lengths():
    for L in (1, 2, 31, 32, 33, 127, 128, 129, 255, 257):
        inp = small_case(3 + L, 1, L, 2, 64, 128, 1, torch.bfloat16)
        run_and_check(inp, 256, f"bf16 L={L}")


@pytest.mark.parametrize("P,S", [(32, 64), (16, 256), (128, 256)])
def test_chunk_kernel_edge_lengths_and_optional_arguments(P, S):
    """The per-(batch, head) kernel at lengths around its sub-chunk and block
    boundaries (a 256-token chunk runs as 128- or 64-token sub-chunks), and
    without D, h0 or the final state."""
    for L in (1, 2, 31, 33, 63, 65, 127, 129, 255, 257, 385):
        inp = small_case(7 + L + P, 1, L, 2, P, S, 1, torch.bfloat16)
        run_and_check(inp, 256, f"chunk kernel P={P} S={S} L={L}")
    inp = small_case(8 + P, 2, 300, 4, P, S, 2, torch.bfloat16, h0=False, D=False)
    y, hf = gpu_run(inp, chunk=256, want_final=False)
    assert hf is None
    parity.check_ssd(inp, y, None, 256, f"chunk kernel P={P} S={S}: no D, no h0, no final state")


@pytest.mark.parametrize("chunk", [32, 64, 128, 256])
def test_whole_chains_many_chunks(chunk):
    """Every (batch, head) chain in one workgroup (one segment), so a
    workgroup walks tens of (sub-)chunks: the loaders' register sets, the
    double-buffered LDS halves and the staged outputs all rotate many times,
    with a ragged last chunk."""
    inp = small_case(90 + chunk, 1, 64 * 40 + 17, 2, 64, 128, 1, torch.bfloat16, dt_shift=-3.0)
    run_and_check(inp, chunk, f"whole chains, chunk={chunk}", plan=cls.plan_request(nsegs=1))


def test_optional_arguments():
    inp = small_case(4, 1, 200, 2, 64, 128, 1, torch.bfloat16, h0=False, D=False)
    y, hf = gpu_run(inp, chunk=64, want_final=False)
    assert hf is None
    parity.check_ssd(inp, y, None, 64, "no D, no h0, no final state")


def test_decay_free_and_zero_timestep():
    inp = small_case(5, 1, 160, 2, 64, 128, 1, torch.bfloat16)
    inp["A"] = torch.zeros_like(inp["A"])  # linear attention
    run_and_check(inp, 64, "a = 0")
    inp = small_case(6, 1, 160, 2, 64, 128, 1, torch.bfloat16)
    inp["dt"] = torch.zeros_like(inp["dt"])  # the state stays h0
    y, hf = run_and_check(inp, 64, "dt = 0")
    assert np.abs(hf - inp["h0"].numpy()).max() == 0.0


def block_decay_case(seed, levels, chunk, L=1000, S=128):
    """Heads whose 32-token blocks decay by a chosen total: with A = -8 and dt
    constant inside a block, the block's log2 decay is 32 * A * log2(e) * dt.
    ``levels[h]`` lists the log2 decays of head h's blocks, cycled along the
    sequence."""
    H = len(levels)
    inp = small_case(seed, 2, L, H, 64, S, 1, torch.bfloat16)
    A = -8.0
    inp["A"] = torch.full((H,), A)
    dt = torch.empty(2, L, H)
    for h, lv in enumerate(levels):
        for t0 in range(0, L, 32):
            ge = lv[(t0 // 32) % len(lv)]
            dt[:, t0:t0 + 32, h] = ge / (32.0 * A * math.log2(math.e))
    inp["dt"] = dt
    inp["chunk"] = chunk
    return inp


@pytest.mark.parametrize("chunk", [32, 64, 128])
def test_diagonal_weights_both_sides_of_the_strong_decay_threshold(chunk):
    """The diagonal-block weights CB dt exp2(GL_i - GL_j) are formed from
    bounded per-token factors when a 32-token block decays by at most 2^100,
    and element by element when it decays more (the factors would overflow).
    Heads sit just above the threshold, just below it, far on each side, and
    alternate between the two forms from block to block."""
    levels = [[-99.99], [-100.01], [-60.0], [-150.0], [-99.99, -100.01], [-150.0, -5.0, -100.01, -0.5]]
    inp = block_decay_case(40 + chunk, levels, chunk)
    run_and_check(inp, chunk, f"block decays around 2^-100, chunk={chunk}")


def test_decay_underflow_to_zero():
    """Blocks whose decay underflows fp32 entirely (2^-400): the state resets
    and only the tokens' own block contributes."""
    inp = block_decay_case(47, [[-400.0], [-400.0, -1.0], [-1.0]], 128)
    run_and_check(inp, 128, "block decays of 2^-400")


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
    parity.check_ssd(inp, y_full.float().cpu().numpy(), h_full.cpu().numpy(), 128, "chained")


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


@pytest.mark.parametrize("plan", [None, {"nsegs": 4, "nsplit": 5}, {"nsegs": 4, "nsplit": 5, "s3": "lookback"},
                                  {"nsegs": 16, "s3": "lookback"}, {"path": "chunk", "nsegs": 3}],
                         ids=["default", "split", "lookback", "lookback16", "chunk-kernel-segments"])
@pytest.mark.parametrize("P", [64, 128])
def test_deterministic_100_runs(plan, P):
    """100 reruns are bit-identical, with whole chains and with split chains
    (reduce-then-fold: the aggregate launch and the fold at each segment
    start; look-back: segments claimed in whatever order the workgroups run,
    folding whatever their predecessors have published, which must not change
    a bit of the result)."""
    inp = small_case(9, 2, 1024, 8, P, 128, 2, torch.bfloat16)
    d = to_dev(inp)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    pr = cls.plan_request(**plan) if plan else None
    run = (lambda: cls.ssd_fwd(*args, chunk=256)) if pr is None else \
        (lambda: cls.ssd_fwd_planned(*args, chunk=256, plan=pr))
    y0, h0 = run()
    for i in range(100):
        y1, h1 = run()
        assert torch.equal(y0.view(torch.int16), y1.view(torch.int16)), i
        assert torch.equal(h0.view(torch.int32), h1.view(torch.int32)), i
    torch.cuda.synchronize()
    parity.check_ssd(inp, y0.float().cpu().numpy(), h0.cpu().numpy(), 256, "determinism")


@pytest.mark.parametrize("name", ["ssd_small", "ssd_large", "ssd_long", "ssd_large_p128"])
def test_full_workloads_whole(name):
    """The full-size workloads as ssd_fwd runs them by default, every output
    compared (the oracle runs over all (batch, head) sequences in a pool)."""
    print(f"[ssd] {name} full size, whole outputs", flush=True)
    inp = workloads.ssd_workload(name)
    y, hf = gpu_run(inp)
    assert np.isfinite(y).all()
    parity.check_ssd_workload(name, y, hf)


@pytest.mark.parametrize("s3", ["reduce", "lookback"])
@pytest.mark.parametrize("nsegs", [1, 2, 3, 7, 64])
def test_segments_forced(nsegs, s3):
    """Every sequence split into segments: reduce-then-fold (start states from
    the aggregate launch's pieces, folded in order) and the single-pass
    look-back (each segment publishes its aggregate, then looks back over the
    chain's earlier segments); one-chunk segments, uneven segments and many
    segments (64: one look-back window reaches back to the first)."""
    inp = small_case(20 + nsegs, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    run_and_check(inp, 32, f"nsegs={nsegs} {s3}", plan=cls.plan_request(nsegs=nsegs, s3=s3))


@pytest.mark.parametrize("s3", ["reduce", "lookback"])
@pytest.mark.parametrize("nsegs,nsplit,chunk", [(2, 1, 128), (5, 4, 128), (4, 5, 32), (3, 2, 64)])
def test_segment_mixed_whole_and_split(nsegs, nsplit, chunk, s3):
    """Plans that run some (batch, head) chains whole and split the last
    `nsplit` chains into segments (the shape of the plan that fills the CUs
    left idle by a partial last round): both kinds of work item in one launch."""
    inp = small_case(60 + nsegs, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    run_and_check(inp, chunk, f"mixed nsegs={nsegs} nsplit={nsplit} chunk={chunk} {s3}",
                  plan=cls.plan_request(nsegs=nsegs, nsplit=nsplit, s3=s3))


@pytest.mark.parametrize("nsegs,pieces,chunk", [(3, 1, 64), (3, 5, 64), (4, 16, 32), (2, 40, 64), (5, 3, 128)])
def test_aggregate_pieces_forced(nsegs, pieces, chunk):
    """The aggregate launch cuts each segment but the last into `pieces`
    pieces (the autotuner searches this count); the output launch folds them
    in order.  Counts from one piece per segment to one chunk per piece (the
    count is capped at the segment's chunks), uneven last pieces included."""
    inp = small_case(80 + pieces, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16, dt_shift=-4.0)
    run_and_check(inp, chunk, f"nsegs={nsegs} pieces={pieces} chunk={chunk}",
                  plan=cls.plan_request(nsegs=nsegs, agg_pieces=pieces))


@pytest.mark.parametrize("s3", ["reduce", "lookback"])
@pytest.mark.parametrize("xcds", [1, 3, 64])
def test_chain_mapping_over_xcds(xcds, s3):
    """The workgroup-to-chain mapping dealt over other XCD counts (1: plain
    index order; for the look-back, that many claim ranges, or one per split
    chain when there are fewer) runs the same chains."""
    inp = small_case(70 + xcds, 3, 700, 6, 64, 128, 2, torch.bfloat16)
    run_and_check(inp, 128, f"xcds={xcds} {s3}", plan=cls.plan_request(nsegs=3, nsplit=7, xcds=xcds, s3=s3))


@pytest.mark.parametrize("plan", [None, dict(s3="lookback"), dict(nsegs=64, s3="lookback", stress_seed=11)],
                         ids=["heuristic", "lookback", "lookback64-stress"])
def test_half_million_token_context(plan):
    """524288 tokens per sequence (4096 chunks): the heuristic cuts the 8
    chains into 32 segments each; the look-back plans fold up to 63
    predecessors.  Every output compared."""
    print(f"[ssd] ssd_context_512k {plan}", flush=True)
    inp = workloads.ssd_workload("ssd_context_512k")
    y, hf = gpu_run(inp, plan=None if plan is None else cls.plan_request(**plan))
    assert np.isfinite(y).all()
    parity.check_ssd_workload("ssd_context_512k", y, hf, label=f"ssd_context_512k {plan}")


def test_long_context_state_size_256():
    """32768 tokens at state size 256 (256 sub-chunks per chain): the
    per-(batch, head) kernel with each of its 8 chains cut into 32 segments,
    every output and the final state compared."""
    print("[ssd] ssd_long_s256 full size, whole outputs", flush=True)
    inp = workloads.ssd_workload("ssd_long_s256")
    y, hf = gpu_run(inp)
    assert np.isfinite(y).all()
    parity.check_ssd_workload("ssd_long_s256", y, hf, label="ssd_long_s256")


@pytest.mark.parametrize("P,S,L,H,G,chunk,nsegs", [
    (32, 64, 3000, 3, 1, 64, 2), (32, 64, 3000, 3, 1, 64, 5), (64, 256, 2000, 2, 2, 128, 3),
    (16, 32, 1500, 4, 2, 32, 64), (128, 128, 999, 2, 1, 256, 7), (64, 128, 700, 2, 2, 16, 4)])
def test_chunk_kernel_segments_forced(P, S, L, H, G, chunk, nsegs):
    """The per-(batch, head) kernel with its chains cut into segments
    (reduce-then-fold: the aggregate launch, then each segment's start state
    folded from h0 and its predecessors' aggregates), including one segment
    per sub-chunk, a ragged last segment and chunk 16; against the oracle."""
    print(f"[ssd chunk segments] P={P} S={S} L={L} chunk={chunk} nsegs={nsegs}", flush=True)
    inp = small_case(31, 2, L, H, P, S, G, torch.bfloat16)
    run_and_check(inp, chunk, f"chunk kernel, {nsegs} segments", plan=cls.plan_request(path="chunk", nsegs=nsegs))


@pytest.mark.parametrize("want_final", [True, False])
def test_chunk_kernel_segments_without_h0_and_d(want_final):
    """Segments with no initial state and no skip term (the first segment
    starts from zero, the fold adds nothing for it), with and without the
    final state."""
    print(f"[ssd chunk segments] no h0, no D, want_final={want_final}", flush=True)
    inp = small_case(33, 1, 2500, 2, 32, 256, 1, torch.bfloat16, h0=False, D=False)
    y, hf = run_and_check(inp, 128, "chunk kernel, 4 segments, no h0/D",
                          plan=cls.plan_request(path="chunk", nsegs=4), want_final=want_final)
    assert (hf is None) == (not want_final)


def test_full_workload_on_the_chunk_kernel():
    """The large-model layer forced onto the per-(batch, head) kernel (the
    configuration the benchmark times for that kernel); every output
    compared."""
    print("[ssd] ssd_large full size, per-(batch, head) kernel", flush=True)
    inp = workloads.ssd_workload("ssd_large")
    y, hf = gpu_run(inp, plan=cls.plan_request(path="chunk"))
    parity.check_ssd_workload("ssd_large", y, hf, label="ssd_large chunk kernel")


@pytest.mark.parametrize("name", ["ssd_large", "ssd_long"])
def test_full_workloads_lookback(name):
    """The two workloads whose plans split chains, with the split chains'
    state passed by the single-pass look-back instead of reduce-then-fold;
    every output compared."""
    print(f"[ssd] {name} full size, look-back plan", flush=True)
    inp = workloads.ssd_workload(name)
    y, hf = gpu_run(inp, plan=cls.plan_request(s3="lookback"))
    parity.check_ssd_workload(name, y, hf, label=f"{name} look-back")


@pytest.mark.parametrize("seed", [3, 1001])
@pytest.mark.parametrize("nsegs,nsplit,L", [(4, 0, 4096), (16, 0, 4096), (64, 3, 8192)])
def test_segment_lookback_stress_gives_the_same_bits(seed, nsegs, nsplit, L):
    """Look-back stress on the SSD segments ("Selective-scan CUDA kernels",
    section "Correctness"): a quarter of the segments, picked by a hash of the
    seed, wait up to ~100 us before they publish their aggregate.  The look-back
    folds from the chain's first segment in segment order whatever the timing,
    so y and h_final equal the unperturbed look-back call bit for bit, and the
    oracle within the bf16 bounds."""
    print(f"[ssd stress] seed={seed} nsegs={nsegs} nsplit={nsplit} L={L}", flush=True)
    inp = small_case(seed, 2, L, 4, 64, 128, 1, torch.bfloat16)
    base = cls.plan_request(nsegs=nsegs, nsplit=nsplit, s3="lookback")
    stress = cls.plan_request(nsegs=nsegs, nsplit=nsplit, s3="lookback", stress_seed=seed)
    y0, h0 = gpu_run(inp, chunk=128, plan=base)
    y1, h1 = gpu_run(inp, chunk=128, plan=stress)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(h0.view(np.uint32), h1.view(np.uint32))
    parity.check_ssd(inp, y1, h1, 128, f"stress {seed}")


@pytest.mark.parametrize("plan", [dict(), dict(nsegs=4), dict(nsegs=4, nsplit=3, s3="lookback"),
                                  dict(nsegs=3, agg_pieces=2)], ids=["heuristic", "split", "lookback", "pieces"])
def test_cache_policies_give_the_same_bits(plan):
    """The non-temporal x/y instances differ from the default ones only in
    the cache policy of two memory operations: y and h_final are equal bit
    for bit, and both match the oracle."""
    print(f"[ssd policy] {plan}", flush=True)
    inp = small_case(11, 2, 5000, 4, 64, 128, 2, torch.bfloat16)
    outs = {}
    for pol in ("default", "nontemporal"):
        outs[pol] = gpu_run(inp, chunk=128, plan=cls.plan_request(cache_policy=pol, **plan))
    (y0, h0), (y1, h1) = outs["default"], outs["nontemporal"]
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(h0.view(np.uint32), h1.view(np.uint32))
    parity.check_ssd(inp, y1, h1, 128, f"non-temporal {plan}")


C_SOURCE_CASES = [
    # (seed, Bt, L, H, P, S, G, chunk, plan)
    (12, 2, 5000, 4, 64, 128, 2, 128, dict()),
    (13, 2, 5000, 4, 64, 128, 2, 128, dict(nsegs=4, nsplit=3, s3="lookback")),
    (14, 1, 3001, 6, 128, 64, 3, 64, dict(nsegs=3)),
    (15, 2, 777, 8, 64, 64, 1, 32, dict(nsegs=2, agg_pieces=3)),
    (16, 1, 2049, 16, 64, 128, 1, 256, dict(nsegs=3, sub_chunk=32)),
]


@pytest.mark.parametrize("case", C_SOURCE_CASES, ids=["heuristic", "lookback", "p128-sub64", "ragged-pieces",
                                                      "sub32"])
def test_c_sources_give_the_same_bits(case):
    """The state term reads C from the CB pass's fragment-major copy or from
    the C rows themselves: the same values in the same MFMA lanes, so y and
    h_final are equal bit for bit, and both match the oracle."""
    seed, Bt, L, H, P, S, G, chunk, plan = case
    print(f"[ssd c-source] {case}", flush=True)
    inp = small_case(seed, Bt, L, H, P, S, G, torch.bfloat16)
    outs = {src: gpu_run(inp, chunk=chunk, plan=cls.plan_request(c_source=src, **plan)) for src in ("copy", "rows")}
    (y0, h0), (y1, h1) = outs["copy"], outs["rows"]
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(h0.view(np.uint32), h1.view(np.uint32))
    parity.check_ssd(inp, y1, h1, chunk, f"C rows {case}")


HEAD128_PLANS = [None, dict(nsegs=3, nsplit=3), dict(nsegs=4, nsplit=5, s3="lookback"),
                 dict(nsegs=2, s3="reduce", sub_chunk=64), dict(nsegs=3, nsplit=1, s3="lookback", cache_policy="nontemporal")]


@pytest.mark.parametrize("chunk", [64, 256])
@pytest.mark.parametrize("S", [64, 128])
@pytest.mark.parametrize("plan", HEAD128_PLANS, ids=["heuristic", "split3", "lookback5", "sub64", "lookback1-nt"])
def test_head_dim_128_on_the_fused_path(plan, S, chunk):
    """Head dim 128 runs on the fused kernels as two chains of head dim 64
    that share the head's dt, A and D.  An odd nsplit splits one half of a
    head into segments and runs the other half whole."""
    inp = small_case(170 + S + chunk, 2, 64 * 25 + 9, 4, 128, S, 2, torch.bfloat16, dt_shift=-3.0)
    assert cls.ssd_fwd_plan(2, 64 * 25 + 9, 4, 128, S, 2, chunk)["nsegs"] >= 1
    run_and_check(inp, chunk, f"P=128 S={S} chunk={chunk} {plan}",
                  plan=None if plan is None else cls.plan_request(**plan))


@pytest.mark.parametrize("plan", HEAD128_PLANS[:3], ids=["heuristic", "split3", "lookback5"])
def test_head_dim_128_equals_two_heads_of_64(plan):
    """A head of dim 128 gives, bit for bit, what two heads of dim 64 give
    when they hold its two halves of x and h0 and both carry its dt, A and D
    (the same memory for x, y and the states; the same chains and plan)."""
    print(f"[ssd P=128 as 2x64] {plan}", flush=True)
    Bt, L, H, S, G = 2, 64 * 20 + 3, 4, 128, 2
    w = small_case(190, Bt, L, H, 128, S, G, torch.bfloat16, dt_shift=-3.0)
    n = {"x": w["x"].reshape(Bt, L, 2 * H, 64), "dt": w["dt"].repeat_interleave(2, dim=-1).contiguous(),
         "A": w["A"].repeat_interleave(2), "B": w["B"], "C": w["C"], "D": w["D"].repeat_interleave(2),
         "h0": w["h0"].reshape(Bt, 2 * H, 64, S), "chunk": 32}
    req = None if plan is None else cls.plan_request(**plan)
    y_w, h_w = gpu_run(w, chunk=128, plan=req)
    y_n, h_n = gpu_run(n, chunk=128, plan=req)
    assert np.array_equal(y_w.reshape(y_n.shape).view(np.uint32), y_n.view(np.uint32))
    assert np.array_equal(h_w.reshape(h_n.shape).view(np.uint32), h_n.view(np.uint32))
    parity.check_ssd(w, y_w, h_w, 128, f"P=128 {plan}")


@pytest.mark.parametrize("P,S,Bt,H,narrow", [(128, 32, 2, 6, 64), (64, 256, 1, 4, 16)])
def test_chunk_kernel_head_split_equals_narrow_heads(P, S, Bt, H, narrow):
    """A head's channels are independent: the per-(batch, head) kernel runs a
    head of dim 128 as two heads of 64 that share its dt, A and D, and bit
    for bit a head gives what narrower heads carrying its column blocks and
    its dt, A and D give (the same sub-chunk tile and whole chains)."""
    k = P // narrow
    L, G, chunk = 64 * 12 + 5, 2 if H % 2 == 0 else 1, 128
    print(f"[ssd split] P={P} S={S} H={H} -> {k} x {narrow}", flush=True)
    w = small_case(200 + P + S, Bt, L, H, P, S, G, torch.bfloat16, dt_shift=-3.0)
    n = {"x": w["x"].reshape(Bt, L, k * H, narrow), "dt": w["dt"].repeat_interleave(k, dim=-1).contiguous(),
         "A": w["A"].repeat_interleave(k), "B": w["B"], "C": w["C"], "D": w["D"].repeat_interleave(k),
         "h0": w["h0"].reshape(Bt, k * H, narrow, S), "chunk": 32}
    req = cls.plan_request(path="chunk")
    y_w, h_w = gpu_run(w, chunk=chunk, plan=req)
    y_n, h_n = gpu_run(n, chunk=chunk, plan=req)
    assert np.array_equal(y_w.reshape(y_n.shape).view(np.uint32), y_n.view(np.uint32))
    assert np.array_equal(h_w.reshape(h_n.shape).view(np.uint32), h_n.view(np.uint32))
    parity.check_ssd(w, y_w, h_w, chunk, f"split P={P} S={S}")


@pytest.mark.parametrize("P,S,chunk", [(128, 128, 128), (128, 128, 256), (128, 256, 256), (64, 256, 256),
                                     (16, 256, 128)])
def test_chunk_kernel_sub_chunks(P, S, chunk):
    """The per-(batch, head) kernel forced on shapes whose chunk tiles would
    overflow LDS: it runs them as sub-chunks of 128 or 64 tokens (only the
    rounding changes)."""
    inp = small_case(197 + P + S + chunk, 2, 700, 4, P, S, 2, torch.bfloat16)
    run_and_check(inp, chunk, f"chunk kernel forced P={P} S={S} chunk={chunk}", plan=cls.plan_request(path="chunk"))


@pytest.mark.parametrize("A_value", [0.0, -1e-3])
@pytest.mark.parametrize("plan", [dict(nsegs=4, s3="reduce"), dict(nsegs=8, s3="lookback"),
                                  dict(nsegs=3, agg_pieces=2, s3="reduce"), dict(nsegs=16, nsplit=2, s3="lookback")],
                         ids=["reduce4", "lookback8", "pieces", "lookback16"])
def test_split_plans_carry_state_without_decay(A_value, plan):
    """Cut chains with no decay (A = 0: every segment's alpha is exactly 1, so
    h0 and every earlier token reach the last output) or nearly none (alpha
    about 0.7 over the sequence): the folds of reduce-then-fold and of the
    look-back carry the whole history, where strong decay would let a wrong
    fold hide behind an alpha that underflows to 0."""
    print(f"[ssd fold] A={A_value} {plan}", flush=True)
    inp = small_case(170, 2, 64 * 40 + 17, 3, 64, 128, 1, torch.bfloat16)
    inp["A"] = torch.full_like(inp["A"], A_value)
    run_and_check(inp, 64, f"fold A={A_value} {plan}", plan=cls.plan_request(**plan))


def test_explicit_workspace_error_word_stays_zero():
    """A caller-owned workspace, reused over shapes and plans (reduce-then-fold
    and look-back, whose claim counters, finish count and epoch must be left
    ready for the next call whatever ran in between): results match the
    oracle and the error word at its start stays 0 (no bounded wait gave up)."""
    lib = cls.load_library()
    shapes = [(2, 1000, 4, 2, 128), (1, 3000, 6, 3, 64), (2, 2000, 8, 1, 256), (1, 700, 4, 2, 32)]
    plans = (None, cls.plan_request(nsegs=5), cls.plan_request(nsegs=5, s3="lookback"),
             cls.plan_request(nsegs=3, nsplit=2, s3="lookback"))
    need = max(lib.ssd_fwd_planned_workspace_size(b, L, H, 64, 128, G, T, cls.SSD_BF16, pl or cls.plan_request())
               for b, L, H, G, T in shapes for pl in plans)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for i, (b, L, H, G, T) in enumerate(shapes):
        inp = small_case(200 + i, b, L, H, 64, 128, G, torch.bfloat16)
        for plan in plans:
            y, hf = gpu_run(inp, chunk=T, plan=plan, workspace=ws)
            parity.check_ssd(inp, y, hf, T, f"shared workspace {i}")
    assert cls.workspace_errors([ws]) == 0


def test_binding_rejects_bad_tensors_before_any_launch():
    """The binding checks device, dtype, shape and layout of every tensor
    before the library is called."""
    inp = to_dev(small_case(3, 1, 64, 2, 64, 128, 1, torch.bfloat16))
    args = [inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["h0"]]
    bad = []
    a = list(args); a[0] = inp["x"].transpose(1, 2)  # non-contiguous x
    bad.append((a, ValueError))
    a = list(args); a[1] = inp["dt"].to(torch.float16)  # wrong dt dtype
    bad.append((a, TypeError))
    a = list(args); a[4] = inp["C"][:, :32]  # C of another length
    bad.append((a, ValueError))
    a = list(args); a[2] = inp["A"].cpu()  # A on the host
    bad.append((a, ValueError))
    a = list(args); a[3] = inp["B"].float()  # B and x of different dtypes
    bad.append((a, TypeError))
    for a, err in bad:
        with pytest.raises(err):
            cls.ssd_fwd(*a, chunk=32)
    with pytest.raises(ValueError):
        cls.linear_scan(torch.ones(4, 100, device="cuda").t(), torch.ones(100, 4, device="cuda"))


def test_planned_call_rejects_bad_plans():
    inp = small_case(3, 1, 64, 2, 64, 128, 1, torch.bfloat16)
    d = to_dev(inp)
    args = (d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"])
    for bad in (cls.plan_request(nsegs=65), cls.PlanRequest(3, 0, 0, 0, 0, 0, 0),
                cls.PlanRequest(0, 3, 0, 0, 0, 0, 0), cls.PlanRequest(0, 0, 0, 0, 0, 0, 1)):
        with pytest.raises(cls.SSDError):
            cls.ssd_fwd_planned(*args, chunk=32, plan=bad)


@pytest.mark.parametrize("chunk,sub,s3", [(128, 64, "reduce"), (256, 64, "lookback"), (256, 32, "reduce"),
                                          (64, 32, "lookback"), (128, 64, "lookback")])
def test_sub_chunk_forced(chunk, sub, s3):
    """The fused kernels run shorter sub-chunks than the chunk (an
    instantiation the autotuner may pick); the chunked form equals the
    recurrence at every chunk length, so only rounding changes."""
    inp = small_case(150 + sub + chunk, 2, 64 * 30 + 5, 3, 64, 128, 1, torch.bfloat16, dt_shift=-3.0)
    run_and_check(inp, chunk, f"chunk={chunk} sub={sub} {s3}",
                  plan=cls.plan_request(nsegs=3, nsplit=4, s3=s3, sub_chunk=sub))
