"""GPU tests of the per-shape autotuner (ssd_fwd_autotune, ssd_fwd_plan,
ssd_fwd_autotune_reset) through the C ABI.

The tuner changes only how long chains are cut into segments, so its result,
and every later ssd_fwd call on the tuned plan, must match the float64 oracle
within the bf16 tolerance of the forward-pass tests (rel-L2 <= 2e-2 for y and
the final state; fp32 shapes 1e-5).  The tuned plan is deterministic: a later
ssd_fwd call returns the tuner's own output bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from oracle import compare, ssd as ossd
import parity

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-5


def case(seed, Bt, L, H, P, S, G, dtype):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(Bt, L, H, P, generator=g).to(dtype)
    B = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    C = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    dt = torch.nn.functional.softplus(torch.randn(Bt, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    D = torch.randn(H, generator=g)
    h0 = 0.3 * torch.randn(Bt, H, P, S, generator=g)
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=h0)


@pytest.mark.parametrize("Bt,L,H,G,chunk,P", [(2, 2048, 24, 2, 128, 64), (1, 1000, 12, 3, 64, 64),
                                             (3, 4096, 8, 1, 256, 64), (1, 3000, 6, 2, 256, 128)])
def test_autotune_result_plan_and_later_calls(Bt, L, H, G, chunk, P):
    """The tuner's plan, kept for the shape, reused bit for bit by later
    calls; a head of dim 128 counts as two chains of the plan."""
    S = 128
    print(f"[autotune] Bt={Bt} L={L} H={H} G={G} chunk={chunk} P={P}", flush=True)
    cls.ssd_fwd_autotune_reset()
    c = case(31 + L, Bt, L, H, P, S, G, torch.bfloat16)
    d = {k: v.cuda() for k, v in c.items()}
    before = cls.ssd_fwd_plan(Bt, L, H, P, S, G, chunk)
    assert before["source"] == "heuristic"
    y, hf, info = cls.ssd_fwd_autotune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=chunk,
                                       reps=2)
    torch.cuda.synchronize()
    print(f"  chosen {info}, heuristic {before}", flush=True)
    nchains = Bt * H * (P // 64)
    assert 1 <= info["nsegs"] <= 32 and info["ms_per_call"] > 0
    assert (info["nsegs"] == 1) == (info["nsplit"] == 0) and 0 <= info["nsplit"] <= nchains
    assert (info["nsegs"] > 1) == (info["s3"] is not None)
    assert (info["agg_pieces"] > 0) == (info["s3"] == "reduce") and info["agg_pieces"] >= 0
    assert info["sub_chunk"] in (min(chunk, 128), 64) and info["sub_chunk"] <= min(chunk, 128)
    assert info["cache_policy"] in ("default", "nontemporal")
    assert info["sub_chunk"] == 128 or info["cache_policy"] == "default"
    parity.check_ssd(c, y.float().cpu().numpy(), hf.cpu().numpy(), chunk, "tuned")
    after = cls.ssd_fwd_plan(Bt, L, H, P, S, G, chunk)
    assert after == {"nsegs": info["nsegs"], "nsplit": info["nsplit"], "agg_pieces": info["agg_pieces"],
                     "sub_chunk": info["sub_chunk"], "s3": info["s3"], "cache_policy": info["cache_policy"],
                     "source": "tuned"}
    y2, hf2 = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    assert torch.equal(hf2.view(torch.int32), hf.view(torch.int32))
    # another shape keeps its own plan
    assert cls.ssd_fwd_plan(Bt, L + 128, H, P, S, G, chunk)["source"] == "heuristic"
    cls.ssd_fwd_autotune_reset()
    assert cls.ssd_fwd_plan(Bt, L, H, P, S, G, chunk) == before


def test_autotune_workspace_sized_before_tuning_suffices():
    """A workspace from ssd_fwd_workspace_size before tuning serves the tuner
    and every later call (it covers every candidate plan)."""
    Bt, L, H, P, S, G, chunk = 1, 2048, 16, 64, 128, 1, 128
    cls.ssd_fwd_autotune_reset()
    c = case(5, Bt, L, H, P, S, G, torch.bfloat16)
    d = {k: v.cuda() for k, v in c.items()}
    need = cls.load_library().ssd_fwd_workspace_size(Bt, L, H, P, S, G, chunk, cls.SSD_BF16)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y, hf, info = cls.ssd_fwd_autotune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=chunk,
                                       reps=1, workspace=ws)
    y2, hf2 = cls.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=chunk, workspace=ws)
    torch.cuda.synchronize()
    parity.check_ssd(c, y2.float().cpu().numpy(), hf2.cpu().numpy(), chunk, "after tuning")
    assert cls.workspace_errors([ws]) == 0
    cls.ssd_fwd_autotune_reset()


def test_autotune_without_a_plan_runs_one_plain_pass():
    """fp32 shapes (and bf16 shapes outside the fused path) have no segment
    plan: the tuner runs ssd_fwd once and reports nsegs 0."""
    for dtype, P, S, tol in [(torch.float32, 16, 32, TOL_F32), (torch.bfloat16, 32, 64, TOL_BF16)]:
        c = case(9, 1, 300, 4, P, S, 2, dtype)
        d = {k: v.cuda() for k, v in c.items()}
        y, hf, info = cls.ssd_fwd_autotune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], d["h0"], chunk=64)
        torch.cuda.synchronize()
        assert info["nsegs"] == 0 and info["nsplit"] == 0 and info["agg_pieces"] == 0 and info["sub_chunk"] == 0
        assert cls.ssd_fwd_plan(1, 300, 4, P, S, 2, 64, dtype)["source"] == "none"
        parity.check_ssd(c, y.float().cpu().numpy(), hf.cpu().numpy(), 64, f"{dtype}")
