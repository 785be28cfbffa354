"""GPU parity tests for ssd_step (one decode token, HIP path through the C ABI)
against the float64 oracle.

Tolerances: rel-L2 <= 1e-5 for fp32 inputs (y and the new state); for bf16
inputs the state stays fp32 (1e-5) and y is rounded to bf16 once (rel-L2
<= 1e-2).  The oracle consumes the same host tensors (bf16 values converted
exactly to float64).
"""
import math

import numpy as np
import pytest
import torch

import chunked_linear_scan_amd as cls
from oracle import compare, ssd as ossd
import parity

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5


def step_case(seed, Bt, H, P, S, G, dtype, D=True, dt_shift=-2.0):
    g = torch.Generator().manual_seed(seed)
    h = 0.5 * torch.randn(Bt, H, P, S, generator=g)
    x = torch.randn(Bt, H, P, generator=g).to(dtype)
    B = torch.randn(Bt, G, S, generator=g).to(dtype)
    C = torch.randn(Bt, G, S, generator=g).to(dtype)
    dt = torch.nn.functional.softplus(torch.randn(Bt, H, generator=g) + dt_shift)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    Dv = torch.randn(H, generator=g) if D else None
    return dict(h=h, x=x, dt=dt, A=A, B=B, C=C, D=Dv)


def np64(t):
    return None if t is None else t.to(torch.float64).numpy()


def gpu_step(c):
    d = {k: (None if v is None else v.cuda()) for k, v in c.items()}
    y = cls.ssd_step(d["h"], d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
    torch.cuda.synchronize()
    return y.float().cpu().numpy(), d["h"].cpu().numpy()


SHAPES = [(2, 4, 64, 128, 2), (3, 6, 17, 16, 3), (1, 2, 130, 256, 1), (2, 2, 5, 4, 2), (1, 8, 64, 64, 8),
          (2, 3, 33, 32, 1), (1, 4, 7, 8, 2)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Bt,H,P,S,G", SHAPES)
def test_step_matches_oracle(Bt, H, P, S, G, dtype):
    print(f"[step] Bt={Bt} H={H} P={P} S={S} G={G} {dtype}", flush=True)
    c = step_case(100 + S + P, Bt, H, P, S, G, dtype)
    y, hn = gpu_step(c)
    parity.check_step(c, y, hn, f"step {dtype}")


def test_step_without_skip_term_and_zero_timestep():
    c = step_case(7, 2, 4, 64, 128, 2, torch.float32, D=False)
    c["dt"] = torch.zeros_like(c["dt"])
    h_before = c["h"].numpy().copy()
    y, hn = gpu_step(c)
    assert np.array_equal(hn, h_before)  # exp(0) h + 0 x^T, exactly
    parity.check_step(c, y, hn, "dt = 0")


def test_step_deterministic_100_runs():
    c = step_case(8, 4, 8, 64, 128, 2, torch.bfloat16)
    d = {k: (None if v is None else v.cuda()) for k, v in c.items()}
    first = None
    for i in range(101):
        h = d["h"].clone()
        y = cls.ssd_step(h, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
        if first is None:
            first = (y.view(torch.int16).clone(), h.view(torch.int32).clone())
        else:
            assert torch.equal(y.view(torch.int16), first[0]) and torch.equal(h.view(torch.int32), first[1]), i
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_after_prefill_matches_token_loop(dtype):
    """Prefill the first tokens with ssd_fwd, then decode the rest one token at
    a time with ssd_step from its final state: the outputs and the last state
    are those of the oracle's token loop over the whole sequence."""
    Bt, L, L1, H, P, S, G = 2, 300, 257, 4, 64, 128, 2
    print(f"[step] prefill {L1} + decode {L - L1}, {dtype}", flush=True)
    g = torch.Generator().manual_seed(11)
    x = torch.randn(Bt, L, H, P, generator=g).to(dtype)
    B = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    C = torch.randn(Bt, L, G, S, generator=g).to(dtype)
    dt = torch.nn.functional.softplus(torch.randn(Bt, L, H, generator=g) - 2.0)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    Dv = torch.randn(H, generator=g)
    h0 = 0.3 * torch.randn(Bt, H, P, S, generator=g)
    dx, dB, dC, ddt, dA, dD, dh0 = (t.cuda() for t in (x, B, C, dt, A, Dv, h0))
    y1, h = cls.ssd_fwd(dx[:, :L1].contiguous(), ddt[:, :L1].contiguous(), dA, dB[:, :L1].contiguous(),
                        dC[:, :L1].contiguous(), dD, dh0, chunk=64)
    ys = [y1.float()]
    for t in range(L1, L):
        y = cls.ssd_step(h, dx[:, t].contiguous(), ddt[:, t].contiguous(), dA, dB[:, t].contiguous(),
                         dC[:, t].contiguous(), dD)
        ys.append(y.float()[:, None])
    got = torch.cat(ys, dim=1).cpu().numpy()
    torch.cuda.synchronize()
    args = (np64(x), np64(dt), np64(A), np64(B), np64(C), np64(Dv), np64(h0))
    ry, rh = ossd.ssd_loop(*args)
    ya, ha = ossd.ssd_abs_terms(*args)
    kind = "f32" if dtype == torch.float32 else "bf16"
    tol = TOL_F32 if dtype == torch.float32 else 2e-2
    yb, hb = parity.SSD_BOUNDS[kind]["y"], parity.SSD_BOUNDS[kind]["h"]
    parity.check_with_scale(got[:, L1:], ry[:, L1:], ya[:, L1:], yb, tol, "decoded y")
    parity.check_with_scale(got[:, :L1], ry[:, :L1], ya[:, :L1], yb, tol, "prefill y", band=64)
    parity.check_with_scale(h.cpu().numpy(), rh, ha, hb, tol, "final state")
