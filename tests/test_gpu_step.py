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

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_Y_BF16 = 1e-2


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


def assert_close(got, ref, tol, label):
    err = compare.rel_l2(got, ref)
    print(f"  {label}: rel-L2 {err:.3e}", flush=True)
    assert err <= tol, (label, err, compare.first_mismatch(got, ref, rtol=50 * tol, atol=50 * tol))


SHAPES = [(2, 4, 64, 128, 2), (3, 6, 17, 16, 3), (1, 2, 130, 256, 1), (2, 2, 5, 4, 2), (1, 8, 64, 64, 8),
          (2, 3, 33, 32, 1), (1, 4, 7, 8, 2)]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Bt,H,P,S,G", SHAPES)
def test_step_matches_oracle(Bt, H, P, S, G, dtype):
    print(f"[step] Bt={Bt} H={H} P={P} S={S} G={G} {dtype}", flush=True)
    c = step_case(100 + S + P, Bt, H, P, S, G, dtype)
    y, hn = gpu_step(c)
    ry, rh = ossd.ssd_step(*(np64(c[k]) for k in ("h", "x", "dt", "A", "B", "C", "D")))
    assert_close(hn, rh, TOL_F32, "state")
    assert_close(y, ry, TOL_F32 if dtype == torch.float32 else TOL_Y_BF16, "y")


def test_step_without_skip_term_and_zero_timestep():
    c = step_case(7, 2, 4, 64, 128, 2, torch.float32, D=False)
    c["dt"] = torch.zeros_like(c["dt"])
    h_before = c["h"].numpy().copy()
    y, hn = gpu_step(c)
    assert np.array_equal(hn, h_before)  # exp(0) h + 0 x^T, exactly
    ry, _ = ossd.ssd_step(*(np64(c[k]) for k in ("h", "x", "dt", "A", "B", "C", "D")))
    assert_close(y, ry, TOL_F32, "y dt=0")


def test_step_deterministic():
    c = step_case(8, 4, 8, 64, 128, 2, torch.bfloat16)
    d = {k: (None if v is None else v.cuda()) for k, v in c.items()}
    outs = []
    for _ in range(3):
        h = d["h"].clone()
        y = cls.ssd_step(h, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"])
        outs.append((y.view(torch.int16).cpu().numpy(), h.view(torch.int32).cpu().numpy()))
    for y, h in outs[1:]:
        assert np.array_equal(y, outs[0][0]) and np.array_equal(h, outs[0][1])


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
    ry, rh = ossd.ssd_loop(np64(x), np64(dt), np64(A), np64(B), np64(C), np64(Dv), np64(h0))
    tol = TOL_F32 if dtype == torch.float32 else 2e-2
    assert_close(got[:, L1:], ry[:, L1:], tol, "decoded y")
    assert_close(got[:, :L1], ry[:, :L1], tol, "prefill y")
    assert_close(h.cpu().numpy(), rh, tol, "final state")
