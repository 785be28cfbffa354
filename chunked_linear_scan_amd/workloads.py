"""Seeded synthetic inputs for the SSD forward pass and the scalar linear scan.

This module only draws random numbers with the value distributions of the
workloads below; it holds none of the recurrence's arithmetic, so both the HIP
path and the float64 oracle can consume the very same host tensors.

Workloads (synthetic; each is named by what it is and its sizes):

* ``ssd_tiny``   batch 1, L=256, 2 heads, P=16, S=16, 1 group, chunk 32, fp32
* ``scan``       384 rows x 65536, fp32; ``scan_ragged`` 384 x 65533
* ``ssd_small``  batch 8, L=2048, 24 heads, P=64, S=128, 1 group, chunk 256, bf16
* ``ssd_large``  batch 4, L=8192, 80 heads, P=64, S=128, 1 group, chunk 256, bf16
* ``ssd_long``   batch 1, L=65536, 64 heads, P=64, S=128, 8 groups, chunk 128,
  bf16, slower decay (dt shift -4) and a nonzero initial state ~ N(0, 0.1^2)
* ``ssd_large_p128`` the large layer's 5120 inner channels as heads of dim 128:
  batch 4, L=8192, 40 heads, P=128, S=128, 1 group, chunk 256, bf16
* ``ssd_context_512k`` a half-million-token context: batch 1, L=524288, 8 heads,
  P=64, S=128, 2 groups, chunk 128, bf16, dt shift -4, h0 ~ N(0, 0.1^2)
* ``ssd_long_s256`` a long context at state size 256 (the per-(batch, head)
  kernel's shape): batch 1, L=32768, 8 heads, P=64, S=256, 2 groups, chunk 128,
  bf16, dt shift -4, h0 ~ N(0, 0.1^2)
* ``decode_large`` one decode token (``ssd_step``) for 64 sequences of the
  large-model layer's heads: batch 64, 80 heads, P=64, S=128, 1 group, bf16,
  state ~ N(0, 0.5^2)

SSD draw order (one ``torch.Generator`` seeded per workload): x, B, C, dt_raw,
A_u, D, h0.  dt = softplus(dt_raw + shift); A = -exp(U(0, ln 16)).  x/B/C are
drawn in fp32 and rounded to bf16 (round-to-nearest-even) where the workload is
bf16.  Scan draw order: a_u, mask_u, b; a ~ U(0.9, 1.0) with an independent 1 %
of entries replaced by 1 - 1e-6 (decay close to one).  Decode-step draw order:
h, x, B, C, dt_raw, A_u, D (same distributions as the SSD workloads).
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class SSDShape:
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str  # "f32" or "bf16" for x, B, C and y
    dt_shift: float = -2.0
    h0_std: float = 0.0  # 0 => no initial state (zeros)

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk)


SSD_WORKLOADS = {
    "ssd_tiny": (SSDShape(1, 256, 2, 16, 16, 1, 32, "f32"), 0),
    "ssd_small": (SSDShape(8, 2048, 24, 64, 128, 1, 256, "bf16"), 2),
    "ssd_large": (SSDShape(4, 8192, 80, 64, 128, 1, 256, "bf16"), 3),
    "ssd_long": (SSDShape(1, 65536, 64, 64, 128, 8, 128, "bf16", dt_shift=-4.0, h0_std=0.1), 4),
    # the large layer's inner width (40 x 128 = 80 x 64 channels) in heads of dim 128
    "ssd_large_p128": (SSDShape(4, 8192, 40, 128, 128, 1, 256, "bf16"), 5),
    # a half-million-token context (4096 chunks per chain, chains cut into many segments)
    "ssd_context_512k": (SSDShape(1, 524288, 8, 64, 128, 2, 128, "bf16", dt_shift=-4.0, h0_std=0.1), 6),
    # a long context at state size 256 (per-(batch, head) kernel, each chain cut into segments)
    "ssd_long_s256": (SSDShape(1, 32768, 8, 64, 256, 2, 128, "bf16", dt_shift=-4.0, h0_std=0.1), 7),
}

SCAN_WORKLOADS = {
    "scan": ((384, 65536), 1),
    "scan_ragged": ((384, 65533), 1),
}


def _torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make_ssd_inputs(shape: SSDShape, seed: int) -> dict:
    """Draw one SSD input set on the host (CPU tensors, contiguous).

    Returns x [Bt,L,H,P], dt [Bt,L,H] fp32, A [H] fp32, B and C [Bt,L,G,S],
    D [H] fp32 and h0 [Bt,H,P,S] fp32 or None.
    """
    g = torch.Generator(device="cpu").manual_seed(seed)
    Bt, L, H, P, S, G = (shape.batch, shape.seqlen, shape.nheads, shape.headdim,
                         shape.dstate, shape.ngroups)
    dt_ = _torch_dtype(shape.dtype)
    x = torch.randn(Bt, L, H, P, generator=g).to(dt_)
    B = torch.randn(Bt, L, G, S, generator=g).to(dt_)
    C = torch.randn(Bt, L, G, S, generator=g).to(dt_)
    dt_raw = torch.randn(Bt, L, H, generator=g)
    dt = torch.nn.functional.softplus(dt_raw + shape.dt_shift)
    A_u = torch.rand(H, generator=g)
    A = -torch.exp(A_u * math.log(16.0))
    D = torch.randn(H, generator=g)
    h0 = None
    if shape.h0_std > 0:
        h0 = torch.randn(Bt, H, P, S, generator=g) * shape.h0_std
    return {"x": x.contiguous(), "dt": dt.contiguous(), "A": A.contiguous(),
            "B": B.contiguous(), "C": C.contiguous(), "D": D.contiguous(),
            "h0": None if h0 is None else h0.contiguous(), "chunk": shape.chunk}


def make_scan_inputs(rows: int, length: int, seed: int) -> dict:
    """Draw a [rows, length] fp32 scan problem: a ~ U(0.9, 1) with 1 % of the
    entries set to 1 - 1e-6, b ~ N(0, 1)."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    a_u = torch.rand(rows, length, generator=g)
    mask_u = torch.rand(rows, length, generator=g)
    b = torch.randn(rows, length, generator=g)
    a = 0.9 + 0.1 * a_u
    a = torch.where(mask_u < 0.01, torch.full_like(a, 1.0 - 1e-6), a)
    return {"a": a.to(torch.float32).contiguous(), "b": b.contiguous()}


@dataclasses.dataclass(frozen=True)
class StepShape:
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    dtype: str  # "f32" or "bf16" for x, B, C and y
    dt_shift: float = -2.0
    h_std: float = 0.5


STEP_WORKLOADS = {
    "decode_large": (StepShape(64, 80, 64, 128, 1, "bf16"), 5),
}


def make_step_inputs(shape: StepShape, seed: int) -> dict:
    """Draw one decode-token input set on the host: h [Bt,H,P,S] fp32, x [Bt,H,P],
    dt [Bt,H] fp32, A [H] fp32, B and C [Bt,G,S], D [H] fp32."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    Bt, H, P, S, G = shape.batch, shape.nheads, shape.headdim, shape.dstate, shape.ngroups
    dt_ = _torch_dtype(shape.dtype)
    h = torch.randn(Bt, H, P, S, generator=g) * shape.h_std
    x = torch.randn(Bt, H, P, generator=g).to(dt_)
    B = torch.randn(Bt, G, S, generator=g).to(dt_)
    C = torch.randn(Bt, G, S, generator=g).to(dt_)
    dt = torch.nn.functional.softplus(torch.randn(Bt, H, generator=g) + shape.dt_shift)
    A = -torch.exp(torch.rand(H, generator=g) * math.log(16.0))
    D = torch.randn(H, generator=g)
    return {"h": h.contiguous(), "x": x.contiguous(), "dt": dt.contiguous(), "A": A.contiguous(),
            "B": B.contiguous(), "C": C.contiguous(), "D": D.contiguous()}


def step_workload(name: str) -> dict:
    shape, seed = STEP_WORKLOADS[name]
    return make_step_inputs(shape, seed)


def ssd_workload(name: str) -> dict:
    shape, seed = SSD_WORKLOADS[name]
    return make_ssd_inputs(shape, seed)


def scan_workload(name: str) -> dict:
    (rows, length), seed = SCAN_WORKLOADS[name]
    return make_scan_inputs(rows, length, seed)
