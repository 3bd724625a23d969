"""Seeded synthetic inputs for Hybrid Linear Temporal Attention workloads.

This module only draws random tensors with the shapes and value distributions
of the workloads (q, k, v, the per-token gates alpha and beta). It holds none
of the method's arithmetic, so both the HIP path and the CPU oracle consume
its output. Everything is deterministic given the workload's seed.

Workloads (frame-major token order, token t in frame t // P):
  tiny_fp32      B1 H2  d64  T16  P16   fp32, k unit-norm, W=4, DSWA 4 taps dil 2
  swa_dswa_bf16  B2 H16 d128 T21  P1560 bf16, q,k,v ~ N(0,1)/sqrt(d), W=3, 4 taps dil 4
  gla_bf16       B1 H16 d128 T21  P1560 bf16, q,k unit-norm, v ~ N(0,1), chunk 64
  hybrid_stream  B2 H16 d128 T21  P1560 bf16 (+64 streamed frames, ring of 13)
  long_horizon   B1 H16 d128 T336 P1560 bf16
  dilated_d6     B1 H16 d128 T61  P1560 bf16, W=3, 4 taps dil 6 (the pages' dilation 6)
  dilated_d12    B1 H16 d128 T61  P1560 bf16, W=3, 4 taps dil 12 (the pages' dilation 12)
Gates: alpha = sigmoid(N(mu_a, 1)), beta = sigmoid(N(0, 1)), per token and head.
The 21 x 1560 shape stands for 81-frame clips after 4x temporal and a 30x52
patch grid after 16x spatial compression; the long horizon for multi-minute
rollouts. At 61 frames, the queries of frames 36 to 60 reach all four taps of
dilation 12 ((4 - 1) * 12 + 1 = 37 frames). No dataset is read: these synthetic draws stand in for video latents.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    P: int
    dk: int
    dv: int
    dtype: torch.dtype
    window: int = 3
    taps: int = 4
    dilation: int = 4
    chunk: int = 64
    qv_std: float = 1.0        # std of q and v draws (before any unit-norm)
    k_std: float = 1.0
    q_unit: bool = False       # L2-normalise q per token
    k_unit: bool = False       # L2-normalise k per token
    alpha_mu: float = 3.0
    beta_mu: float = 0.0
    stream_frames: int = 0     # frames appended one at a time after the prefix
    ring: int = 13
    seed: int = 0

    @property
    def L(self) -> int:
        return self.T * self.P

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_INV_SQRT128 = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 2, 16, 16, 64, 64, torch.float32,
                          window=4, taps=4, dilation=2, chunk=64, k_unit=True,
                          alpha_mu=3.0, seed=0),
    "swa_dswa_bf16": Workload("swa_dswa_bf16", 2, 16, 21, 1560, 128, 128, torch.bfloat16,
                              window=3, taps=4, dilation=4, qv_std=_INV_SQRT128,
                              k_std=_INV_SQRT128, seed=1),
    "gla_bf16": Workload("gla_bf16", 1, 16, 21, 1560, 128, 128, torch.bfloat16,
                         chunk=64, q_unit=True, k_unit=True, alpha_mu=4.0, seed=2),
    "hybrid_stream": Workload("hybrid_stream", 2, 16, 21, 1560, 128, 128, torch.bfloat16,
                              window=3, taps=4, dilation=4, chunk=64,
                              qv_std=_INV_SQRT128, k_unit=True, alpha_mu=4.0,
                              stream_frames=64, ring=13, seed=3),
    "long_horizon": Workload("long_horizon", 1, 16, 336, 1560, 128, 128, torch.bfloat16,
                             window=3, taps=4, dilation=4, chunk=64,
                             qv_std=_INV_SQRT128, k_unit=True, alpha_mu=4.0, seed=4),
    "dilated_d6": Workload("dilated_d6", 1, 16, 61, 1560, 128, 128, torch.bfloat16,
                           window=3, taps=4, dilation=6, chunk=64,
                           qv_std=_INV_SQRT128, k_unit=True, alpha_mu=4.0, seed=5),
    "dilated_d12": Workload("dilated_d12", 1, 16, 61, 1560, 128, 128, torch.bfloat16,
                            window=3, taps=4, dilation=12, chunk=64,
                            qv_std=_INV_SQRT128, k_unit=True, alpha_mu=4.0, seed=6),
}


def _unit_rows(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def make_inputs(w: Workload, device="cpu", frames: int | None = None) -> dict:
    """Draw q, k, v [B,H,F*P,d] (storage dtype), alpha, beta [B,H,F*P] (fp32).

    F = frames if given, else T + stream_frames. Draws happen in fp32 on
    ``device`` from one generator seeded with ``w.seed`` and are rounded once
    to the storage dtype, so every consumer sees identical values.
    """
    F = (w.T + w.stream_frames) if frames is None else int(frames)
    n = F * w.P
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(w.seed))
    shp = (w.B, w.H, n)
    q = torch.randn(shp + (w.dk,), generator=g, device=dev, dtype=torch.float32)
    k = torch.randn(shp + (w.dk,), generator=g, device=dev, dtype=torch.float32)
    v = torch.randn(shp + (w.dv,), generator=g, device=dev, dtype=torch.float32)
    za = torch.randn(shp, generator=g, device=dev, dtype=torch.float32)
    zb = torch.randn(shp, generator=g, device=dev, dtype=torch.float32)
    q = _unit_rows(q) if w.q_unit else q * w.qv_std
    k = _unit_rows(k) if w.k_unit else k * w.k_std
    v = v * w.qv_std
    alpha = torch.sigmoid(za + w.alpha_mu)
    beta = torch.sigmoid(zb + w.beta_mu)
    return {
        "q": q.to(w.dtype).contiguous(),
        "k": k.to(w.dtype).contiguous(),
        "v": v.to(w.dtype).contiguous(),
        "alpha": alpha.contiguous(),
        "beta": beta.contiguous(),
        "frames": F,
    }


def make_output_grad(w: Workload, device="cpu", frames: int | None = None,
                     std: float = 1.0) -> torch.Tensor:
    """A seeded output gradient dL/do [B,H,F*P,dv] ~ N(0, std^2), drawn in fp32
    from its own generator (seed + 1000) and rounded once to the storage dtype:
    the input of a backward pass, standing in for the gradient a loss would send."""
    F = w.T if frames is None else int(frames)
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(w.seed) + 1000)
    d = torch.randn((w.B, w.H, F * w.P, w.dv), generator=g, device=dev, dtype=torch.float32)
    return (d * std).to(w.dtype).contiguous()
