"""GPU parity of the attention backward pass (hta_swa_bwd, hta_dswa_bwd, and
the log-sum-exp of hta_*_fwd_lse) against the fp64 oracle's gradients.

The GPU backward takes the GPU forward's own o and lse, as a training step
would; the oracle differentiates its exact forward. Inputs are seeded draws of
the workloads' distributions (q, k, v ~ N(0,1)/sqrt(d) for bf16 as in the
windowed-attention workload), with a seeded output gradient ~ N(0, 1).
Tolerance: max |gpu - oracle| <= tol * RMS(oracle) per tensor, tol 1e-4 for
fp32 and 2e-2 for bf16; bf16 gradients are written in bf16, so their check adds
the half-ulp of that one final rounding (as for the forward's bf16 outputs).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, assert_parity, assert_parity_rounded, f64
from hybrid_linear_temporal_hta_amd import hta
from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs, make_output_grad

pytestmark = pytest.mark.gpu


def _run(kind, x, dout, w, out_dtype):
    q, k, v = x["q"], x["k"], x["v"]
    B, H, L, d = q.shape
    o = torch.empty(B, H, L, d, dtype=out_dtype, device="cuda")
    lse = torch.empty(B, H, L, device="cuda")
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    if kind == "swa":
        hta.hta_swa_fwd_lse(q, k, v, o, lse, w.P, w.window)
        hta.hta_swa_bwd(q, k, v, o, lse, dout, dq, dk, dv, w.P, w.window)
    else:
        hta.hta_dswa_fwd_lse(q, k, v, o, lse, w.P, w.taps, w.dilation)
        hta.hta_dswa_bwd(q, k, v, o, lse, dout, dq, dk, dv, w.P, w.taps, w.dilation)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _case(base, kind, out_dtype, seed, **kw):
    w = WORKLOADS[base].replace(seed=seed, **kw)
    print(f"[case] attn bwd {kind} {w.name} B{w.B} H{w.H} T{w.T} P{w.P} d{w.dk} "
          f"W{w.window} taps{w.taps} dil{w.dilation} out {out_dtype}", flush=True)
    x = make_inputs(w, device="cuda", frames=w.T)
    dout = make_output_grad(w.replace(dtype=out_dtype), device="cuda")   # fp32: unrounded
    o, lse, dq, dk, dv = _run(kind, x, dout, w, out_dtype)
    q, k, v, do = f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(dout)   # the exact gradient
    if kind == "swa":
        ref = oracle.swa_bwd(q, k, v, do, w.T, w.P, w.window)
        lse_ref, _ = oracle.window_stats("swa", q, k, v, do, w.T, w.P, w.window, 0,
                                         np.arange(w.B * w.H * w.L))
    else:
        ref = oracle.dswa_bwd(q, k, v, do, w.T, w.P, w.taps, w.dilation)
        lse_ref, _ = oracle.window_stats("dswa", q, k, v, do, w.T, w.P, w.taps, w.dilation,
                                         np.arange(w.B * w.H * w.L))
    assert_parity(lse.reshape(-1), lse_ref, w.dtype, f"{kind} lse")
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        _grad_parity(g, r, w.dtype, f"{kind} {name}")


def _grad_parity(got, ref, dtype, what):
    if dtype == torch.bfloat16:
        assert_parity_rounded(got, ref, TOL[dtype], what)
    else:
        assert_parity(got, ref, dtype, what)


@pytest.mark.parametrize("kind", ["swa", "dswa"])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_attn_bwd_bf16_ragged(kind, out_dtype):
    """P = 200: query and key tiles with ragged tails (128-row workgroups, 64-row tiles)."""
    _case("swa_dswa_bf16", kind, out_dtype, seed=21, B=1, H=2, T=6, P=200, dilation=2)


@pytest.mark.parametrize("kind,T,P,window,taps,dil", [
    ("swa", 3, 64, 3, 4, 4),      # exact tiles, every frame short of a full window
    ("dswa", 9, 100, 3, 4, 2),    # missing taps in early frames
    ("swa", 4, 17, 2, 4, 4),      # one ragged tile per frame
    ("dswa", 13, 33, 3, 3, 6),    # dilation 6
    ("swa", 2, 1, 3, 4, 4),       # one token per frame
])
def test_attn_bwd_bf16_shapes(kind, T, P, window, taps, dil):
    _case("swa_dswa_bf16", kind, torch.float32, seed=22 + T, B=2, H=1, T=T, P=P, window=window,
          taps=taps, dilation=dil)


@pytest.mark.parametrize("kind", ["swa", "dswa"])
@pytest.mark.parametrize("d", [64, 128])
def test_attn_bwd_fp32(kind, d):
    _case("tiny_fp32", kind, torch.float32, seed=31, dk=d, dv=d, P=20, T=9)


@pytest.mark.slow
@pytest.mark.parametrize("kind", ["swa", "dswa"])
def test_attn_bwd_full_size_sampled(kind):
    """The windowed-attention workload (B2 H16 T21 P1560 bf16, fp32 o) in the
    launch configuration the benchmark times; dq on sampled query rows and
    dk, dv on sampled key rows of two key frames, against the oracle."""
    w = WORKLOADS["swa_dswa_bf16"]
    print(f"[case] attn bwd {kind} full size B{w.B} H{w.H} T{w.T} P{w.P}", flush=True)
    x = make_inputs(w, device="cuda", frames=w.T)
    dout = make_output_grad(w, device="cuda").to(torch.float32)
    o, lse, dq, dk, dv = _run(kind, x, dout, w, torch.float32)
    q, k, v = x["q"].cpu(), x["k"].cpu(), x["v"].cpu()
    do = f64(dout.to(torch.bfloat16))
    a, b = (w.window, 0) if kind == "swa" else (w.taps, w.dilation)
    rng = np.random.default_rng(5)
    L = w.L
    qrows = np.unique(np.concatenate([[0, 1559, 1560, L - 1, 31 * L + 20 * w.P + 1559],
                                      rng.integers(0, w.B * w.H * L, 120)]))
    ref_dq = oracle.window_dq_rows(kind, q, k, v, do, w.T, w.P, a, b, qrows)
    _grad_parity(dq.reshape(-1, 128)[torch.from_numpy(qrows).cuda()], ref_dq, w.dtype,
                 f"{kind} full-size dq (sampled rows)")
    # key rows in key frames 0 (every tap attends) and 19 (few attend), two heads
    krows = []
    for bh, kf in ((3, 0), (30, 19)):
        pos = np.unique(np.concatenate([[0, 63, 64, 127, 128, 1535, 1536, 1559],
                                        rng.integers(0, w.P, 8)]))
        krows += [bh * L + kf * w.P + p for p in pos]
    krows = np.array(krows)
    ref_dk, ref_dv = oracle.window_dkv_rows(kind, q, k, v, do, w.T, w.P, a, b, krows)
    idx = torch.from_numpy(krows).cuda()
    _grad_parity(dk.reshape(-1, 128)[idx], ref_dk, w.dtype, f"{kind} full-size dk (sampled rows)")
    _grad_parity(dv.reshape(-1, 128)[idx], ref_dv, w.dtype, f"{kind} full-size dv (sampled rows)")
