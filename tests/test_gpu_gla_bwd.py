"""GPU parity of the GLA backward pass (hta_gla_bwd) against the oracle's
gradients (token-by-token reverse recurrence in fp64), for both update forms,
with a non-zero initial state and a non-zero gradient of the final state.

Inputs follow the GLA workloads: unit-norm q, k, v ~ N(0, 1), alpha =
sigmoid(N(mu, 1)), beta = sigmoid(N(0, 1)), and a seeded output gradient.
Tolerance: max |gpu - oracle| <= tol * RMS(oracle) per tensor (1e-4 fp32,
2e-2 bf16 plus the half-ulp of bf16 outputs).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, assert_parity, assert_parity_rounded, f64
from hybrid_linear_temporal_hta_amd import hta
from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, Workload, make_inputs, make_output_grad

pytestmark = pytest.mark.gpu


def _case(w, form, out_dtype=torch.float32, seed_state=5):
    print(f"[case] gla bwd {w.name} B{w.B} H{w.H} L{w.L} d{w.dk} {w.dtype} form{form}", flush=True)
    x = make_inputs(w, device="cuda", frames=w.T)
    dout = make_output_grad(w.replace(dtype=out_dtype), device="cuda")   # fp32: unrounded
    g = torch.Generator(device="cuda")
    g.manual_seed(seed_state)
    s0 = 0.3 * torch.randn(w.B, w.H, w.dk, w.dv, generator=g, device="cuda")
    dsf = torch.randn(w.B, w.H, w.dk, w.dv, generator=g, device="cuda")
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    da, db = torch.empty_like(a), torch.empty_like(b)
    dst = dsf.clone()
    prm = hta.make_params(chunk=w.chunk, gla_form=form)
    hta.hta_gla_bwd(q, k, v, a, b, s0, dout, dst, dq, dk, dv, da, db, w.P, prm)
    torch.cuda.synchronize()
    do = f64(dout)
    ref = oracle.gla_bwd(f64(q), f64(k), f64(v), f64(a), f64(b), do, f64(s0), f64(dsf),
                         form=form)
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        if w.dtype == torch.bfloat16:
            assert_parity_rounded(got, ref[name], TOL[w.dtype], f"gla {name}")
        else:
            assert_parity(got, ref[name], w.dtype, f"gla {name}")
    assert_parity(da, ref["dalpha"], w.dtype, "gla dalpha")
    assert_parity(db, ref["dbeta"], w.dtype, "gla dbeta")
    assert_parity(dst, ref["dstate0"], w.dtype, "gla dstate0")


@pytest.mark.parametrize("form", [0, 1])
def test_gla_bwd_fp32_tiny(form):
    _case(WORKLOADS["tiny_fp32"], form)


@pytest.mark.parametrize("form", [0, 1])
def test_gla_bwd_fp32_d128_ragged(form):
    w = WORKLOADS["tiny_fp32"].replace(dk=128, dv=128, T=3, P=50, seed=7)   # L = 150
    _case(w, form)


@pytest.mark.parametrize("form", [0, 1])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_gla_bwd_bf16_ragged(form, out_dtype):
    """bf16 chunked path: L = 200 (three full chunks and a ragged fourth)."""
    w = WORKLOADS["gla_bf16"].replace(B=1, H=2, T=4, P=50, seed=8)
    _case(w, form, out_dtype)


@pytest.mark.parametrize("form", [0, 1])
def test_gla_bwd_bf16_long(form):
    """bf16 chunked path over 31 chunks with a ragged tail and gates as in the
    GLA workload (alpha = sigmoid(N(4, 1)))."""
    w = WORKLOADS["gla_bf16"].replace(B=2, H=4, T=13, P=151, seed=9)   # L = 1963
    _case(w, form, torch.float32)


@pytest.mark.parametrize("form", [0, 1])
def test_gla_bwd_deterministic(form):
    """hta_gla_bwd is bitwise reproducible (per-wave partial row sums in a fixed
    order; no float atomics)."""
    w = Workload("det", 1, 2, 3, 150, 128, 128, torch.bfloat16, chunk=64, k_unit=True,
                 alpha_mu=3.0, seed=48)
    print(f"[case] gla bwd determinism form {form}", flush=True)
    x = make_inputs(w, device="cuda", frames=w.T)
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    s0 = 0.5 * torch.randn(w.B, w.H, 128, 128, generator=g, device="cuda")
    dsf = torch.randn(w.B, w.H, 128, 128, generator=g, device="cuda")
    dout = make_output_grad(w.replace(dtype=torch.float32), device="cuda")
    prm = hta.make_params(chunk=64, gla_form=form)
    runs = []
    for _ in range(3):
        gr = [torch.empty_like(t) for t in (q, k, v, a, b)]
        dst = dsf.clone()
        hta.hta_gla_bwd(q, k, v, a, b, s0, dout, dst, *gr, w.P, prm)
        runs.append(gr + [dst])
    torch.cuda.synchronize()
    for r in runs[1:]:
        for name, x0, x1 in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate0"), runs[0], r):
            assert torch.equal(x0, x1), f"{name} differs between identical calls"
