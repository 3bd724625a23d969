"""GPU parity of the hybrid layer's training pair (hta_hybrid_fwd_train,
hta_hybrid_bwd) against the oracle: the forward output equals hta_hybrid_fwd's,
and the gradients of o = o_swa + o_dswa + o_gla (dq, dk, dv summed over the
branches, dalpha, dbeta, dL/dM_0) match the oracle's exact gradients.

Inputs: the hybrid workload's distributions (q, v ~ N(0,1)/sqrt(d), unit-norm
k, alpha = sigmoid(N(4, 1)), beta = sigmoid(N(0, 1))), a seeded output
gradient ~ N(0, 1), a non-zero initial state and final-state gradient.
Tolerance: max |gpu - oracle| <= tol * RMS(oracle) (1e-4 fp32, 2e-2 bf16 plus
the half-ulp of bf16 outputs).
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, assert_parity, assert_parity_rounded, f64
from hybrid_linear_temporal_hta_amd import hta
from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, make_inputs, make_output_grad

pytestmark = pytest.mark.gpu


def _run(w, x, dout, s0, dsf, prm, out_dtype):
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    B, H, L, d = q.shape
    st = s0.clone()
    o = torch.empty(B, H, L, d, dtype=out_dtype, device="cuda")
    shape = hta.make_shape(q, v, w.P, o)
    saved = torch.empty(hta.hta_hybrid_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    hta.hta_hybrid_fwd_train(q, k, v, a, b, st, o, saved, w.P, prm)
    st2 = s0.clone()
    o2 = torch.empty_like(o)
    hta.hta_hybrid_fwd(q, k, v, a, b, st2, o2, w.P, prm)
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    da, db = torch.empty_like(a), torch.empty_like(b)
    dst = dsf.clone()
    hta.hta_hybrid_bwd(q, k, v, a, b, saved, dout, dst, dq, dk, dv, da, db, w.P, prm)
    torch.cuda.synchronize()
    # inference sums both attention branches in one pass (the training forward keeps
    # them apart to save each): same results up to rounding order
    if o.dtype == torch.bfloat16:
        assert_parity_rounded(o, f64(o2), TOL[w.dtype], "fwd_train vs fwd output")
    else:
        assert_parity(o, f64(o2), w.dtype, "fwd_train vs fwd output")
    assert torch.equal(st, st2), "final states differ"
    return dict(dq=dq, dk=dk, dv=dv, dalpha=da, dbeta=db, dstate0=dst)


def _inputs(w, out_dtype):
    """dL/do in the output dtype: an fp32 one is drawn unrounded (the bf16 kernels
    round it themselves; the oracle differentiates the exact values)."""
    x = make_inputs(w, device="cuda", frames=w.T)
    dout = make_output_grad(w.replace(dtype=out_dtype), device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 77)
    s0 = 0.3 * torch.randn(w.B, w.H, w.dk, w.dv, generator=g, device="cuda")
    dsf = torch.randn(w.B, w.H, w.dk, w.dv, generator=g, device="cuda")
    return x, dout, s0, dsf


def _check(got, ref, dtype, what):
    for name in ("dq", "dk", "dv"):
        if dtype == torch.bfloat16:
            assert_parity_rounded(got[name], ref[name], TOL[dtype], f"{what} {name}")
        else:
            assert_parity(got[name], ref[name], dtype, f"{what} {name}")
    for name in ("dalpha", "dbeta", "dstate0"):
        assert_parity(got[name], ref[name], dtype, f"{what} {name}")


@pytest.mark.parametrize("side", [False, True])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("form", [0, 1])
def test_hybrid_bwd_bf16(out_dtype, form, side):
    """side: the caller's side stream in params (the attention work beside the GLA
    work), which must give the same results."""
    w = WORKLOADS["hybrid_stream"].replace(B=1, H=2, T=9, P=70, stream_frames=0, dilation=2,
                                           seed=41)
    print(f"[case] hybrid bwd B{w.B} H{w.H} T{w.T} P{w.P} form{form} out {out_dtype} side {side}",
          flush=True)
    x, dout, s0, dsf = _inputs(w, out_dtype)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, gla_form=form,
                          side=hta.SideStream() if side else None)
    got = _run(w, x, dout, s0, dsf, prm, out_dtype)
    do = f64(dout)
    ref = oracle.hybrid_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                            f64(x["beta"]), do, w.T, w.P, w.window, w.taps, w.dilation,
                            f64(s0), f64(dsf), form=form)
    _check(got, ref, w.dtype, "hybrid")


@pytest.mark.parametrize("T,P,window,taps,dil", [(20, 40, 16, 16, 1), (4100, 1, 1, 2, 4095)])
def test_hybrid_bwd_at_limits(T, P, window, taps, dil):
    """The training pair at the largest window and tap count, and at the largest tap
    span (4096 frames, P = 1), with a side stream, against the oracle's gradients."""
    w = WORKLOADS["hybrid_stream"].replace(B=1, H=2, T=T, P=P, stream_frames=0, window=window,
                                           taps=taps, dilation=dil, seed=51)
    print(f"[case] hybrid bwd limits T{T} P{P} W{window} taps{taps} dil{dil}", flush=True)
    x, dout, s0, dsf = _inputs(w, torch.float32)
    prm = hta.make_params(window, taps, dil, w.chunk, side=hta.SideStream())
    got = _run(w, x, dout, s0, dsf, prm, torch.float32)
    ref = oracle.hybrid_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                            f64(x["beta"]), f64(dout), T, P, window, taps, dil, f64(s0), f64(dsf))
    _check(got, ref, w.dtype, "hybrid at limits")


def test_hybrid_bwd_fp32():
    w = WORKLOADS["tiny_fp32"]
    print(f"[case] hybrid bwd {w.name}", flush=True)
    x, dout, s0, dsf = _inputs(w, torch.float32)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    got = _run(w, x, dout, s0, dsf, prm, torch.float32)
    ref = oracle.hybrid_bwd(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(x["alpha"]),
                            f64(x["beta"]), f64(dout), w.T, w.P, w.window, w.taps, w.dilation,
                            f64(s0), f64(dsf))
    _check(got, ref, w.dtype, "hybrid fp32")


@pytest.mark.slow
def test_hybrid_bwd_full_size_sampled():
    """The hybrid workload (B2 H16 T21 P1560, bf16 in, fp32 out) in the launch
    configuration the benchmark times. For two (b, h) slices: the GLA
    gradients over the whole sequence, and dq / dk / dv on sampled rows (the
    attention part from the oracle's row routines plus the GLA part)."""
    w = WORKLOADS["hybrid_stream"].replace(stream_frames=0)
    print(f"[case] hybrid bwd full size B{w.B} H{w.H} T{w.T} P{w.P}", flush=True)
    x, dout, s0, dsf = _inputs(w, torch.float32)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    got = _run(w, x, dout, s0, dsf, prm, torch.float32)
    q, k, v = x["q"].cpu(), x["k"].cpu(), x["v"].cpu()
    do = f64(dout)
    L = w.L
    rng = np.random.default_rng(3)
    for b_, h_ in ((0, 3), (1, 14)):
        bh = b_ * w.H + h_
        sl = (slice(b_, b_ + 1), slice(h_, h_ + 1))
        print(f"[case] oracle GLA backward of (b, h) = ({b_}, {h_})", flush=True)
        g = oracle.gla_bwd(f64(q[sl]), f64(k[sl]), f64(v[sl]), f64(x["alpha"][sl]),
                           f64(x["beta"][sl]), do[sl], f64(s0[sl]), f64(dsf[sl]))
        for name in ("dalpha", "dbeta", "dstate0"):
            assert_parity(got[name][sl], g[name], w.dtype, f"full-size {name} (b,h)=({b_},{h_})")
        pos = np.unique(np.concatenate([[0, 1559, 1560, L - 1], rng.integers(0, L, 24)]))
        rows = bh * L + pos
        att_dq = sum(oracle.window_dq_rows(kind, q, k, v, do, w.T, w.P, a, dd, rows)
                     for kind, a, dd in (("swa", w.window, 0), ("dswa", w.taps, w.dilation)))
        kv = [oracle.window_dkv_rows(kind, q, k, v, do, w.T, w.P, a, dd, rows)
              for kind, a, dd in (("swa", w.window, 0), ("dswa", w.taps, w.dilation))]
        att_dk, att_dv = kv[0][0] + kv[1][0], kv[0][1] + kv[1][1]
        for name, att in (("dq", att_dq), ("dk", att_dk), ("dv", att_dv)):
            ref = att + g[name][0, 0, pos]
            assert_parity_rounded(got[name][b_, h_, torch.from_numpy(pos).cuda()], ref,
                                  TOL[w.dtype], f"full-size {name} sampled rows (b,h)=({b_},{h_})")


@pytest.mark.slow
def test_hybrid_bwd_offsets_beyond_2_31():
    """The training pair at B2 H16 T337 P1560 (L = 525720): each sequence tensor holds
    2 153 349 120 elements, more than 2^31; the last head's last 31 frames lie past
    2^31. For that head's last 14 frames: the GLA gradients (the oracle's forward
    over the frames before gives the state entering them, its backward over them the
    exact gradients of their tokens) and dq / dk / dv of the last two frames (the
    attention part from the oracle's row routines over those 14 frames)."""
    w = WORKLOADS["long_horizon"].replace(B=2, T=337, seed=6)
    assert w.B * w.H * w.L * w.dk > 2 ** 31
    print(f"[case] hybrid bwd offsets beyond 2^31: B{w.B} H{w.H} T{w.T} P{w.P}", flush=True)
    x, dout, s0, dsf = _inputs(w, torch.float32)
    torch.cuda.empty_cache()   # the draws' fp32 temporaries (the backward needs ~160 GB)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=hta.SideStream())
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    o = torch.empty(w.B, w.H, w.L, w.dv, device="cuda")
    saved = torch.empty(hta.hta_hybrid_saved_bytes(hta.make_shape(q, v, w.P, o)),
                        dtype=torch.uint8, device="cuda")
    hta.hta_hybrid_fwd_train(q, k, v, a, b, s0.clone(), o, saved, w.P, prm)
    torch.cuda.synchronize()
    del o
    torch.cuda.empty_cache()   # the forward's workspace
    dq, dk, dv = (torch.empty_like(t) for t in (q, k, v))
    da, db = torch.empty_like(a), torch.empty_like(b)
    hta.hta_hybrid_bwd(q, k, v, a, b, saved, dout, dsf.clone(), dq, dk, dv, da, db, w.P, prm)
    torch.cuda.synchronize()
    got = dict(dq=dq, dk=dk, dv=dv, dalpha=da, dbeta=db)
    del saved, q, k, v, a, b, dq, dk, dv, da, db
    b_, h_ = w.B - 1, w.H - 1
    nt = 14                                   # frames checked: the last taps reach 12 back
    t0 = (w.T - nt) * w.P
    head = {n: f64(x[n][b_:b_ + 1, h_:h_ + 1]) for n in ("q", "k", "v", "alpha", "beta")}
    do = f64(dout[b_:b_ + 1, h_:h_ + 1])
    got = {n: t[b_, h_].cpu() for n, t in got.items()}
    del x, dout
    torch.cuda.empty_cache()
    print("[case] oracle GLA forward to the checked frames, backward over them", flush=True)
    _, st_mid = oracle.gla(*(head[n][:, :, :t0] for n in ("q", "k", "v", "alpha", "beta")),
                           f64(s0[b_:b_ + 1, h_:h_ + 1]))
    tail = {n: head[n][:, :, t0:] for n in head}
    g = oracle.gla_bwd(tail["q"], tail["k"], tail["v"], tail["alpha"], tail["beta"],
                       do[:, :, t0:], st_mid, f64(dsf[b_:b_ + 1, h_:h_ + 1]))
    for name in ("dalpha", "dbeta"):
        assert_parity(got[name][t0:], g[name][0, 0], w.dtype, f"tail {name}")
    pos = np.arange((nt - 2) * w.P, nt * w.P)   # the last two frames, within the tail
    q, k, v = tail["q"], tail["k"], tail["v"]
    att_dq = sum(oracle.window_dq_rows(kind, q, k, v, do[:, :, t0:], nt, w.P, a, dd, pos)
                 for kind, a, dd in (("swa", w.window, 0), ("dswa", w.taps, w.dilation)))
    kv = [oracle.window_dkv_rows(kind, q, k, v, do[:, :, t0:], nt, w.P, a, dd, pos)
          for kind, a, dd in (("swa", w.window, 0), ("dswa", w.taps, w.dilation))]
    att_dk, att_dv = kv[0][0] + kv[1][0], kv[0][1] + kv[1][1]
    for name, att in (("dq", att_dq), ("dk", att_dk), ("dv", att_dv)):
        ref = att + g[name][0, 0, pos]
        assert_parity_rounded(got[name][t0 + pos], ref, TOL[w.dtype], f"last two frames {name}")


@pytest.mark.parametrize("side", [False, True])
def test_hybrid_bwd_deterministic(side):
    """The training pair is bitwise reproducible: two backward calls on the same
    saved activations give identical gradients (no order-dependent reductions:
    the GLA gradient's row sums are per-wave partials summed in a fixed order)."""
    w = WORKLOADS["hybrid_stream"].replace(B=1, H=2, T=7, P=130, stream_frames=0, seed=46)
    print(f"[case] hybrid bwd determinism B{w.B} H{w.H} T{w.T} P{w.P} side {side}", flush=True)
    x, dout, s0, dsf = _inputs(w, torch.float32)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk,
                          side=hta.SideStream() if side else None)
    q, k, v, a, b = x["q"], x["k"], x["v"], x["alpha"], x["beta"]
    o = torch.empty(w.B, w.H, w.L, w.dv, device="cuda")
    st = s0.clone()
    shape = hta.make_shape(q, v, w.P, o)
    saved = torch.empty(hta.hta_hybrid_saved_bytes(shape), dtype=torch.uint8, device="cuda")
    hta.hta_hybrid_fwd_train(q, k, v, a, b, st, o, saved, w.P, prm)
    runs = []
    for _ in range(3):
        g = [torch.empty_like(t) for t in (q, k, v, a, b)]
        dst = dsf.clone()
        hta.hta_hybrid_bwd(q, k, v, a, b, saved, dout, dst, *g, w.P, prm)
        runs.append(g + [dst])
    torch.cuda.synchronize()
    for r in runs[1:]:
        for name, x0, x1 in zip(("dq", "dk", "dv", "dalpha", "dbeta", "dstate0"), runs[0], r):
            assert torch.equal(x0, x1), f"{name} differs between identical calls"
