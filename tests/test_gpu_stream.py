"""GPU tests of the one-frame streaming step (ring-buffer K/V + carried GLA state).

Expected values come from the oracle evaluated on the WHOLE history (no ring):
SWA/DSWA rows of the new frame over every earlier frame, and the token-by-token
GLA recurrence over the full concatenated sequence. The ring itself must hold
exact copies of the last R frames.
"""
import numpy as np
import pytest
import torch

import oracle
from helpers import TOL, assert_parity, assert_parity_rounded, f64
from hybrid_linear_temporal_hta_amd import hta
from hybrid_linear_temporal_hta_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def _frames(full, P, n):
    sl = slice(n * P, (n + 1) * P)
    return {k: full[k][:, :, sl].contiguous() for k in ("q", "k", "v", "alpha", "beta")}


def _prefix(full, P, T0):
    return {k: full[k][:, :, :T0 * P].contiguous() for k in ("q", "k", "v", "alpha", "beta")}


def _start_stream(w, full, T0, prm, out_dtype=torch.float32):
    """Hybrid forward over the prefix, then a stream seeded with its K/V and state."""
    x = _prefix(full, w.P, T0)
    st0 = torch.zeros(w.B, w.H, w.dk, w.dv, device="cuda")
    o = torch.empty(w.B, w.H, T0 * w.P, w.dv, dtype=torch.float32, device="cuda")
    hta.hta_hybrid_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], st0, o, w.P, prm)
    s = hta.Stream(w.B, w.H, w.P, w.dk, w.dtype, prm, w.ring, out_dtype=out_dtype)
    hta.hta_stream_init(s, x["k"], x["v"], T0, st0)
    return s, o


def _run_and_check(w, T0, N, check_steps=None, rows=None, form=0, out_dtype=torch.float32,
                   side=False):
    """out_dtype: the steps' output dtype (bf16: the fp32 sum rounded once);
    side: a caller side stream in the context's params."""
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, gla_form=form,
                          side=hta.SideStream() if side else None)
    full = make_inputs(w, device="cuda", frames=T0 + N)
    s, _ = _start_stream(w, full, T0, prm, out_dtype)
    outs = {}
    for n in range(N):
        f = _frames(full, w.P, T0 + n)
        o = torch.empty(w.B, w.H, w.P, w.dv, dtype=out_dtype, device="cuda")
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], o)
        if check_steps is None or (n + 1) in check_steps:
            outs[n] = o
    torch.cuda.synchronize()
    assert s.n_frames == T0 + N
    # oracle on the whole history
    q, k, v = f64(full["q"]), f64(full["k"]), f64(full["v"])
    gla_ref = oracle.gla_literal if form == hta.HTA_GLA_PRINTED else oracle.gla
    ref_g, ref_st = gla_ref(q, k, v, full["alpha"], full["beta"])
    assert_parity(s.state, ref_st, w.dtype, f"stream final state after {N} steps")
    for n, o in outs.items():
        fr = T0 + n
        pos = np.arange(w.P) if rows is None else rows
        ref_att = oracle.stream_frame(k[:, :, :(fr + 1) * w.P], v[:, :, :(fr + 1) * w.P],
                                      q[:, :, fr * w.P:(fr + 1) * w.P], w.P, w.window, w.taps,
                                      w.dilation, rows=pos)
        ref = ref_att + ref_g[:, :, fr * w.P + pos]
        if out_dtype == torch.bfloat16:
            assert_parity_rounded(f64(o)[:, :, pos], ref, TOL[w.dtype],
                                  f"stream step {n + 1} (frame {fr}), bf16 out")
        else:
            assert_parity(f64(o)[:, :, pos], ref, w.dtype, f"stream step {n + 1} (frame {fr})")
    # ring holds exact copies of the last R frames
    last = T0 + N
    for fr in range(max(0, last - w.ring), last):
        slot = fr % w.ring
        assert torch.equal(s.ring_k[:, :, slot], full["k"][:, :, fr * w.P:(fr + 1) * w.P])
        assert torch.equal(s.ring_v[:, :, slot], full["v"][:, :, fr * w.P:(fr + 1) * w.P])
    return s


@pytest.mark.parametrize("dtype,out_dtype", [(torch.bfloat16, torch.float32),
                                             (torch.bfloat16, torch.bfloat16),
                                             (torch.float32, torch.float32)])
def test_stream_small(dtype, out_dtype):
    print(f"[case] stream small {dtype} out {out_dtype}", flush=True)
    w = Workload("case", 1, 2, 5, 150, 128, 128, dtype, window=3, taps=4, dilation=4, chunk=64,
                 k_unit=True, alpha_mu=3.0, ring=13, seed=41)
    _run_and_check(w, T0=5, N=14, out_dtype=out_dtype)


def test_stream_dilation_12_printed_form():
    """The pages' dilation of 12 frames (ring of 37 frames) with the printed GLA
    update: outputs of every step against the whole-history definition."""
    print("[case] stream dil 12, printed GLA form", flush=True)
    w = Workload("case", 1, 2, 30, 48, 128, 128, torch.bfloat16, window=3, taps=4, dilation=12,
                 chunk=64, k_unit=True, alpha_mu=2.0, ring=37, seed=45)
    _run_and_check(w, T0=30, N=10, form=hta.HTA_GLA_PRINTED)


def test_stream_farthest_tap():
    """The largest tap span (a 4095-frame dilation: 4096 frames) at P = 1 through a
    4096-frame ring, with a side stream: the DSWA tap of each step reads the slot
    written 4095 frames earlier (frame 4096's tap reads frame 1 after frame 4096 has
    replaced frame 0 in slot 0)."""
    print("[case] stream farthest tap: dil 4095, ring 4096, P 1", flush=True)
    w = Workload("case", 1, 2, 4094, 1, 128, 128, torch.bfloat16, window=1, taps=2, dilation=4095,
                 q_unit=True, k_unit=True, ring=4096, seed=46)
    _run_and_check(w, T0=4094, N=4, side=True)


@pytest.mark.slow
def test_stream_ring_offsets_beyond_2_31():
    """A ring of 4097 frames at B2 H16 P128 holds 2 148 007 936 elements per tensor,
    more than 2^31, so the last head's slots sit past 2^31; with a 4095-frame dilation
    each step's DSWA tap reads a slot 4095 frames back. Side stream. The oracle checks
    the last head: both steps' outputs from the whole history and its final state;
    the ring must hold that head's frames exactly."""
    w = Workload("case", 2, 16, 4096, 128, 128, 128, torch.bfloat16, window=1, taps=2,
                 dilation=4095, q_unit=True, k_unit=True, ring=4097, seed=47)
    T0, N = w.T, 2
    assert w.B * w.H * w.ring * w.P * w.dk > 2 ** 31
    print(f"[case] stream ring beyond 2^31: B{w.B} H{w.H} P{w.P} ring {w.ring}", flush=True)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk, side=hta.SideStream())
    full = make_inputs(w, device="cuda", frames=T0 + N)
    torch.cuda.empty_cache()
    s, o_prefix = _start_stream(w, full, T0, prm)
    del o_prefix
    torch.cuda.empty_cache()
    b_, h_ = w.B - 1, w.H - 1
    outs = []
    for n in range(N):
        f = _frames(full, w.P, T0 + n)
        o = torch.empty(w.B, w.H, w.P, w.dv, device="cuda")
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], o)
        outs.append(o[b_, h_].clone())
    torch.cuda.synchronize()
    assert s.n_frames == T0 + N
    last = T0 + N
    for fr in (0, 1, last - 2, last - 1):   # slots of the oldest and the newest frames
        if fr < last - w.ring:
            continue
        slot = fr % w.ring
        sl = slice(fr * w.P, (fr + 1) * w.P)
        assert torch.equal(s.ring_k[b_, h_, slot], full["k"][b_, h_, sl])
        assert torch.equal(s.ring_v[b_, h_, slot], full["v"][b_, h_, sl])
    st_gpu = f64(s.state[b_:b_ + 1, h_:h_ + 1])
    head = {n: f64(full[n][b_:b_ + 1, h_:h_ + 1]) for n in ("q", "k", "v", "alpha", "beta")}
    del s, full
    torch.cuda.empty_cache()
    ref_g, ref_st = oracle.gla(head["q"], head["k"], head["v"], head["alpha"], head["beta"])
    assert_parity(st_gpu, ref_st, w.dtype, "last head's state after the steps")
    for n, o in enumerate(outs):
        fr = T0 + n
        ref_att = oracle.stream_frame(head["k"][:, :, :(fr + 1) * w.P], head["v"][:, :, :(fr + 1) * w.P],
                                      head["q"][:, :, fr * w.P:(fr + 1) * w.P], w.P, w.window,
                                      w.taps, w.dilation)
        ref = ref_att + ref_g[:, :, fr * w.P:(fr + 1) * w.P]
        assert_parity(f64(o)[None, None], ref, w.dtype, f"last head, step {n + 1} (frame {fr})")


def test_stream_from_empty_prefix():
    """A stream started with no prefix: early frames see only the taps that exist."""
    print("[case] stream from empty prefix", flush=True)
    w = Workload("case", 1, 2, 1, 70, 128, 128, torch.bfloat16, window=3, taps=4, dilation=2,
                 k_unit=True, ring=7, seed=42)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    N = 9
    full = make_inputs(w, device="cuda", frames=N)
    s = hta.Stream(w.B, w.H, w.P, w.dk, w.dtype, prm, w.ring)
    hta.hta_stream_init(s, None, None, 0, None)
    outs = []
    for n in range(N):
        f = _frames(full, w.P, n)
        o = torch.empty(w.B, w.H, w.P, w.dv, dtype=torch.float32, device="cuda")
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], o)
        outs.append(o)
    torch.cuda.synchronize()
    q, k, v = f64(full["q"]), f64(full["k"]), f64(full["v"])
    ref_o, ref_st, _ = oracle.hybrid(q, k, v, full["alpha"], full["beta"], N, w.P, w.window,
                                     w.taps, w.dilation)
    got = torch.cat(outs, dim=2)
    assert_parity(got, ref_o, w.dtype, "stream from empty == batch definition")
    assert_parity(s.state, ref_st, w.dtype, "stream from empty state")


@pytest.mark.parametrize("out_dtype,side", [(torch.float32, False), (torch.bfloat16, False),
                                           (torch.bfloat16, True)])
def test_stream_step_wide_grid(out_dtype, side):
    """A stream step whose attention grid spans more than one wave of workgroups
    (B4 H16 P1040: 64 heads x 9 query tiles = 576 workgroups, over two per CU on
    256 CUs), with fp32 or bf16 output, on one stream or with the attention on a
    caller side stream: sampled rows of two steps against the oracle on the whole
    history, the final state and the ring."""
    print(f"[case] stream step, wide grid B4 H16 P1040, out {out_dtype}, side {side}", flush=True)
    w = Workload("case", 4, 16, 4, 1040, 128, 128, torch.bfloat16, window=3, taps=4, dilation=4,
                 k_unit=True, alpha_mu=3.0, ring=13, seed=47)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.array([0, 1, 127, 128, 1023, 1024, 1039]),
                                     rng.integers(0, w.P, 40)]))
    _run_and_check(w, 4, 2, rows=rows, out_dtype=out_dtype, side=side)


def test_stream_equals_batch_and_commit_only():
    """I9: stream steps reproduce the batch hybrid over prefix + frames (GPU vs
    GPU, different chunk boundaries, so within tolerance); commit-only steps
    advance the state exactly like full steps."""
    print("[case] stream == batch, commit-only", flush=True)
    w = Workload("case", 1, 2, 4, 200, 128, 128, torch.bfloat16, window=3, taps=4, dilation=4,
                 k_unit=True, alpha_mu=3.0, ring=13, seed=43)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    T0, N = 4, 10
    full = make_inputs(w, device="cuda", frames=T0 + N)
    s, _ = _start_stream(w, full, T0, prm)
    s2, _ = _start_stream(w, full, T0, prm)
    outs = []
    for n in range(N):
        f = _frames(full, w.P, T0 + n)
        o = torch.empty(w.B, w.H, w.P, w.dv, dtype=torch.float32, device="cuda")
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], o)
        hta.hta_stream_step(s2, f["q"], f["k"], f["v"], f["alpha"], f["beta"], None)
        outs.append(o)
    st_b = torch.zeros(w.B, w.H, w.dk, w.dv, device="cuda")
    ob = torch.empty(w.B, w.H, (T0 + N) * w.P, w.dv, dtype=torch.float32, device="cuda")
    hta.hta_hybrid_fwd(full["q"], full["k"], full["v"], full["alpha"], full["beta"], st_b, ob,
                       w.P, prm)
    torch.cuda.synchronize()
    ref = ob[:, :, T0 * w.P:]
    assert_parity(torch.cat(outs, dim=2), ref, w.dtype, "stream vs batch outputs")
    assert_parity(s.state, st_b, w.dtype, "stream vs batch state")
    assert torch.equal(s.state, s2.state), "commit-only state differs from full-step state"
    assert torch.equal(s.ring_k, s2.ring_k) and torch.equal(s.ring_v, s2.ring_v)


def test_stream_checkpoint_resume_bitwise():
    """The ring, the state and n_frames are the whole resumable memory: a copy
    continued in a fresh context gives bitwise identical outputs."""
    print("[case] stream checkpoint/resume", flush=True)
    w = Workload("case", 1, 2, 3, 100, 128, 128, torch.bfloat16, window=3, taps=4, dilation=4,
                 k_unit=True, ring=13, seed=44)
    prm = hta.make_params(w.window, w.taps, w.dilation, w.chunk)
    T0, N, K = 3, 12, 6
    full = make_inputs(w, device="cuda", frames=T0 + N)
    s, _ = _start_stream(w, full, T0, prm)
    for n in range(K):
        f = _frames(full, w.P, T0 + n)
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], None)
    torch.cuda.synchronize()
    ck = (s.ring_k.cpu(), s.ring_v.cpu(), s.state.cpu(), s.n_frames)
    r = hta.Stream(w.B, w.H, w.P, w.dk, w.dtype, prm, w.ring)
    r.ring_k.copy_(ck[0]); r.ring_v.copy_(ck[1]); r.state.copy_(ck[2]); r.ctx.n_frames = ck[3]
    for n in range(K, N):
        f = _frames(full, w.P, T0 + n)
        oa = torch.empty(w.B, w.H, w.P, w.dv, dtype=torch.float32, device="cuda")
        ob = torch.empty_like(oa)
        hta.hta_stream_step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], oa)
        hta.hta_stream_step(r, f["q"], f["k"], f["v"], f["alpha"], f["beta"], ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), f"resumed stream differs at step {n}"
    assert torch.equal(s.state, r.state)


@pytest.mark.slow
def test_stream_full_size_sampled():
    """The streaming workload at full size: prefix of 21 frames (hybrid forward),
    then 64 steps of 1560 tokens (B2 H16, ring of 13). Final state against the
    full recurrence over 85 frames; outputs of steps 1, 2, 32, 63, 64 on sampled
    rows; the ring against the last 13 frames."""
    w = WORKLOADS["hybrid_stream"]
    print(f"[case] full-size stream {w.name}", flush=True)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(1500, w.P),
                                     np.random.default_rng(5).integers(0, w.P, 60)]))
    _run_and_check(w, T0=w.T, N=w.stream_frames, check_steps={1, 2, 32, 63, 64}, rows=rows)
