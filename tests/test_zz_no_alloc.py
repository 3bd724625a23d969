"""hta_stream_step_noalloc (the library's fixed per-GPU scratch, no workspace
argument) against hta_stream_step (a caller workspace), through the C ABI.

Both run the same kernels, so outputs, the carried state and the ring must be
equal bit for bit. The no-allocation calls run back to back, the later ones on
smaller inputs, so each finds the previous call's contents in the scratch; the
reference workspace is filled with 0xFF bytes (NaN as fp32 / bf16) before use.
Neither may depend on what the memory held. A commit-only step (o = NULL) sits
between the output steps.
"""
import pytest
import torch

from hybrid_linear_temporal_hta_amd import hta
from hybrid_linear_temporal_hta_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu

# (B, H, P, dtype, out_dtype, side stream, prefix frames, steps), largest first:
# the first needs 108.8 MiB of the 128 MiB scratch.
CASES = [
    (2, 16, 1560, torch.bfloat16, torch.bfloat16, True, 4, 3),
    (1, 2, 300, torch.bfloat16, torch.float32, False, 14, 3),
    (1, 2, 100, torch.float32, torch.float32, False, 6, 3),
]


def _workload(B, H, P, dtype, T0, N, seed):
    return Workload("noalloc", B, H, T0 + N, P, 128, 128, dtype, window=3, taps=4, dilation=4,
                    chunk=64, k_unit=True, alpha_mu=3.0, ring=13, seed=seed)


def _steps(case, noalloc, seed):
    B, H, P, dtype, out_dtype, side, T0, N = case
    w = _workload(B, H, P, dtype, T0, N, seed)
    full = make_inputs(w, device="cuda", frames=T0 + N)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    state0 = 0.5 * torch.randn(B, H, 128, 128, generator=g, device="cuda")
    prm = hta.make_params(w.window, w.taps, w.dilation, 64,
                          side=hta.SideStream() if side else None)
    s = hta.Stream(B, H, P, 128, dtype, prm, w.ring, out_dtype=out_dtype)
    if not noalloc:
        s.workspace.fill_(255)
    hta.hta_stream_init(s, full["k"][:, :, :T0 * P].contiguous(),
                        full["v"][:, :, :T0 * P].contiguous(), T0, state0)
    step = hta.hta_stream_step_noalloc if noalloc else hta.hta_stream_step
    outs = []
    for n in range(N):
        sl = slice((T0 + n) * P, (T0 + n + 1) * P)
        f = {k: full[k][:, :, sl].contiguous() for k in ("q", "k", "v", "alpha", "beta")}
        o = None if n == 1 else torch.empty(B, H, P, 128, dtype=out_dtype, device="cuda")
        step(s, f["q"], f["k"], f["v"], f["alpha"], f["beta"], o)
        if o is not None:
            outs.append(o)
    torch.cuda.synchronize()
    assert s.n_frames == T0 + N
    return outs, s.state, s.ring_k, s.ring_v


def test_stream_step_noalloc_matches_workspace_step():
    got = []
    for i, case in enumerate(CASES):
        print(f"[case] noalloc stream step B{case[0]} H{case[1]} P{case[2]} {case[3]} "
              f"out {case[4]} side {case[5]}", flush=True)
        got.append(_steps(case, True, 60 + i))
    for i, case in enumerate(CASES):
        print(f"[case] workspace stream step B{case[0]} H{case[1]} P{case[2]}", flush=True)
        ref = _steps(case, False, 60 + i)
        outs, state, rk, rv = got[i]
        for n, (a, b) in enumerate(zip(outs, ref[0])):
            assert torch.equal(a, b), f"case {i} output {n}"
        assert torch.equal(state, ref[1]), f"case {i} state"
        assert torch.equal(rk, ref[2]) and torch.equal(rv, ref[3]), f"case {i} ring"
        assert all(torch.isfinite(o.float()).all() for o in outs), f"case {i} non-finite"


def test_stream_step_noalloc_rejects_oversized_step():
    """A step needing more than the fixed scratch returns HTA_ERR_SCRATCH and
    leaves the context as it was."""
    prm = hta.make_params(3, 4, 4, 64)
    s = hta.Stream(4, 16, 16, 128, torch.bfloat16, prm, 13)
    s.ctx.s.P = 4096   # the context claims a frame of 4096 tokens; nothing is launched
    assert hta.hta_workspace_bytes(hta.HTA_OP_STREAM_STEP, s.ctx.s, prm) > \
        hta.HTA_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    a = torch.zeros(16, device="cuda")
    with pytest.raises(hta.HTAError) as e:
        hta.hta_stream_step_noalloc(s, x, x, x, a, a, None)
    assert e.value.status == hta.HTA_ERR_SCRATCH
    assert s.n_frames == 0
