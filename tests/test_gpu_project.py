"""GPU parity of the per-token projections and gates (hta_project_fwd) against
the fp64 oracle (oracle/project.py) on the same seeded bf16 inputs.

q, k, v are written in bf16, so they are compared with the bf16 tolerance plus
one output rounding; alpha and beta are fp32 outputs of bf16 inputs.
"""
import numpy as np
import pytest
import torch

from helpers import TOL, assert_parity, assert_parity_rounded, f64
from hybrid_linear_temporal_hta_amd import hta
from oracle.project import project

pytestmark = pytest.mark.gpu


def _inputs(B, L, Dm, H, seed):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    N = 3 * H * 128 + 2 * H
    x = torch.randn(B, L, Dm, generator=g, device="cuda").to(torch.bfloat16)
    w = (torch.randn(Dm, N, generator=g, device="cuda") / Dm ** 0.5).to(torch.bfloat16)
    return x, w


def _run(x, w, B, L, H, P, flags):
    q, k, v = (torch.empty(B, H, L, 128, dtype=torch.bfloat16, device="cuda") for _ in range(3))
    al, be = (torch.empty(B, H, L, device="cuda") for _ in range(2))
    hta.hta_project_fwd(x, w, q, k, v, al, be, P, flags)
    torch.cuda.synchronize()
    return q, k, v, al, be


def _check(got, ref, what):
    tol = TOL[torch.bfloat16]
    for name, g, r in zip(("q", "k", "v"), got[:3], ref[:3]):
        assert_parity_rounded(g, r, tol, f"{what} {name}")
    for name, g, r in zip(("alpha", "beta"), got[3:], ref[3:]):
        assert_parity(g, r, torch.bfloat16, f"{what} {name}")


@pytest.mark.parametrize("B,T,P,H,Dm,flags", [
    (1, 3, 50, 4, 256, hta.HTA_NORM_Q | hta.HTA_NORM_K),   # ragged token tail
    (2, 2, 50, 8, 128, hta.HTA_NORM_K),                    # a token tile across the batch edge
    (1, 1, 1, 4, 64, 0),                                   # one token, no normalisation
    (3, 5, 77, 16, 512, hta.HTA_NORM_Q | hta.HTA_NORM_K),  # gate tile of 32 columns
])
def test_project_parity(B, T, P, H, Dm, flags):
    print(f"[case] project B{B} T{T} P{P} H{H} Dm{Dm} flags{flags}", flush=True)
    L = T * P
    x, w = _inputs(B, L, Dm, H, seed=B * 100 + L + H)
    got = _run(x, w, B, L, H, P, flags)
    ref = project(f64(x), f64(w), H, 128, 128, bool(flags & 1), bool(flags & 2))
    _check(got, ref, "project")


def test_project_zero_token_stays_zero():
    B, T, P, H, Dm = 1, 2, 64, 4, 128
    x, w = _inputs(B, T * P, Dm, H, seed=7)
    x[0, 5] = 0
    q, k, v, al, be = _run(x, w, B, T * P, H, P, hta.HTA_NORM_Q | hta.HTA_NORM_K)
    assert torch.all(q[0, :, 5] == 0) and torch.all(k[0, :, 5] == 0) and torch.all(v[0, :, 5] == 0)
    assert torch.all(al[0, :, 5] == 0.5) and torch.all(be[0, :, 5] == 0.5)


@pytest.mark.slow
def test_project_full_size_sampled():
    """The workload's shape (B2 H16, L = 21 x 1560, model width 2048) in the
    launch configuration the benchmark times; sampled tokens against the oracle,
    including both ends of each sequence and the tile edges."""
    B, T, P, H, Dm = 2, 21, 1560, 16, 2048
    L = T * P
    print(f"[case] project full size B{B} L{L} H{H} Dm{Dm}", flush=True)
    x, w = _inputs(B, L, Dm, H, seed=11)
    got = _run(x, w, B, L, H, P, hta.HTA_NORM_Q | hta.HTA_NORM_K)
    rng = np.random.default_rng(12)
    toks = np.unique(np.concatenate([[0, 1, 127, 128, L - 129, L - 128, L - 1],
                                     rng.integers(0, L, 200)]))
    xs = f64(x[:, toks])                                      # [B, n, Dm]
    ref = project(xs, f64(w), H, 128, 128, True, True)
    sub = [t[:, :, toks] for t in got]
    _check(sub, ref, "project full-size sampled")


@pytest.mark.slow
def test_project_offsets_beyond_2_31():
    """B2 L525720 H16 at model width 2048: x and each of q, k, v hold 2.15e9 elements,
    more than 2^31; sampled tokens (the sequence's last ones, where batch 1's offsets
    pass 2^31, and both tile edges) against the oracle."""
    B, T, P, H, Dm = 2, 337, 1560, 16, 2048
    L = T * P
    assert B * L * Dm > 2 ** 31 and B * H * L * 128 > 2 ** 31
    print(f"[case] project offsets beyond 2^31: B{B} L{L} H{H} Dm{Dm}", flush=True)
    x, w = _inputs(B, L, Dm, H, seed=13)
    torch.cuda.empty_cache()
    got = _run(x, w, B, L, H, P, hta.HTA_NORM_Q | hta.HTA_NORM_K)
    rng = np.random.default_rng(14)
    toks = np.unique(np.concatenate([[0, 127, 128, L - 129, L - 128, L - 1],
                                     rng.integers(L - 40000, L, 120)]))
    xs = f64(x[:, toks])
    ref = project(xs, f64(w), H, 128, 128, True, True)
    sub = [t[:, :, toks] for t in got]
    _check(sub, ref, "project beyond 2^31 sampled")
