"""Pins of the oracle's backward pass (gradients of SWA, DSWA, GLA, hybrid).

The backward rules in oracle.c are the chain rule written out by hand. They are
pinned to things other than themselves:
  - central finite differences of the (separately pinned) forward oracle, in
    fp64, on tiny inputs, for every input element: a dropped term, a wrong
    sign, a transposed operand or a wrong index in any rule fails here;
  - for attention, torch's autograd of scaled_dot_product_attention with the
    block mask of the window (a library routine for the same function);
  - closed forms and invariants: softmax shift invariance (the key gradients
    of one (b, h) slice sum to zero), the value gradients summing to the
    output gradients, the identity attention of a one-token window, and the
    GLA special case beta = 0 (pure decay of the initial state);
  - the sampled-row routines against the full backward.

Sources: [P1] Kairos paper-read (yingwang.github.io), section 二、方法: SWA /
DSWA / GLA paragraphs and the GLA update equations define the forward whose
gradient this is.
"""
import numpy as np
import pytest
import torch

import oracle


def _fd(fun, x, h=1e-6):
    """Central differences of scalar fun() with respect to every entry of x."""
    g = np.zeros_like(x)
    flat, gf = x.reshape(-1), g.reshape(-1)
    for i in range(flat.size):
        x0 = flat[i]
        flat[i] = x0 + h
        fp = fun()
        flat[i] = x0 - h
        fm = fun()
        flat[i] = x0
        gf[i] = (fp - fm) / (2 * h)
    return g


def _attn_inputs(seed, B=1, H=2, T=5, P=3, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    L = T * P
    return (rng.standard_normal((B, H, L, dk)), rng.standard_normal((B, H, L, dk)),
            rng.standard_normal((B, H, L, dv)), rng.standard_normal((B, H, L, dv)))


def _gla_inputs(seed, B=1, H=1, L=150, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, L, d)) for d in (dk, dk, dv, dv))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, (B, H, L))))
    b = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, (B, H, L))))
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.5
    dsf = rng.standard_normal((B, H, dk, dv))
    return q, k, v, do, a, b, s0, dsf


@pytest.mark.parametrize("kind,a,b", [("swa", 3, 0), ("dswa", 3, 2), ("dswa", 2, 3)])
def test_window_bwd_matches_finite_differences(kind, a, b):
    T, P = 5, 3
    q, k, v, do = _attn_inputs(1)
    if kind == "swa":
        fwd = lambda: float(np.sum(oracle.swa(q, k, v, T, P, a) * do))
        got = oracle.swa_bwd(q, k, v, do, T, P, a)
    else:
        fwd = lambda: float(np.sum(oracle.dswa(q, k, v, T, P, a, b) * do))
        got = oracle.dswa_bwd(q, k, v, do, T, P, a, b)
    for name, x, g in zip(("dq", "dk", "dv"), (q, k, v), got):
        num = _fd(fwd, x)
        assert np.max(np.abs(num - g)) < 1e-7 * max(1.0, np.max(np.abs(g))), name


def _mask(T, P, frames_of):
    L = T * P
    m = np.zeros((L, L), dtype=bool)
    for f in range(T):
        for kf in frames_of(f):
            m[f * P:(f + 1) * P, kf * P:(kf + 1) * P] = True
    return m


@pytest.mark.parametrize("kind", ["swa", "dswa"])
def test_window_bwd_matches_torch_autograd_of_masked_sdpa(kind):
    T, P, dk, dv = 7, 4, 8, 5
    q, k, v, do = _attn_inputs(2, B=2, H=2, T=T, P=P, dk=dk, dv=dv)
    if kind == "swa":
        W = 3
        mask = _mask(T, P, lambda f: [f - j for j in range(W) if f - j >= 0])
        got = oracle.swa_bwd(q, k, v, do, T, P, W)
    else:
        taps, dil = 3, 2
        mask = _mask(T, P, lambda f: [f - j * dil for j in range(taps) if f - j * dil >= 0])
        got = oracle.dswa_bwd(q, k, v, do, T, P, taps, dil)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv,
                                                           attn_mask=torch.from_numpy(mask))
    out.backward(torch.from_numpy(do))
    for name, t, g in zip(("dq", "dk", "dv"), (tq, tk, tv), got):
        np.testing.assert_allclose(g, t.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


@pytest.mark.parametrize("kind", ["swa", "dswa"])
def test_window_bwd_invariants(kind):
    """Adding one vector to every key leaves each row's softmax unchanged, so
    the key gradients of a (b, h) slice sum to zero; each row's probabilities
    sum to one, so the value gradients sum to the output gradients."""
    T, P = 6, 5
    q, k, v, do = _attn_inputs(3, B=2, H=3, T=T, P=P, dk=6, dv=4)
    dq, dk_, dv_ = (oracle.swa_bwd(q, k, v, do, T, P, 3) if kind == "swa"
                    else oracle.dswa_bwd(q, k, v, do, T, P, 4, 2))
    np.testing.assert_allclose(dk_.sum(axis=2), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv_.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)
    assert np.max(np.abs(dq)) > 1e-3


def test_window_bwd_one_token_window_is_identity():
    """P = 1, window 1: every query sees only its own key, o = v, so dv = dO
    and the q, k gradients vanish."""
    T, P = 9, 1
    q, k, v, do = _attn_inputs(4, T=T, P=P)
    dq, dk_, dv_ = oracle.swa_bwd(q, k, v, do, T, P, 1)
    np.testing.assert_array_equal(dv_, do)
    assert np.max(np.abs(dq)) < 1e-15 and np.max(np.abs(dk_)) < 1e-15


def test_window_stats_lse_is_logsumexp():
    T, P, W = 6, 4, 3
    q, k, v, do = _attn_inputs(5, B=1, H=1, T=T, P=P, dk=8, dv=8)
    rows = np.arange(T * P)
    lse, D = oracle.window_stats("swa", q, k, v, do, T, P, W, 0, rows)
    o = oracle.swa(q, k, v, T, P, W)
    s = 1 / np.sqrt(8)
    for t in rows:
        f = t // P
        keys = np.arange(max(0, f - W + 1) * P, (f + 1) * P)
        z = s * (k[0, 0, keys] @ q[0, 0, t])
        assert abs(lse[t] - float(torch.logsumexp(torch.from_numpy(z), 0))) < 1e-12
        assert abs(D[t] - do[0, 0, t] @ o[0, 0, t]) < 1e-12


@pytest.mark.parametrize("kind,a,b", [("swa", 3, 0), ("dswa", 4, 2)])
def test_window_row_routines_match_full_backward(kind, a, b):
    T, P = 7, 6
    q, k, v, do = _attn_inputs(6, B=2, H=2, T=T, P=P, dk=8, dv=8)
    full = (oracle.swa_bwd(q, k, v, do, T, P, a) if kind == "swa"
            else oracle.dswa_bwd(q, k, v, do, T, P, a, b))
    rows = np.array([0, 5, 6, 17, 41, 42 + 3, 84 + 40, 3 * 42 - 1])
    dq = oracle.window_dq_rows(kind, q, k, v, do, T, P, a, b, rows)
    dkr, dvr = oracle.window_dkv_rows(kind, q, k, v, do, T, P, a, b, rows)
    np.testing.assert_allclose(dq, full[0].reshape(-1, 8)[rows], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dkr, full[1].reshape(-1, 8)[rows], rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(dvr, full[2].reshape(-1, 8)[rows], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("form", [0, 1])
def test_gla_bwd_matches_finite_differences(form):
    """L = 150 spans two checkpoint segments of 64 tokens and a ragged third;
    non-zero initial state and final-state gradient."""
    q, k, v, do, a, b, s0, dsf = _gla_inputs(7)
    fn = oracle.gla if form == 0 else oracle.gla_literal

    def loss():
        o, st = fn(q, k, v, a, b, s0)
        return float(np.sum(o * do) + np.sum(st * dsf))

    got = oracle.gla_bwd(q, k, v, a, b, do, s0, dsf, form=form)
    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", a), ("dbeta", b),
                    ("dstate0", s0)):
        num = _fd(loss, x)
        assert np.max(np.abs(num - got[name])) < 1e-6 * max(1.0, np.max(np.abs(got[name]))), name


def test_gla_bwd_scale_and_zero_final_gradient():
    """gla_scale multiplies the output; with no final-state gradient every
    gradient scales with it linearly."""
    q, k, v, do, a, b, s0, _ = _gla_inputs(8, L=40)
    g1 = oracle.gla_bwd(q, k, v, a, b, do, s0, None, scale=1.0)
    g2 = oracle.gla_bwd(q, k, v, a, b, do, s0, None, scale=2.5)
    for name in g1:
        np.testing.assert_allclose(g2[name], 2.5 * g1[name], rtol=1e-12, atol=1e-12)


def test_gla_bwd_zero_write_strength_closed_form():
    """beta = 0: the state only decays, M_t = (prod_{r<=t} alpha_r) M_0 and
    o_t = c_t M_0^T q_t with c_t that product. Hence dq_t = c_t M_0 dO_t,
    dk = dv = 0, and dalpha_t = sum_{t'>=t} c_t' / alpha_t * q_t'^T M_0 dO_t'."""
    q, k, v, do, a, _, s0, _ = _gla_inputs(9, L=30, dk=4, dv=3)
    b = np.zeros_like(a)
    g = oracle.gla_bwd(q, k, v, a, b, do, s0)
    c = np.cumprod(a[0, 0])
    M0 = s0[0, 0]
    dq = c[:, None] * (do[0, 0] @ M0.T)
    np.testing.assert_allclose(g["dq"][0, 0], dq, rtol=1e-12, atol=1e-13)
    assert np.max(np.abs(g["dk"])) == 0.0 and np.max(np.abs(g["dv"])) == 0.0
    term = c * np.einsum("ti,ij,tj->t", q[0, 0], M0, do[0, 0])
    dal = np.cumsum(term[::-1])[::-1] / a[0, 0]
    np.testing.assert_allclose(g["dalpha"][0, 0], dal, rtol=1e-11, atol=1e-13)
    dst0 = np.einsum("t,ti,tj->ij", c, q[0, 0], do[0, 0])
    np.testing.assert_allclose(g["dstate0"][0, 0], dst0, rtol=1e-11, atol=1e-13)


def test_hybrid_bwd_is_sum_of_branches_and_matches_finite_differences():
    T, P, W, taps, dil = 5, 2, 3, 3, 2
    q, k, v, do = _attn_inputs(10, B=1, H=1, T=T, P=P, dk=3, dv=3)
    rng = np.random.default_rng(11)
    a = 1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, q.shape[:3])))
    b = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, q.shape[:3])))
    g = oracle.hybrid_bwd(q, k, v, a, b, do, T, P, W, taps, dil)

    def loss():
        return float(np.sum(oracle.hybrid(q, k, v, a, b, T, P, W, taps, dil)[0] * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", a), ("dbeta", b)):
        num = _fd(loss, x)
        assert np.max(np.abs(num - g[name])) < 1e-7 * max(1.0, np.max(np.abs(g[name]))), name
