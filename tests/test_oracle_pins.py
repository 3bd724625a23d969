"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Every test here runs the oracle alone (no GPU). Each one is chosen so that a
plausible slip in the oracle (wrong window edge, zero-padded dilation taps,
causal mask inside a frame, missing softmax scale, transposed state, dropped
forget gate on the erase term, wrong sign) fails at least one of them.

Sources: [P1] Kairos paper-read (yingwang.github.io), section 二、方法:
SWA / DSWA / GLA paragraphs, GLA update equations, Theorem 2 (contraction);
[P2] ai-papers.net Kairos article, 誤差蓄積の理論的保証 (geometric decay).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.gla_chunked import gla_chunked
from oracle.project import project

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _frac(x):
    return np.array(np.vectorize(lambda s: float(Fraction(s)))(np.array(x, dtype=object)),
                    dtype=np.float64)


def _rand_attn(seed, B=2, H=2, T=7, P=5, dk=8, dv=6, std=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T * P, dk)) * std
    k = rng.standard_normal((B, H, T * P, dk)) * std
    v = rng.standard_normal((B, H, T * P, dv))
    return q, k, v


def _rand_gla(seed, B=2, H=2, L=37, dk=8, dv=6, amu=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, L, dk))
    k = rng.standard_normal((B, H, L, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, L, dv))
    a = 1.0 / (1.0 + np.exp(-(rng.standard_normal((B, H, L)) + amu)))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, L))))
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    return q, k, v, a, b, s0


def _sdpa(q, k, v, mask, scale=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    out = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=torch.from_numpy(mask), scale=scale)
    return out.numpy()


def _block_mask(T, P, lo_frames):
    """Boolean [L, L] mask: query frame f sees key frames f-lo_frames+1 .. f (all tokens)."""
    f = np.arange(T * P) // P
    d = f[:, None] - f[None, :]
    return (d >= 0) & (d < lo_frames)


# ---------------------------------------------------------------- golden, by hand

def test_golden_window_one_token_frames():
    g = json.load(open(os.path.join(GOLDEN, "window_tiny_worked.json")))["case_a"]
    T, P = g["T"], g["P"]
    q = _frac(g["q"]).reshape(1, 1, T, 1)
    k = np.log(_frac(g["k_exp"])).reshape(1, 1, T, 1)
    v = _frac(g["v"]).reshape(1, 1, T, 1)
    o_s = oracle.swa(q, k, v, T, P, 2, scale=1.0)
    o_d = oracle.dswa(q, k, v, T, P, 2, 2, scale=1.0)
    np.testing.assert_allclose(o_s.ravel(), _frac(g["swa_window2"]), rtol=1e-14)
    np.testing.assert_allclose(o_d.ravel(), _frac(g["dswa_taps2_dil2"]), rtol=1e-14)


def test_golden_window_full_inside_frame():
    g = json.load(open(os.path.join(GOLDEN, "window_tiny_worked.json")))["case_b"]
    T, P = g["T"], g["P"]
    z = np.zeros((1, 1, T * P, 1))
    v = _frac(g["v"]).reshape(1, 1, T * P, 1)
    np.testing.assert_allclose(oracle.swa(z, z, v, T, P, 1, 1.0).ravel(), _frac(g["swa_window1"]),
                               rtol=1e-14)
    np.testing.assert_allclose(oracle.swa(z, z, v, T, P, 2, 1.0).ravel(), _frac(g["swa_window2"]),
                               rtol=1e-14)


@pytest.mark.parametrize("form", ["gdn", "literal"])
def test_golden_gla_worked_example(form):
    g = json.load(open(os.path.join(GOLDEN, "gla_d2_worked.json")))
    q = _frac(g["q"]).reshape(1, 1, 3, 2)
    k = _frac(g["k"]).reshape(1, 1, 3, 2)
    v = _frac(g["v"]).reshape(1, 1, 3, 2)
    a = _frac(g["alpha"]).reshape(1, 1, 3)
    b = _frac(g["beta"]).reshape(1, 1, 3)
    fn = oracle.gla if form == "gdn" else oracle.gla_literal
    o, st = fn(q, k, v, a, b)
    np.testing.assert_allclose(o.reshape(3, 2), _frac(g["o_" + form]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st.reshape(2, 2), _frac(g["state_%s_dk_dv" % form]),
                               rtol=0, atol=1e-14)
    # the chunked closed form, in both readings, reaches the same hand values
    oc, sc = gla_chunked(q, k, v, a, b, chunk=2, literal=(form == "literal"))
    np.testing.assert_allclose(oc.reshape(3, 2), _frac(g["o_" + form]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(sc.reshape(2, 2), _frac(g["state_%s_dk_dv" % form]),
                               rtol=0, atol=1e-14)


# ---------------------------------------------------------------- SWA / DSWA

def test_swa_whole_sequence_window_is_block_causal_sdpa():
    """I2: a window covering every frame equals full block-causal attention."""
    T, P = 6, 4
    q, k, v = _rand_attn(1, T=T, P=P)
    o = oracle.swa(q, k, v, T, P, window=T + 3)
    ref = _sdpa(q, k, v, _block_mask(T, P, T))     # default scale 1/sqrt(dk)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window", [1, 2, 3])
def test_swa_matches_sdpa_block_mask(window):
    """I2: window W equals SDPA with the frame-block mask of width W (W=1: per-frame)."""
    T, P = 7, 5
    q, k, v = _rand_attn(2, T=T, P=P)
    o = oracle.swa(q, k, v, T, P, window)
    np.testing.assert_allclose(o, _sdpa(q, k, v, _block_mask(T, P, window)),
                               rtol=1e-12, atol=1e-13)


def test_swa_explicit_scale_is_used():
    T, P = 4, 3
    q, k, v = _rand_attn(3, T=T, P=P)
    o = oracle.swa(q, k, v, T, P, 2, scale=0.37)
    np.testing.assert_allclose(o, _sdpa(q, k, v, _block_mask(T, P, 2), scale=0.37),
                               rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("taps", [1, 3, 4])
def test_dswa_dilation_one_is_swa(taps):
    """I1: DSWA with dilation 1 is SWA with window = taps."""
    T, P = 9, 3
    q, k, v = _rand_attn(4, T=T, P=P)
    np.testing.assert_allclose(oracle.dswa(q, k, v, T, P, taps, 1),
                               oracle.swa(q, k, v, T, P, taps), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("T,taps,dil", [(12, 3, 3), (21, 4, 4), (10, 4, 2), (7, 4, 6)])
def test_dswa_is_swa_on_interleaved_relayout(T, taps, dil):
    """I3: the page's re-layout (B, F*L, D) -> (B*d, F/d*L, D): frame f goes to
    group f mod d at position f // d; SWA with window = taps inside each group,
    then the inverse re-layout, equals DSWA. Groups may be ragged (F % d != 0)."""
    P = 3
    q, k, v = _rand_attn(5, B=1, H=2, T=T, P=P)
    o = oracle.dswa(q, k, v, T, P, taps, dil)
    ref = np.empty_like(o)
    for grp in range(dil):
        frames = np.arange(grp, T, dil)
        idx = (frames[:, None] * P + np.arange(P)[None, :]).ravel()
        Tg = frames.size
        sub = _sdpa(q[:, :, idx], k[:, :, idx], v[:, :, idx], _block_mask(Tg, P, taps))
        ref[:, :, idx] = sub
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_window_rows_match_full():
    T, P = 8, 4
    q, k, v = _rand_attn(6, T=T, P=P)
    rows = np.array([0, 3, 17, 31, 64, 95, 127])
    np.testing.assert_allclose(oracle.swa_rows(q, k, v, T, P, 3, rows),
                               oracle.swa(q, k, v, T, P, 3).reshape(-1, v.shape[3])[rows],
                               rtol=0, atol=0)
    np.testing.assert_allclose(oracle.dswa_rows(q, k, v, T, P, 3, 2, rows),
                               oracle.dswa(q, k, v, T, P, 3, 2).reshape(-1, v.shape[3])[rows],
                               rtol=0, atol=0)


def test_window_outputs_in_convex_hull():
    """I11: softmax weights are a probability vector over the window's keys."""
    T, P = 6, 4
    q, k, v = _rand_attn(7, T=T, P=P, std=3.0)
    for fn, args in ((oracle.swa, (3,)), (oracle.dswa, (3, 2))):
        o = fn(q, k, v, T, P, *args)
        assert np.all(o <= v.max(axis=2, keepdims=True) + 1e-12)
        assert np.all(o >= v.min(axis=2, keepdims=True) - 1e-12)
    # frame 0 with window 1 only mixes frame-0 values
    o = oracle.swa(q, k, v, T, P, 1)
    assert np.all(o[:, :, :P] <= v[:, :, :P].max(axis=2, keepdims=True) + 1e-12)


# ---------------------------------------------------------------- GLA

def test_gla_beta_zero_keeps_zero_state():
    """I4: beta = 0 and S0 = 0: nothing is written, outputs and state are zero."""
    q, k, v, a, b, _ = _rand_gla(10)
    o, st = oracle.gla(q, k, v, a, np.zeros_like(b))
    assert np.all(o == 0) and np.all(st == 0)


@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("literal", [False, True])
def test_gla_recurrence_equals_chunked_closed_form(chunk, literal):
    """I5: token recurrence == chunked closed form (ragged last chunk, S0 != 0)."""
    q, k, v, a, b, s0 = _rand_gla(11, L=203, dk=8, dv=6)
    fn = oracle.gla_literal if literal else oracle.gla
    o1, st1 = fn(q, k, v, a, b, s0)
    o2, st2 = gla_chunked(q, k, v, a, b, chunk, s0, literal=literal)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(st1, st2, rtol=1e-11, atol=1e-12)


def test_gla_pure_decay_closed_form():
    """I7: alpha == a, beta == 0: o_t = a^(t+1) S0 q_t and S_L = a^L S0."""
    q, k, v, _, b, s0 = _rand_gla(12, L=19)
    a = np.full(b.shape, 0.9)
    o, st = oracle.gla(q, k, v, a, np.zeros_like(b), s0)
    L = q.shape[2]
    for t in range(L):
        # o_t = S_t q_t with S_t = a^(t+1) S0 ; in [dk][dv] storage that is q_t^T M
        exp = 0.9 ** (t + 1) * np.einsum("bhi,bhij->bhj", q[:, :, t], s0)
        np.testing.assert_allclose(o[:, :, t], exp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st, 0.9 ** L * s0, rtol=1e-12)


def test_gla_exact_recall_orthonormal_keys():
    """I8: alpha = beta = 1, S0 = 0, orthonormal keys: after writing, S k_j = v_j.
    Reading the state as S^T ([dk][dv]): k_j^T M = v_j. A transposed state or a
    left-multiplied erase would break this."""
    rng = np.random.default_rng(13)
    d, n = 8, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm[:, :n].T.reshape(1, 1, n, d)
    v = rng.standard_normal((1, 1, n, 5))
    q = k.copy()                       # o_t = S_t k_t = v_t at its own write
    ones = np.ones((1, 1, n))
    o, st = oracle.gla(q, k, v, ones, ones)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)
    recall = np.einsum("ti,ij->tj", k[0, 0], st[0, 0])
    np.testing.assert_allclose(recall, v[0, 0], rtol=0, atol=1e-13)


def test_gla_forms_agree_when_no_forgetting():
    """With alpha = 1 the GatedDeltaNet reading and the printed three-line form
    are the same update, so the oracle's beta handling is pinned to the page."""
    q, k, v, _, b, s0 = _rand_gla(14, L=41)
    ones = np.ones_like(b)
    o1, s1 = oracle.gla(q, k, v, ones, b, s0)
    o2, s2 = oracle.gla_literal(q, k, v, ones, b, s0)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-13)
    # and with forgetting they differ (the reading matters)
    q, k, v, a, b, s0 = _rand_gla(14, L=41)
    o3, _ = oracle.gla(q, k, v, a, b, s0)
    o4, _ = oracle.gla_literal(q, k, v, a, b, s0)
    assert np.abs(o3 - o4).max() > 1e-3


def test_gla_perturbation_decays_geometrically():
    """I6 (Theorem 2's contraction): perturbing v_s by delta changes o_t (t >= s) by at
    most (prod_{r=s+1..t} alpha_r) * beta_s * |delta| * |q_t| for unit keys, and
    leaves o_t (t < s) untouched."""
    q, k, v, a, b, s0 = _rand_gla(15, B=1, H=3, L=60, amu=0.5)
    o, _ = oracle.gla(q, k, v, a, b, s0)
    s = 17
    delta = np.random.default_rng(16).standard_normal(v.shape[3])
    v2 = v.copy()
    v2[:, :, s] += delta
    o2, _ = oracle.gla(q, k, v2, a, b, s0)
    d = np.linalg.norm(o2 - o, axis=-1)             # [B,H,L]
    assert np.all(d[:, :, :s] == 0)
    L = q.shape[2]
    for t in range(s, L):
        decay = np.prod(a[:, :, s + 1:t + 1], axis=-1)
        bound = decay * b[:, :, s] * np.linalg.norm(delta) * np.linalg.norm(q[:, :, t], axis=-1)
        assert np.all(d[:, :, t] <= bound * (1 + 1e-9) + 1e-14)
    # the bound is not vacuous: the effect at s itself is the bound (rank-one write)
    bnd_s = b[:, :, s] * np.linalg.norm(delta) * np.abs(np.einsum("bhi,bhi->bh", k[:, :, s],
                                                                    q[:, :, s]))
    np.testing.assert_allclose(d[:, :, s], bnd_s, rtol=1e-10)


def test_gla_literal_form_is_not_a_contraction_when_beta_exceeds_two_alpha():
    """The same bound fails for the printed form when beta > 2 alpha (erase not gated),
    which is why the contraction property selects the GatedDeltaNet reading."""
    L, d = 12, 4
    k = np.zeros((1, 1, L, d)); k[..., 0] = 1.0      # the same unit key every step
    q = k.copy()
    v = np.zeros((1, 1, L, 3))
    a = np.full((1, 1, L), 0.3)
    b = np.full((1, 1, L), 1.0)
    delta = np.array([1.0, 0.0, 0.0])
    v2 = v.copy(); v2[:, :, 0] += delta
    for fn, ok in ((oracle.gla, True), (oracle.gla_literal, False)):
        d0 = np.linalg.norm(fn(q, k, v2, a, b)[0] - fn(q, k, v, a, b)[0], axis=-1)[0, 0]
        bound = 0.3 ** np.arange(L)                   # prod of alphas since s=0
        assert bool(np.all(d0 <= bound * (1 + 1e-12))) == ok


def test_linearity_in_v_all_branches():
    """I10: every branch is linear in v (softmax weights and the gated delta
    transition depend on q, k, alpha, beta only); with S0 = 0 GLA is linear too."""
    T, P = 5, 4
    q, k, v1 = _rand_attn(20, T=T, P=P)
    _, _, v2 = _rand_attn(21, T=T, P=P)
    lam, mu = 0.7, -1.3
    for fn, args in ((oracle.swa, (2,)), (oracle.dswa, (3, 2))):
        np.testing.assert_allclose(fn(q, k, lam * v1 + mu * v2, T, P, *args),
                                   lam * fn(q, k, v1, T, P, *args) + mu * fn(q, k, v2, T, P, *args),
                                   rtol=1e-11, atol=1e-12)
    qg, kg, _, a, b, _ = _rand_gla(22, L=T * P, dv=v1.shape[3])
    og = lambda vv: oracle.gla(qg, kg, vv, a, b)[0]
    np.testing.assert_allclose(og(lam * v1 + mu * v2), lam * og(v1) + mu * og(v2),
                               rtol=1e-11, atol=1e-12)


def test_heads_and_batch_are_independent():
    """I12: permuting (batch, head) slices permutes every branch output."""
    T, P = 5, 3
    q, k, v = _rand_attn(23, B=2, H=3, T=T, P=P)
    qg, kg, vg, a, b, s0 = _rand_gla(24, B=2, H=3, L=T * P)
    perm_b, perm_h = [1, 0], [2, 0, 1]
    pb = lambda x: x[perm_b][:, perm_h]
    np.testing.assert_array_equal(oracle.swa(pb(q), pb(k), pb(v), T, P, 2),
                                  pb(oracle.swa(q, k, v, T, P, 2)))
    o, st = oracle.gla(qg, kg, vg, a, b, s0)
    o2, st2 = oracle.gla(pb(qg), pb(kg), pb(vg), pb(a), pb(b), pb(s0))
    np.testing.assert_array_equal(o2, pb(o))
    np.testing.assert_array_equal(st2, pb(st))


def test_gla_state_carry_splits_sequence():
    """Running GLA over [0, n) then [n, L) from the carried state equals one run
    over [0, L): the state is the complete memory (what the stream step carries)."""
    q, k, v, a, b, s0 = _rand_gla(25, L=50)
    o, st = oracle.gla(q, k, v, a, b, s0)
    n = 23
    oa, sa = oracle.gla(q[:, :, :n], k[:, :, :n], v[:, :, :n], a[:, :, :n], b[:, :, :n], s0)
    ob, sb = oracle.gla(q[:, :, n:], k[:, :, n:], v[:, :, n:], a[:, :, n:], b[:, :, n:], sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sb, st, rtol=1e-13, atol=1e-14)


def test_stream_frame_from_history_equals_batch_rows():
    """The oracle's streaming attention (whole history, no ring) is the batch
    definition restricted to the newest frame."""
    T, P = 15, 3
    q, k, v = _rand_attn(26, T=T, P=P)
    o_b = oracle.swa(q, k, v, T, P, 3) + oracle.dswa(q, k, v, T, P, 4, 4)
    for n in (0, 5, 14):
        hk, hv = k[:, :, :(n + 1) * P], v[:, :, :(n + 1) * P]
        o_s = oracle.stream_frame(hk, hv, q[:, :, n * P:(n + 1) * P], P, 3, 4, 4)
        np.testing.assert_allclose(o_s, o_b[:, :, n * P:(n + 1) * P], rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- projections

def test_golden_projection_worked_example():
    """Hand-worked single token: column order q | k | v | alpha | beta, the L2
    normalisation of q and k, and sigmoid(0) = 1/2 for both gates."""
    g = json.load(open(os.path.join(GOLDEN, "project_tiny_worked.json")))
    x = np.array([[[float(_frac(a)) for a in g["x"][0]]]])
    w = np.array([[float(_frac(a)) for a in row] for row in g["w_rows"]])
    q, k, v, al, be = project(x, w, H=1, dk=2, dv=2)
    fx = lambda key: np.array([[float(_frac(a)) for a in row] for row in g[key]])
    assert np.allclose(q[0, 0], fx("q"), atol=1e-15, rtol=0)
    assert np.allclose(k[0, 0], fx("k"), atol=1e-15, rtol=0)
    assert np.allclose(v[0, 0], fx("v"), atol=1e-15, rtol=0)
    assert al[0, 0, 0] == 0.5 and be[0, 0, 0] == 0.5
    q2, k2, *_ = project(x, w, H=1, dk=2, dv=2, norm_q=False, norm_k=False)
    assert np.allclose(q2[0, 0], fx("q_raw"), atol=1e-15, rtol=0)
    assert np.allclose(k2[0, 0], fx("k_raw"), atol=1e-15, rtol=0)


def _rand_proj(seed, B=2, L=9, Dm=16, H=3, dk=4, dv=5):
    r = np.random.default_rng(seed)
    x = r.standard_normal((B, L, Dm))
    w = r.standard_normal((Dm, 2 * H * dk + H * dv + 2 * H)) / np.sqrt(Dm)
    return x, w, H, dk, dv


def test_projection_gate_special_values():
    """sigmoid at 0, at ln 3 (exactly 3/4) and its symmetry, through the gate columns."""
    x = np.array([[[0.0], [np.log(3.0)], [-np.log(3.0)]]])          # B=1, L=3, Dm=1
    w = np.zeros((1, 2 * 1 * 1 + 1 + 2))                             # H=1, dk=dv=1
    w[0, 3] = 1.0                                                    # alpha column
    w[0, 4] = -1.0                                                   # beta column
    _, _, _, al, be = project(x, w, H=1, dk=1, dv=1)
    assert np.allclose(al[0, 0], [0.5, 0.75, 0.25], atol=1e-15, rtol=0)
    assert np.allclose(be[0, 0], [0.5, 0.25, 0.75], atol=1e-15, rtol=0)


def test_projection_unit_norm_and_zero_rows():
    x, w, H, dk, dv = _rand_proj(1)
    x[0, 3] = 0.0                                                     # a zero token
    q, k, v, al, be = project(x, w, H, dk, dv)
    n = np.sqrt((q * q).sum(-1))
    assert np.allclose(np.delete(n, 3, axis=2), 1.0, atol=1e-14)
    assert np.all(q[0, :, 3] == 0) and np.all(k[0, :, 3] == 0)
    assert np.all((al > 0) & (al < 1)) and np.all((be > 0) & (be < 1))


def test_projection_linear_before_normalisation_and_token_local():
    """Without normalisation q, k, v are linear in x, and each token's outputs
    depend only on that token (permuting tokens permutes every output)."""
    x, w, H, dk, dv = _rand_proj(2)
    x2 = np.random.default_rng(3).standard_normal(x.shape)
    a = project(2.0 * x - 0.5 * x2, w, H, dk, dv, False, False)
    b = project(x, w, H, dk, dv, False, False)
    c = project(x2, w, H, dk, dv, False, False)
    for i in range(3):
        assert np.allclose(a[i], 2.0 * b[i] - 0.5 * c[i], atol=1e-12)
    perm = np.random.default_rng(4).permutation(x.shape[1])
    p = project(x[:, perm], w, H, dk, dv)
    base = project(x, w, H, dk, dv)
    for i in range(3):
        assert np.allclose(p[i], base[i][:, :, perm], atol=1e-14)
    for i in (3, 4):
        assert np.allclose(p[i], base[i][:, :, perm], atol=1e-14)


def test_projection_head_blocks_map_to_heads():
    """Swapping two heads' column blocks in w (in every group) swaps those heads
    in every output."""
    x, w, H, dk, dv = _rand_proj(5)
    groups = [(0, dk), (H * dk, dk), (2 * H * dk, dv), (2 * H * dk + H * dv, 1),
              (2 * H * dk + H * dv + H, 1)]
    w2 = w.copy()
    for off, d in groups:
        a = slice(off, off + d)
        b = slice(off + 2 * d, off + 3 * d)                          # heads 0 and 2
        w2[:, a], w2[:, b] = w[:, b], w[:, a]
    base = project(x, w, H, dk, dv)
    sw = project(x, w2, H, dk, dv)
    for i in range(5):
        assert np.allclose(sw[i][:, 0], base[i][:, 2], atol=1e-14)
        assert np.allclose(sw[i][:, 2], base[i][:, 0], atol=1e-14)
        assert np.allclose(sw[i][:, 1], base[i][:, 1], atol=1e-14)

