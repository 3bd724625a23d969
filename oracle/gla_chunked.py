"""Chunked closed form of the GLA gated delta recurrence (fp64, numpy).

TEST INFRASTRUCTURE: a second, independent route to the GLA result, used only
to pin the token-by-token oracle (and to be pinned by it). It is the algebra
the chunked GPU kernels are built on, written plainly.

Source: [P1] "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io
paper-reads), section 二、方法, GLA update equations, GatedDeltaNet reading:
    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,  o_t = S_t q_t.

Derivation (state kept as M = S^T, dk x dv). Within a chunk of C tokens that
starts from M0, let g_t = sum_{r<=t} log alpha_r (inclusive, chunk-local) and
write the update as S_t = alpha_t S_{t-1} + u_t k_t^T with
u_t = beta_t (v_t - alpha_t S_{t-1} k_t). Unrolling S_{t-1} inside the chunk:
    u_t + beta_t sum_{s<t} e^{g_t - g_s} (k_t . k_s) u_s = beta_t (v_t - e^{g_t} M0^T k_t)
i.e. (I + A) U = diag(beta) (V - diag(e^g) K M0),  A = strictly-lower part of
diag(beta) (K K^T o Gamma), Gamma_ts = e^{g_t - g_s}. Then
    O   = diag(e^g) Q M0 + tril(Q K^T o Gamma) U          (o_t = S_t q_t)
    M_C = e^{g_C} M0 + K^T diag(e^{g_C - g}) U.
``literal=True`` applies the page's printed form instead (forget gate not on
the erase term): u_t = beta_t (v_t - S_{t-1} k_t), which shifts g_t to g_{t-1}
in A and in the M0 term.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def gla_chunked(q, k, v, alpha, beta, chunk: int, state0=None, scale: float = 1.0,
                literal: bool = False):
    """Returns (o [B,H,L,dv], final state [B,H,dk,dv]) by the chunked closed form."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    alpha, beta = np.asarray(alpha, np.float64), np.asarray(beta, np.float64)
    B, H, L, dk = q.shape
    dv = v.shape[3]
    o = np.zeros((B, H, L, dv))
    out_state = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = np.zeros((dk, dv)) if state0 is None else np.array(state0[b, h], np.float64)
            for c0 in range(0, L, chunk):
                sl = slice(c0, min(c0 + chunk, L))
                Q, K, V = q[b, h, sl], k[b, h, sl], v[b, h, sl]
                a, be = alpha[b, h, sl], beta[b, h, sl]
                g = np.cumsum(np.log(a))                    # inclusive
                g_prev = np.concatenate([[0.0], g[:-1]])    # exclusive
                gr = g_prev if literal else g               # decay seen by the erase term
                Gam = np.exp(g[:, None] - g[None, :])
                Gam_r = np.exp(gr[:, None] - g[None, :])
                n = K.shape[0]
                A = np.tril(be[:, None] * (K @ K.T) * Gam_r, -1)
                rhs = be[:, None] * (V - np.exp(gr)[:, None] * (K @ M))
                U = solve_triangular(np.eye(n) + A, rhs, lower=True, unit_diagonal=True)
                Pm = np.tril((Q @ K.T) * Gam)
                o[b, h, sl] = scale * (np.exp(g)[:, None] * (Q @ M) + Pm @ U)
                M = np.exp(g[-1]) * M + K.T @ (np.exp(g[-1] - g)[:, None] * U)
            out_state[b, h] = M
    return o, out_state
