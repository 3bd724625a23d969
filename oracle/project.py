"""Input side of the GLA branch: per-token projections and gates (fp64, numpy).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; it shares nothing with the HIP
library.

Source: [P1] "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io
paper-reads), section 二、方法, second pillar, GLA paragraph: every token
feature x_t is projected to q_t = W_Q x_t, k_t = W_K x_t, v_t = W_V x_t and a
write strength beta_t = sigmoid(W_beta x_t); the forget gate alpha_t lies in
(0, 1) and is computed from the input. Readings taken here:
  - alpha_t = sigmoid(W_alpha x_t), the plainest map from the input into (0, 1);
  - q and k are L2-normalised per token and head when asked (the workloads
    normalise them; a zero vector stays zero);
  - one weight matrix holds every head's projections side by side.

Layouts: x [B, L, Dm]; w [Dm, N] with N = H*dk + H*dk + H*dv + H + H, the
columns ordered q (head 0, head 1, ...), k, v, alpha, beta. Outputs in the
layout of every other entry point: q, k [B, H, L, dk], v [B, H, L, dv], alpha,
beta [B, H, L].
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)


def _heads(y, B, L, H, d):
    """[B, L, H*d] (head-major columns) -> [B, H, L, d]."""
    return np.ascontiguousarray(y.reshape(B, L, H, d).transpose(0, 2, 1, 3))


def _unit(a):
    n = np.sqrt(np.sum(a * a, axis=-1, keepdims=True))
    return np.where(n > 0, a / np.where(n > 0, n, 1.0), 0.0)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def project(x, w, H: int, dk: int, dv: int, norm_q: bool = True, norm_k: bool = True):
    """Returns (q, k, v, alpha, beta) for token features x and weights w."""
    x, w = _f64(x), _f64(w)
    B, L, Dm = x.shape
    N = 2 * H * dk + H * dv + 2 * H
    if w.shape != (Dm, N):
        raise ValueError(f"w must be [{Dm}, {N}]")
    y = x @ w                                   # [B, L, N]: one product per token
    o = 0
    q = _heads(y[..., o:o + H * dk], B, L, H, dk); o += H * dk
    k = _heads(y[..., o:o + H * dk], B, L, H, dk); o += H * dk
    v = _heads(y[..., o:o + H * dv], B, L, H, dv); o += H * dv
    za = y[..., o:o + H]; o += H
    zb = y[..., o:o + H]
    alpha = np.ascontiguousarray(_sigmoid(za).transpose(0, 2, 1))
    beta = np.ascontiguousarray(_sigmoid(zb).transpose(0, 2, 1))
    if norm_q:
        q = _unit(q)
    if norm_k:
        k = _unit(k)
    return q, k, v, alpha, beta
