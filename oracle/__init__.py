"""fp64 CPU oracle for Hybrid Linear Temporal Attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
and its Python binding never import it, and it imports nothing from them.

The arithmetic lives in ``oracle.c`` (plain loops, fp64, OpenMP over rows or
heads) and in ``gla_chunked.py`` (the chunked closed form of the GLA
recurrence, used only as a second route to pin the first). This module only
builds/loads the C library, marshals numpy arrays, and composes the branch
outputs into the hybrid and streaming results the pages describe.

Sources: [P1] "Kairos：面向物理 AI 的原生世界模型栈" (yingwang.github.io
paper-reads), section 二、方法 (Method), second pillar: SWA, DSWA and GLA
paragraphs, the GLA update equations and the three-branch figure.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

_dp = ctypes.POINTER(ctypes.c_double)
_llp = ctypes.POINTER(ctypes.c_longlong)


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i, ll, d = ctypes.c_int, ctypes.c_longlong, ctypes.c_double
        for name in ("oracle_swa_rows", "oracle_dswa_rows"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp, i, i, d, ll, _llp, _dp] \
                if name == "oracle_dswa_rows" else \
                [i, i, i, i, i, i, _dp, _dp, _dp, i, d, ll, _llp, _dp]
        lib.oracle_swa.restype = i
        lib.oracle_swa.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp, i, d, _dp]
        lib.oracle_dswa.restype = i
        lib.oracle_dswa.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp, i, i, d, _dp]
        for name in ("oracle_gla", "oracle_gla_literal"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = [i, i, ll, i, i, _dp, _dp, _dp, _dp, _dp, d, _dp, _dp]
        for name in ("oracle_swa_bwd", "oracle_dswa_bwd"):
            fn = getattr(lib, name)
            fn.restype = i
            fn.argtypes = [i, i, i, i, i, i, _dp, _dp, _dp, _dp] + \
                ([i, i] if name == "oracle_dswa_bwd" else [i]) + [d, _dp, _dp, _dp]
        lib.oracle_window_stats.restype = i
        lib.oracle_window_stats.argtypes = [i, i, i, i, i, i, i, _dp, _dp, _dp, _dp, i, i, d,
                                            ll, _llp, _dp, _dp]
        lib.oracle_window_dq_rows.restype = i
        lib.oracle_window_dq_rows.argtypes = [i, i, i, i, i, i, i, _dp, _dp, _dp, _dp, i, i, d,
                                              ll, _llp, _dp]
        lib.oracle_window_dkv_rows.restype = i
        lib.oracle_window_dkv_rows.argtypes = [i, i, i, i, i, i, i, _dp, _dp, _dp, _dp, _dp, _dp,
                                               i, i, d, ll, _llp, _dp, _dp]
        lib.oracle_gla_bwd.restype = i
        lib.oracle_gla_bwd.argtypes = [i, i, i, ll, i, i, _dp, _dp, _dp, _dp, _dp, d, _dp, _dp,
                                       _dp, _dp, _dp, _dp, _dp, _dp, _dp]
        lib.oracle_num_threads.restype = i
        lib.oracle_num_threads.argtypes = []
        _lib = lib
        return lib


def _f64(x) -> np.ndarray:
    """Contiguous float64 copy/view of a numpy array or a CPU torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _check(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def _dims(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, L, d]")
    B, H, L, dk = q.shape
    if k.shape != (B, H, L, dk) or v.shape[:3] != (B, H, L):
        raise ValueError("q, k, v shapes disagree")
    return B, H, L, dk, v.shape[3]


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().oracle_num_threads())


def default_scale(dk: int) -> float:
    """Softmax scale 1/sqrt(dk) of standard scaled dot-product attention."""
    return 1.0 / float(np.sqrt(dk))


def swa(q, k, v, T: int, P: int, window: int, scale: float | None = None) -> np.ndarray:
    """SWA over all tokens: query in frame f attends to frames f-window+1..f."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk, dv = _dims(q, k, v)
    if L != T * P:
        raise ValueError("L must equal T*P")
    o = np.empty((B, H, L, dv), np.float64)
    s = default_scale(dk) if not scale else float(scale)
    _check(_load().oracle_swa(B, H, T, P, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                              int(window), s, _ptr(o)), "oracle_swa")
    return o


def dswa(q, k, v, T: int, P: int, taps: int, dilation: int,
         scale: float | None = None) -> np.ndarray:
    """DSWA over all tokens: query in frame f attends to frames f - j*dilation."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk, dv = _dims(q, k, v)
    if L != T * P:
        raise ValueError("L must equal T*P")
    o = np.empty((B, H, L, dv), np.float64)
    s = default_scale(dk) if not scale else float(scale)
    _check(_load().oracle_dswa(B, H, T, P, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                               int(taps), int(dilation), s, _ptr(o)), "oracle_dswa")
    return o


def _rows_call(fn_name, q, k, v, T, P, rows, scale, qrows, *args):
    k, v = _f64(k), _f64(v)
    if k.ndim != 4 or v.ndim != 4 or k.shape[:3] != v.shape[:3]:
        raise ValueError("k, v must be [B, H, L, d]")
    B, H, L, dk = k.shape
    dv = v.shape[3]
    if L != T * P:
        raise ValueError("L must equal T*P")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if qrows is None:
        qrows = _f64(q).reshape(-1, dk)[rows]
    qrows = np.ascontiguousarray(np.asarray(qrows, dtype=np.float64).reshape(rows.size, dk))
    o = np.empty((rows.size, dv), np.float64)
    s = default_scale(dk) if not scale else float(scale)
    fn = getattr(_load(), fn_name)
    _check(fn(B, H, T, P, dk, dv, _ptr(qrows), _ptr(k), _ptr(v), *args, s, rows.size,
              rows.ctypes.data_as(_llp), _ptr(o)), fn_name)
    return o


def swa_rows(q, k, v, T: int, P: int, window: int, rows,
             scale: float | None = None, qrows=None) -> np.ndarray:
    """SWA for the listed flat query rows (bh*L + t); returns [n_rows, dv].
    The query vectors are q's rows, or ``qrows`` ([n_rows, dk]) when q is None."""
    return _rows_call("oracle_swa_rows", q, k, v, T, P, rows, scale, qrows, int(window))


def dswa_rows(q, k, v, T: int, P: int, taps: int, dilation: int, rows,
              scale: float | None = None, qrows=None) -> np.ndarray:
    """DSWA for the listed flat query rows (bh*L + t); returns [n_rows, dv]."""
    return _rows_call("oracle_dswa_rows", q, k, v, T, P, rows, scale, qrows, int(taps),
                      int(dilation))


def _gla(fn_name, q, k, v, alpha, beta, state0, scale):
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, L, dk, dv = _dims(q, k, v)
    alpha, beta = _f64(alpha), _f64(beta)
    if alpha.shape != (B, H, L) or beta.shape != (B, H, L):
        raise ValueError("alpha, beta must be [B, H, L]")
    state = np.zeros((B, H, dk, dv), np.float64) if state0 is None else _f64(state0).copy()
    if state.shape != (B, H, dk, dv):
        raise ValueError("state must be [B, H, dk, dv]")
    o = np.empty((B, H, L, dv), np.float64)
    fn = getattr(_load(), fn_name)
    _check(fn(B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
              float(scale), _ptr(state), _ptr(o)), fn_name)
    return o, state


def gla(q, k, v, alpha, beta, state0=None, scale: float = 1.0):
    """Token-by-token gated delta recurrence (GatedDeltaNet reading).

    Returns (o [B,H,L,dv], final state [B,H,dk,dv] = S_L^T).
    """
    return _gla("oracle_gla", q, k, v, alpha, beta, state0, scale)


def gla_literal(q, k, v, alpha, beta, state0=None, scale: float = 1.0):
    """The three GLA update lines exactly as printed on the page (v_old, v_new, S)."""
    return _gla("oracle_gla_literal", q, k, v, alpha, beta, state0, scale)


def hybrid(q, k, v, alpha, beta, T: int, P: int, window: int, taps: int,
           dilation: int, state0=None, attn_scale: float | None = None,
           gla_scale: float = 1.0):
    """Hybrid output = SWA + DSWA + GLA (the three-branch figure, summed).

    Returns (o, final GLA state, (o_swa, o_dswa, o_gla)).
    """
    o_s = swa(q, k, v, T, P, window, attn_scale)
    o_d = dswa(q, k, v, T, P, taps, dilation, attn_scale)
    o_g, st = gla(q, k, v, alpha, beta, state0, gla_scale)
    return o_s + o_d + o_g, st, (o_s, o_d, o_g)


def stream_frame(k_hist, v_hist, q_new, P: int, window: int, taps: int, dilation: int,
                 attn_scale: float | None = None, rows=None):
    """Attention part of one streaming step, from the WHOLE K/V history.

    k_hist, v_hist: [B, H, (n+1)*P, d] holding every frame up to and including
    the new frame n; q_new: [B, H, P, dk]. No ring buffer: the window is taken
    from the full history, exactly as the batch definition would.
    Returns (o_swa + o_dswa) for the new frame, [B, H, P, dv] (or only the
    listed in-frame positions when rows is given: [B, H, len(rows), dv]).
    """
    k_hist, v_hist, q_new = _f64(k_hist), _f64(v_hist), _f64(q_new)
    B, H, Lh, dk = k_hist.shape
    dv = v_hist.shape[3]
    T = Lh // P
    if T * P != Lh or q_new.shape != (B, H, P, dk):
        raise ValueError("history must hold whole frames and q_new one frame")
    pos = np.arange(P) if rows is None else np.asarray(rows, dtype=np.int64)
    flat = (np.arange(B * H)[:, None] * Lh + (T - 1) * P + pos[None, :]).reshape(-1)
    qr = q_new[:, :, pos, :].reshape(-1, dk)
    o = swa_rows(None, k_hist, v_hist, T, P, window, flat, attn_scale, qrows=qr) + \
        dswa_rows(None, k_hist, v_hist, T, P, taps, dilation, flat, attn_scale, qrows=qr)
    return o.reshape(B, H, pos.size, dv)


# ---------------------------------------------------------------------------
# Backward pass: exact gradients of the definitions above (chain rule written
# out in oracle.c; pinned by finite differences in the tests).
# ---------------------------------------------------------------------------

_KIND = {"swa": 0, "dswa": 1}


def _window_args(kind: str, window_or_taps: int, dilation: int):
    if kind not in _KIND:
        raise ValueError("kind must be 'swa' or 'dswa'")
    return _KIND[kind], int(window_or_taps), int(dilation if kind == "dswa" else 0)


def swa_bwd(q, k, v, dout, T: int, P: int, window: int, scale: float | None = None):
    """Gradients (dq, dk, dv) of SWA for output gradient dout."""
    return _window_bwd("swa", q, k, v, dout, T, P, window, 0, scale)


def dswa_bwd(q, k, v, dout, T: int, P: int, taps: int, dilation: int,
             scale: float | None = None):
    """Gradients (dq, dk, dv) of DSWA for output gradient dout."""
    return _window_bwd("dswa", q, k, v, dout, T, P, taps, dilation, scale)


def _window_bwd(kind, q, k, v, dout, T, P, a, b, scale):
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, dk, dv = _dims(q, k, v)
    if L != T * P or dout.shape != v.shape:
        raise ValueError("L must equal T*P and dout match v")
    s = default_scale(dk) if not scale else float(scale)
    dq, dkk, dvv = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    lib = _load()
    if kind == "swa":
        st = lib.oracle_swa_bwd(B, H, T, P, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                int(a), s, _ptr(dq), _ptr(dkk), _ptr(dvv))
    else:
        st = lib.oracle_dswa_bwd(B, H, T, P, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                 int(a), int(b), s, _ptr(dq), _ptr(dkk), _ptr(dvv))
    _check(st, f"oracle_{kind}_bwd")
    return dq, dkk, dvv


def window_stats(kind: str, q, k, v, dout, T: int, P: int, window_or_taps: int,
                 dilation: int, rows, scale: float | None = None):
    """Per-row softmax statistics for the listed flat query rows (bh*L + t):
    (lse, D) with lse the log-sum-exp of the scaled logits over the row's
    window and D = dout_t . o_t."""
    kd, a, b = _window_args(kind, window_or_taps, dilation)
    k, v = _f64(k), _f64(v)
    B, H, L, dk = k.shape
    dv = v.shape[3]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    qr = np.ascontiguousarray(_f64(q).reshape(-1, dk)[rows])
    dr = np.ascontiguousarray(_f64(dout).reshape(-1, dv)[rows])
    lse, D = np.empty(rows.size), np.empty(rows.size)
    s = default_scale(dk) if not scale else float(scale)
    _check(_load().oracle_window_stats(kd, B, H, T, P, dk, dv, _ptr(qr), _ptr(dr), _ptr(k),
                                       _ptr(v), a, b, s, rows.size, rows.ctypes.data_as(_llp),
                                       _ptr(lse), _ptr(D)), "oracle_window_stats")
    return lse, D


def window_dq_rows(kind: str, q, k, v, dout, T: int, P: int, window_or_taps: int,
                   dilation: int, rows, scale: float | None = None):
    """dq of SWA/DSWA for the listed flat query rows; returns [n, dk]."""
    kd, a, b = _window_args(kind, window_or_taps, dilation)
    k, v = _f64(k), _f64(v)
    B, H, L, dk = k.shape
    dv = v.shape[3]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    qr = np.ascontiguousarray(_f64(q).reshape(-1, dk)[rows])
    dr = np.ascontiguousarray(_f64(dout).reshape(-1, dv)[rows])
    out = np.empty((rows.size, dk))
    s = default_scale(dk) if not scale else float(scale)
    _check(_load().oracle_window_dq_rows(kd, B, H, T, P, dk, dv, _ptr(qr), _ptr(dr), _ptr(k),
                                         _ptr(v), a, b, s, rows.size,
                                         rows.ctypes.data_as(_llp), _ptr(out)),
           "oracle_window_dq_rows")
    return out


def window_dkv_rows(kind: str, q, k, v, dout, T: int, P: int, window_or_taps: int,
                    dilation: int, rows, scale: float | None = None):
    """dk, dv of SWA/DSWA for the listed flat key rows ([n, dk], [n, dv]).

    The statistics are computed only for the queries that attend to those
    rows (query frames f_k + j * step of each key frame f_k)."""
    kd, a, b = _window_args(kind, window_or_taps, dilation)
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, dk, dv = _dims(q, k, v)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    step = 1 if kind == "swa" else b
    need = set()
    for r in rows.tolist():
        bh, kf = divmod(r, L)[0], (r % L) // P
        for j in range(a):
            fq = kf + j * step
            if fq >= T:
                break
            need.add((bh, fq))
    qrows = np.array(sorted(bh * L + fq * P + p for bh, fq in need for p in range(P)),
                     dtype=np.int64)
    lse_full, D_full = np.zeros(B * H * L), np.zeros(B * H * L)
    if qrows.size:
        lse, D = window_stats(kind, q, k, v, dout, T, P, a, b, qrows, scale)
        lse_full[qrows], D_full[qrows] = lse, D
    dko, dvo = np.empty((rows.size, dk)), np.empty((rows.size, dv))
    s = default_scale(dk) if not scale else float(scale)
    _check(_load().oracle_window_dkv_rows(kd, B, H, T, P, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                          _ptr(dout), _ptr(lse_full), _ptr(D_full), a, b, s,
                                          rows.size, rows.ctypes.data_as(_llp), _ptr(dko),
                                          _ptr(dvo)), "oracle_window_dkv_rows")
    return dko, dvo


def gla_bwd(q, k, v, alpha, beta, dout, state0=None, dstate_final=None,
            scale: float = 1.0, form: int = 0):
    """Gradients of the GLA recurrence (form 0: GatedDeltaNet reading, 1: the
    printed update) for output gradient dout and, optionally, a gradient of the
    final state (dL/dM_L, [B,H,dk,dv]).

    Returns dict(dq, dk, dv, dalpha, dbeta, dstate0) with dstate0 = dL/dM_0.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, H, L, dk, dv = _dims(q, k, v)
    alpha, beta = _f64(alpha), _f64(beta)
    if alpha.shape != (B, H, L) or beta.shape != (B, H, L) or dout.shape != v.shape:
        raise ValueError("alpha, beta must be [B, H, L] and dout match v")
    s0 = np.zeros((B, H, dk, dv)) if state0 is None else _f64(state0)
    dsf = None if dstate_final is None else _f64(dstate_final)
    if s0.shape != (B, H, dk, dv) or (dsf is not None and dsf.shape != s0.shape):
        raise ValueError("states must be [B, H, dk, dv]")
    out = dict(dq=np.empty_like(q), dk=np.empty_like(k), dv=np.empty_like(v),
               dalpha=np.empty_like(alpha), dbeta=np.empty_like(beta),
               dstate0=np.empty_like(s0))
    _check(_load().oracle_gla_bwd(int(form), B, H, L, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(alpha), _ptr(beta), float(scale), _ptr(s0), _ptr(dout),
                                  _ptr(dsf) if dsf is not None else None,
                                  _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                  _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(out["dstate0"])),
           "oracle_gla_bwd")
    return out


def hybrid_bwd(q, k, v, alpha, beta, dout, T: int, P: int, window: int, taps: int,
               dilation: int, state0=None, dstate_final=None, attn_scale: float | None = None,
               gla_scale: float = 1.0, form: int = 0):
    """Gradients of the hybrid sum: each branch's gradient for the shared
    output gradient, summed over branches for q, k, v."""
    s = swa_bwd(q, k, v, dout, T, P, window, attn_scale)
    d = dswa_bwd(q, k, v, dout, T, P, taps, dilation, attn_scale)
    g = gla_bwd(q, k, v, alpha, beta, dout, state0, dstate_final, gla_scale, form)
    return dict(dq=s[0] + d[0] + g["dq"], dk=s[1] + d[1] + g["dk"], dv=s[2] + d[2] + g["dv"],
                dalpha=g["dalpha"], dbeta=g["dbeta"], dstate0=g["dstate0"])
