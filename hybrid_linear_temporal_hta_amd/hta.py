"""Thin ctypes binding of libhta (include/hta.h): argument marshalling only.

Each function has the name of the C entry point it calls. Tensors are torch
tensors already on the GPU; only their data pointers, shapes and the current
HIP stream cross the boundary. Every step of the computation runs in libhta's
HIP kernels; there is no fallback: if libhta.so cannot be loaded, the first
call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhta.so")

HTA_OK = 0
HTA_ERR_NULL = -1
HTA_ERR_SHAPE = -2
HTA_ERR_WINDOW = -3
HTA_ERR_DTYPE = -4
HTA_ERR_UNSUPPORTED = -5
HTA_ERR_WORKSPACE = -6
HTA_ERR_RING = -7
HTA_ERR_HIP = -8
HTA_ERR_ALIAS = -9
HTA_ERR_ALIGN = -10
HTA_ERR_SCRATCH = -11
HTA_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024

HTA_F32 = 0
HTA_BF16 = 1

HTA_OP_GLA = 1
HTA_OP_HYBRID = 2
HTA_OP_STREAM_STEP = 3
HTA_OP_ATTN_BWD = 4
HTA_OP_GLA_BWD = 5
HTA_OP_HYBRID_BWD = 6
HTA_OP_SWA_DSWA = 7

HTA_NORM_Q = 1
HTA_NORM_K = 2

HTA_GLA_GATED_DELTA = 0   # S = alpha (S - beta (S k) k^T) + beta v k^T
HTA_GLA_PRINTED = 1       # S = alpha S - beta (S k) k^T + beta v k^T

EXPORTED = (
    "hta_workspace_bytes", "hta_swa_fwd", "hta_dswa_fwd", "hta_swa_fwd_lse", "hta_dswa_fwd_lse",
    "hta_swa_bwd", "hta_dswa_bwd", "hta_swa_dswa_fwd", "hta_swa_dswa_fwd_ex", "hta_gla_fwd",
    "hta_gla_fwd_ex", "hta_gla_bwd", "hta_hybrid_fwd", "hta_hybrid_saved_bytes",
    "hta_hybrid_fwd_train", "hta_hybrid_bwd", "hta_project_fwd",
    "hta_stream_init", "hta_stream_step", "hta_stream_step_noalloc", "hta_status_string", "hta_last_hip_error",
    "hta_version",
)


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("P", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int),
                ("dtype", ctypes.c_int), ("out_dtype", ctypes.c_int)]


class Params(ctypes.Structure):
    _fields_ = [("swa_window", ctypes.c_int), ("dswa_taps", ctypes.c_int),
                ("dswa_dilation", ctypes.c_int), ("gla_chunk", ctypes.c_int),
                ("attn_scale", ctypes.c_float), ("gla_scale", ctypes.c_float),
                ("gla_form", ctypes.c_int), ("side_stream", ctypes.c_void_p),
                ("fork_event", ctypes.c_void_p), ("join_event", ctypes.c_void_p)]


class SideStream:
    """A second stream on the current device and the two events hta_params needs
    to run work on it (held here so that they outlive the calls using them). The
    overlap needs the stream on another hardware queue than the caller's: HIP
    deals streams out over a few queues in turn, and two on one queue run one
    after the other (same results, no overlap)."""

    def __init__(self, device=None):
        self.stream = torch.cuda.Stream(device=device)
        self.fork = torch.cuda.Event()
        self.join = torch.cuda.Event()
        self.fork.record()          # torch creates an event on its first record
        self.join.record()


class StreamCtx(ctypes.Structure):
    _fields_ = [("s", Shape), ("p", Params), ("R", ctypes.c_int),
                ("ring_k", ctypes.c_void_p), ("ring_v", ctypes.c_void_p),
                ("state", ctypes.c_void_p), ("n_frames", ctypes.c_longlong)]


class HTAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().hta_status_string(status).decode()
        if status == HTA_ERR_HIP:
            msg += f" (hipError_t {lib().hta_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhta.so (building it only if no library is present)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    sp, pp = ctypes.POINTER(Shape), ctypes.POINTER(Params)
    L.hta_workspace_bytes.restype = sz
    L.hta_workspace_bytes.argtypes = [i, sp, pp]
    L.hta_swa_fwd.restype = i
    L.hta_swa_fwd.argtypes = [sp, vp, vp, vp, vp, i, f, vp]
    L.hta_dswa_fwd.restype = i
    L.hta_dswa_fwd.argtypes = [sp, vp, vp, vp, vp, i, i, f, vp]
    L.hta_swa_fwd_lse.restype = i
    L.hta_swa_fwd_lse.argtypes = [sp, vp, vp, vp, vp, vp, i, f, vp]
    L.hta_dswa_fwd_lse.restype = i
    L.hta_dswa_fwd_lse.argtypes = [sp, vp, vp, vp, vp, vp, i, i, f, vp]
    L.hta_swa_bwd.restype = i
    L.hta_swa_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, f, vp, sz, vp]
    L.hta_dswa_bwd.restype = i
    L.hta_dswa_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, f, vp, sz, vp]
    L.hta_swa_dswa_fwd_ex.restype = i
    L.hta_swa_dswa_fwd_ex.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hta_swa_dswa_fwd.restype = i
    L.hta_swa_dswa_fwd.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp]
    L.hta_gla_fwd.restype = i
    L.hta_gla_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, i, f, vp, sz, vp]
    L.hta_gla_fwd_ex.restype = i
    L.hta_gla_fwd_ex.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hta_gla_bwd.restype = i
    L.hta_gla_bwd.argtypes = [sp, pp] + [vp] * 14 + [sz, vp]
    L.hta_hybrid_saved_bytes.restype = sz
    L.hta_hybrid_saved_bytes.argtypes = [sp]
    L.hta_hybrid_fwd_train.restype = i
    L.hta_hybrid_fwd_train.argtypes = [sp, pp] + [vp] * 9 + [sz, vp]
    L.hta_hybrid_bwd.restype = i
    L.hta_hybrid_bwd.argtypes = [sp, pp] + [vp] * 14 + [sz, vp]
    L.hta_hybrid_fwd.restype = i
    L.hta_hybrid_fwd.argtypes = [sp, pp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hta_project_fwd.restype = i
    L.hta_project_fwd.argtypes = [sp, i, vp, vp, vp, vp, vp, vp, vp, i, vp]
    L.hta_stream_init.restype = i
    L.hta_stream_init.argtypes = [ctypes.POINTER(StreamCtx), vp, vp, i, vp, vp]
    L.hta_stream_step.restype = i
    L.hta_stream_step.argtypes = [ctypes.POINTER(StreamCtx), vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.hta_stream_step_noalloc.restype = i
    L.hta_stream_step_noalloc.argtypes = [ctypes.POINTER(StreamCtx), vp, vp, vp, vp, vp, vp, vp]
    L.hta_status_string.restype = ctypes.c_char_p
    L.hta_status_string.argtypes = [i]
    L.hta_last_hip_error.restype = i
    L.hta_last_hip_error.argtypes = []
    L.hta_version.restype = ctypes.c_char_p
    L.hta_version.argtypes = []
    _lib = L
    return L


def _check(status: int, where: str):
    if status != HTA_OK:
        raise HTAError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("libhta takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libhta takes contiguous tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HTA_BF16
    if t.dtype == torch.float32:
        return HTA_F32
    return 99   # rejected by the library with HTA_ERR_DTYPE


def make_shape(q: torch.Tensor, v: torch.Tensor, P: int, o: torch.Tensor | None = None) -> Shape:
    """hta_shape of [B, H, L, d] tensors with P tokens per frame (T = L / P);
    out_dtype follows o (fp32 if o is None)."""
    B, H, L, dk = q.shape
    if P < 1 or L % P:
        raise ValueError(f"sequence length {L} is not a whole number of {P}-token frames")
    out = _dtype_code(o) if o is not None else HTA_F32
    return Shape(B, H, L // P, P, dk, v.shape[-1], _dtype_code(q), out)


def make_params(window=3, taps=4, dilation=4, chunk=64, attn_scale=0.0, gla_scale=0.0,
                gla_form=0, side: SideStream | None = None) -> Params:
    """gla_form: HTA_GLA_GATED_DELTA (0) or HTA_GLA_PRINTED (1); side: an optional
    SideStream for the hybrid calls to run their attention work on."""
    p = Params(int(window), int(taps), int(dilation), int(chunk), float(attn_scale),
               float(gla_scale), int(gla_form), None, None, None)
    if side is not None:
        p.side_stream = side.stream.cuda_stream
        p.fork_event = side.fork.cuda_event
        p.join_event = side.join.cuda_event
        p._side = side      # the handles are valid while the SideStream lives
    return p


def hta_workspace_bytes(op: int, shape: Shape, params: Params | None) -> int:
    return int(lib().hta_workspace_bytes(int(op), ctypes.byref(shape),
                                         ctypes.byref(params) if params is not None else None))


def hta_swa_fwd(q, k, v, o, P: int, window_frames: int, scale: float = 0.0, stream=None):
    s = make_shape(q, v, P, o)
    _check(lib().hta_swa_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                             int(window_frames), float(scale), _stream(stream)), "hta_swa_fwd")


def hta_dswa_fwd(q, k, v, o, P: int, taps: int, dilation_frames: int, scale: float = 0.0,
                 stream=None):
    s = make_shape(q, v, P, o)
    _check(lib().hta_dswa_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), int(taps),
                              int(dilation_frames), float(scale), _stream(stream)), "hta_dswa_fwd")


def hta_swa_fwd_lse(q, k, v, o, lse, P: int, window_frames: int, scale: float = 0.0,
                    stream=None):
    s = make_shape(q, v, P, o)
    _check(lib().hta_swa_fwd_lse(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                 int(window_frames), float(scale), _stream(stream)),
           "hta_swa_fwd_lse")


def hta_dswa_fwd_lse(q, k, v, o, lse, P: int, taps: int, dilation_frames: int,
                     scale: float = 0.0, stream=None):
    s = make_shape(q, v, P, o)
    _check(lib().hta_dswa_fwd_lse(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  int(taps), int(dilation_frames), float(scale), _stream(stream)),
           "hta_dswa_fwd_lse")


def _bwd_ws(s: Shape, workspace, device):
    need = hta_workspace_bytes(HTA_OP_ATTN_BWD, s, None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    return workspace


def hta_swa_bwd(q, k, v, o, lse, dout, dq, dk, dv, P: int, window_frames: int,
                scale: float = 0.0, workspace=None, stream=None):
    s = make_shape(q, v, P, o)
    workspace = _bwd_ws(s, workspace, q.device)
    _check(lib().hta_swa_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), int(window_frames),
                             float(scale), _ptr(workspace), workspace.numel(), _stream(stream)),
           "hta_swa_bwd")


def hta_dswa_bwd(q, k, v, o, lse, dout, dq, dk, dv, P: int, taps: int, dilation_frames: int,
                 scale: float = 0.0, workspace=None, stream=None):
    s = make_shape(q, v, P, o)
    workspace = _bwd_ws(s, workspace, q.device)
    _check(lib().hta_dswa_bwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), int(taps),
                              int(dilation_frames), float(scale), _ptr(workspace),
                              workspace.numel(), _stream(stream)), "hta_dswa_bwd")


def hta_swa_dswa_fwd(q, k, v, o, P: int, params: Params, add=None, stream=None):
    s = make_shape(q, v, P, o)
    _check(lib().hta_swa_dswa_fwd(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k),
                                  _ptr(v), _ptr(add), _ptr(o), _stream(stream)),
           "hta_swa_dswa_fwd")


def hta_swa_dswa_fwd_ex(q, k, v, o, P: int, params: Params, add=None, workspace=None,
                        stream=None):
    s = make_shape(q, v, P, o)
    need = hta_workspace_bytes(HTA_OP_SWA_DSWA, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_swa_dswa_fwd_ex(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k),
                                     _ptr(v), _ptr(add), _ptr(o), _ptr(workspace),
                                     workspace.numel(), _stream(stream)), "hta_swa_dswa_fwd_ex")


def hta_gla_fwd(q, k, v, alpha, beta, state, o, P: int, chunk: int = 64, scale: float = 0.0,
                workspace=None, stream=None):
    s = make_shape(q, v, P, o)
    pr = make_params(chunk=chunk)
    need = hta_workspace_bytes(HTA_OP_GLA, s, pr)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_gla_fwd(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                             _ptr(state), _ptr(o), int(chunk), float(scale), _ptr(workspace),
                             workspace.numel(), _stream(stream)), "hta_gla_fwd")


def hta_gla_fwd_ex(q, k, v, alpha, beta, state, o, P: int, params: Params, workspace=None,
                   stream=None):
    s = make_shape(q, v, P, o)
    need = hta_workspace_bytes(HTA_OP_GLA, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_gla_fwd_ex(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "hta_gla_fwd_ex")


def hta_gla_bwd(q, k, v, alpha, beta, state0, dout, dstate, dq, dk, dv, dalpha, dbeta,
                P: int, params: Params, workspace=None, stream=None):
    """Gradients of the GLA branch; dstate is dL/dM_L on entry and dL/dM_0 on exit."""
    s = make_shape(q, v, P, dout)
    need = hta_workspace_bytes(HTA_OP_GLA_BWD, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_gla_bwd(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                             _ptr(alpha), _ptr(beta), _ptr(state0), _ptr(dout), _ptr(dstate),
                             _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(dbeta),
                             _ptr(workspace), workspace.numel(), _stream(stream)), "hta_gla_bwd")


def hta_project_fwd(x, w, q, k, v, alpha, beta, P: int, flags: int = HTA_NORM_Q | HTA_NORM_K,
                    stream=None):
    """x [B, L, Dm] bf16, w [Dm, 3*H*128 + 2*H] bf16 -> q, k, v [B, H, L, 128] bf16 and
    alpha, beta [B, H, L] fp32 (all preallocated)."""
    B, H, L, d = q.shape
    s = Shape(B, H, L // P, P, d, v.shape[3], HTA_BF16, HTA_BF16)
    _check(lib().hta_project_fwd(ctypes.byref(s), int(x.shape[2]), _ptr(x), _ptr(w), _ptr(q),
                                 _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), int(flags),
                                 _stream(stream)), "hta_project_fwd")


def hta_hybrid_fwd(q, k, v, alpha, beta, state, o, P: int, params: Params, workspace=None,
                   stream=None):
    s = make_shape(q, v, P, o)
    need = hta_workspace_bytes(HTA_OP_HYBRID, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_hybrid_fwd(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "hta_hybrid_fwd")


def hta_hybrid_saved_bytes(shape: Shape) -> int:
    return int(lib().hta_hybrid_saved_bytes(ctypes.byref(shape)))


def hta_hybrid_fwd_train(q, k, v, alpha, beta, state, o, saved, P: int, params: Params,
                         workspace=None, stream=None):
    """hta_hybrid_fwd that also fills `saved` (uint8, hta_hybrid_saved_bytes bytes)."""
    s = make_shape(q, v, P, o)
    need = hta_workspace_bytes(HTA_OP_HYBRID, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_hybrid_fwd_train(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(o),
                                      _ptr(saved), _ptr(workspace), workspace.numel(),
                                      _stream(stream)), "hta_hybrid_fwd_train")


def hta_hybrid_bwd(q, k, v, alpha, beta, saved, dout, dstate, dq, dk, dv, dalpha, dbeta,
                   P: int, params: Params, workspace=None, stream=None):
    """Gradients of the hybrid layer; dstate is dL/dM_L on entry and dL/dM_0 on exit."""
    s = make_shape(q, v, P, dout)
    need = hta_workspace_bytes(HTA_OP_HYBRID_BWD, s, params)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib().hta_hybrid_bwd(ctypes.byref(s), ctypes.byref(params), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(alpha), _ptr(beta), _ptr(saved), _ptr(dout), _ptr(dstate),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dalpha), _ptr(dbeta),
                                _ptr(workspace), workspace.numel(), _stream(stream)),
           "hta_hybrid_bwd")


class Stream:
    """Caller-owned streaming context (ring K/V of R frames + GLA state)."""

    def __init__(self, B, H, P, d, dtype, params: Params, R: int, device="cuda",
                 out_dtype=torch.float32):
        self.ring_k = torch.zeros(B, H, R, P, d, dtype=dtype, device=device)
        self.ring_v = torch.zeros(B, H, R, P, d, dtype=dtype, device=device)
        self.state = torch.zeros(B, H, d, d, dtype=torch.float32, device=device)
        code = HTA_BF16 if dtype == torch.bfloat16 else (HTA_F32 if dtype == torch.float32 else 99)
        ocode = HTA_BF16 if out_dtype == torch.bfloat16 else (HTA_F32 if out_dtype == torch.float32 else 99)
        self.out_dtype = out_dtype
        self.params = params        # holds the side stream's handles alive, if any
        self.ctx = StreamCtx(Shape(B, H, 1, P, d, d, code, ocode), params, int(R),
                             self.ring_k.data_ptr(), self.ring_v.data_ptr(),
                             self.state.data_ptr(), 0)
        need = hta_workspace_bytes(HTA_OP_STREAM_STEP, self.ctx.s, params)
        self.workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)

    @property
    def n_frames(self) -> int:
        return int(self.ctx.n_frames)


def hta_stream_init(st: Stream, k_prefix, v_prefix, T_prefix: int, state_prefix=None, stream=None):
    _check(lib().hta_stream_init(ctypes.byref(st.ctx), _ptr(k_prefix), _ptr(v_prefix),
                                 int(T_prefix), _ptr(state_prefix), _stream(stream)),
           "hta_stream_init")


def hta_stream_step(st: Stream, q, k, v, alpha, beta, o=None, stream=None):
    _check(lib().hta_stream_step(ctypes.byref(st.ctx), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                 _ptr(beta), _ptr(o), _ptr(st.workspace), st.workspace.numel(),
                                 _stream(stream)), "hta_stream_step")


def hta_stream_step_noalloc(st: Stream, q, k, v, alpha, beta, o=None, stream=None):
    """hta_stream_step on the library's fixed per-GPU scratch (no workspace)."""
    _check(lib().hta_stream_step_noalloc(ctypes.byref(st.ctx), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(alpha), _ptr(beta), _ptr(o), _stream(stream)),
           "hta_stream_step_noalloc")
